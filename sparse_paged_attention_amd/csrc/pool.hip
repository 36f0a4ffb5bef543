// Physical-page pool writes and min/max page summaries.
//
// LServe write-up (bqwf.cn), "2.2 分层分页KV缓存": tokens live in logical
// pages (the selection unit) packed inside physical pages (the allocation
// unit); a page table maps a sequence's positions to physical pages.
// "2.1 混合稀疏注意力机制": each block (logical page) is summarised by
// min-max pooling of its keys.
//
// In-page layout: keys token-major [P][D] per (physical page, head); values
// channel-major [D][p] per logical page, so the attention kernel can feed
// both straight into matrix-core operands.
#include "pool_rows.h"

namespace spa {
namespace {

// One wave per (sequence, KV head): writes token L-1; for dynamic heads (when
// summaries are kept) the same wave rebuilds the summary of the logical page
// receiving the token.
__global__ void __launch_bounds__(64) append_kernel(PoolArgs pl, BatchArgs bt,
                                                    const uint32_t* __restrict__ k_new,
                                                    const uint16_t* __restrict__ v_new,
                                                    HeadList dyn, int32_t with_summary) {
  const int32_t b = blockIdx.x / pl.hkv, h = blockIdx.x % pl.hkv;
  bool is_dyn = false;
  for (int32_t d = 0; d < dyn.n; ++d) is_dyn |= dyn.id[d] == h;
  const int32_t hsl = head_slot(pl, h, dyn_rank(dyn, h), is_dyn);
  if (pl.q8)
    append_token_q8(pl, bt, b, h, hsl, k_new, reinterpret_cast<const uint32_t*>(v_new), with_summary && is_dyn,
                    bt.ring != nullptr && !is_dyn);
  else
    append_token(pl, bt, b, h, hsl, k_new, v_new, with_summary && is_dyn, bt.ring != nullptr && !is_dyn);
}

// Bulk write of tokens [start, start + count) of one sequence (prefill), one
// wave per (logical page, KV head). Lane l owns channels 2l and 2l + 1 of each
// of the page's PG tokens, so every load instruction reads one whole 256-byte
// row of the caller's [H_kv][count][D] arrays. Keys are stored row by row;
// values channel-major, each channel's PG tokens as one contiguous run built
// in registers. For dynamic heads (bit h of `dyn`) the lane's minimum and
// maximum over the page are its part of the page summary, written in the same
// pass: the summary covers the page's tokens below start + count, those
// before `start` (a page only partly inside the range) read from the pool.
// With a ring (ring_base >= 0), streaming heads keep only what a later step
// can attend: the sink's pages and the last ring_win pages of the range, at
// their ring slots.
struct DynMask {
  uint32_t w[kMaxKvHeads / 32];
};

template <int PG>
__global__ void __launch_bounds__(64) write_kernel(PoolArgs pl, const int32_t* __restrict__ pt, int64_t start,
                                                   int64_t count, const uint32_t* __restrict__ k,
                                                   const uint32_t* __restrict__ v, DynMask dyn,
                                                   int32_t ring_base, int32_t ring_sink, int32_t ring_win) {
  const int32_t h = blockIdx.y;
  const int64_t j = start / PG + blockIdx.x;       // logical page
  const int64_t t0 = j * PG, end = start + count;
  const int64_t lo = t0 > start ? t0 : start, hi = t0 + PG < end ? t0 + PG : end;
  if (lo >= hi) return;
  const bool dynamic = (dyn.w[h >> 5] >> (h & 31)) & 1u;
  int32_t phys;
  if (ring_base >= 0 && !dynamic) {
    const int64_t pg = j / pl.r, last = (end - 1) / pl.P;
    if (pg >= ring_sink && pg < last - (ring_win - 1)) return;   // overwritten later in this range
    phys = ring_base + (int32_t)(pg < ring_sink ? pg : ring_sink + (pg - ring_sink) % ring_win);
  } else {
    phys = pt[j / pl.r];
  }
  if (phys < 0 || phys >= pl.N) return;
  const int32_t lp = (int32_t)(j % pl.r);
  int32_t below = 0;
#pragma unroll
  for (int w = 0; w < kMaxKvHeads / 32; ++w) below += __popc(dyn.w[w] & (32 * w + 32 <= h ? ~0u : 32 * w >= h ? 0u : (1u << (h - 32 * w)) - 1u));
  const int32_t hsl = head_slot(pl, h, below, dynamic);
  const int lane = threadIdx.x;
  uint32_t kw[PG], vw[PG];
#pragma unroll
  for (int u = 0; u < PG; ++u) {                   // rows outside the range re-read row lo
    const int64_t t = t0 + u;
    const int64_t row = (int64_t)h * count + ((t >= lo && t < hi) ? t : lo) - start;
    kw[u] = k[row * 64 + lane];
    vw[u] = v[row * 64 + lane];
  }
  uint32_t* kd = reinterpret_cast<uint32_t*>(pl.k + k_row(pl, phys, hsl, lp * PG) * kHeadDim) + lane;
  uint16_t* vd = pl.v + v_page(pl, phys, hsl, lp);   // [D][PG]
  if (lo == t0 && hi == t0 + PG) {
#pragma unroll
    for (int u = 0; u < PG; ++u) kd[u * 64] = kw[u];
    uint32_t a[PG / 2], c[PG / 2];                   // channel 2l / 2l + 1, tokens 2i and 2i + 1
#pragma unroll
    for (int i = 0; i < PG / 2; ++i) {
      a[i] = (vw[2 * i] & 0xFFFFu) | (vw[2 * i + 1] << 16);
      c[i] = (vw[2 * i] >> 16) | (vw[2 * i + 1] & 0xFFFF0000u);
    }
    uint4* d0 = reinterpret_cast<uint4*>(vd + (2 * lane) * PG);
    uint4* d1 = reinterpret_cast<uint4*>(vd + (2 * lane + 1) * PG);
#pragma unroll
    for (int i = 0; i < PG / 8; ++i) {
      d0[i] = uint4{a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]};
      d1[i] = uint4{c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]};
    }
  } else {
#pragma unroll
    for (int u = 0; u < PG; ++u) {
      const int64_t t = t0 + u;
      if (t >= lo && t < hi) {
        kd[u * 64] = kw[u];
        vd[(2 * lane) * PG + u] = (uint16_t)vw[u];
        vd[(2 * lane + 1) * PG + u] = (uint16_t)(vw[u] >> 16);
      }
    }
  }
  if (!dynamic) return;
  uint32_t lo0 = 0xFFFFFFFFu, hi0 = 0u, lo1 = 0xFFFFFFFFu, hi1 = 0u;
#pragma unroll
  for (int u = 0; u < PG; ++u) {
    const int64_t t = t0 + u;
    if (t < hi) {                                   // tokens before `start` are already in the pool
      const uint32_t w = t >= lo ? kw[u] : kd[u * 64];
      const uint32_t x = order_key((uint16_t)w), y = order_key((uint16_t)(w >> 16));
      lo0 = min(lo0, x); hi0 = max(hi0, x);
      lo1 = min(lo1, y); hi1 = max(hi1, y);
    }
  }
  uint32_t* sp = reinterpret_cast<uint32_t*>(pl.summ + summ_page(pl, phys, hsl, lp));
  sp[lane] = (uint32_t)from_key(lo0) | ((uint32_t)from_key(lo1) << 16);
  sp[kHeadDim / 2 + lane] = (uint32_t)from_key(hi0) | ((uint32_t)from_key(hi1) << 16);
}

// write_kernel for fp8 pages: each token's key and value rows are quantized
// and codes and scales are written; the summary of a dynamic head's page is
// the min / max of the dequantized keys (tokens before `start` read back
// from the pool), rounded outward to bf16. Per chunk of 16 tokens, the 32
// key and value row maxima are reduced across the wave together, two rows
// per word, by a reduce-scatter that leaves each lane with two of them; the
// lanes compute those rows' scales and reciprocal brackets in parallel and
// store the scales, and each row's bracket is read from its lane into scalar
// registers for coding the row (codes_bracketed).
template <int PG>
__global__ void __launch_bounds__(64) write_kernel_q8(PoolArgs pl, const int32_t* __restrict__ pt, int64_t start,
                                                      int64_t count, const uint32_t* __restrict__ k,
                                                      const uint32_t* __restrict__ v, DynMask dyn,
                                                      int32_t ring_base, int32_t ring_sink, int32_t ring_win) {
  const int32_t h = blockIdx.y;
  const int64_t j = start / PG + blockIdx.x;       // logical page
  const int64_t t0 = j * PG, end = start + count;
  const int64_t lo = t0 > start ? t0 : start, hi = t0 + PG < end ? t0 + PG : end;
  if (lo >= hi) return;
  const bool dynamic = (dyn.w[h >> 5] >> (h & 31)) & 1u;
  int32_t phys;
  if (ring_base >= 0 && !dynamic) {
    const int64_t pg = j / pl.r, last = (end - 1) / pl.P;
    if (pg >= ring_sink && pg < last - (ring_win - 1)) return;   // overwritten later in this range
    phys = ring_base + (int32_t)(pg < ring_sink ? pg : ring_sink + (pg - ring_sink) % ring_win);
  } else {
    phys = pt[j / pl.r];
  }
  if (phys < 0 || phys >= pl.N) return;
  const int32_t lp = (int32_t)(j % pl.r);
  int32_t below = 0;
#pragma unroll
  for (int w = 0; w < kMaxKvHeads / 32; ++w) below += __popc(dyn.w[w] & (32 * w + 32 <= h ? ~0u : 32 * w >= h ? 0u : (1u << (h - 32 * w)) - 1u));
  const int32_t hsl = head_slot(pl, h, below, dynamic);
  const int lane = threadIdx.x;
  const int64_t row0 = k_row(pl, phys, hsl, lp * PG);
  uint8_t* kd = reinterpret_cast<uint8_t*>(pl.k) + row0 * kHeadDim;                 // [PG][D] codes
  uint8_t* vd = reinterpret_cast<uint8_t*>(pl.v) + v_page(pl, phys, hsl, lp);        // [D][PG] codes
  MinMax2 mm;
  if (dynamic)
    for (int64_t t = t0; t < lo; ++t)               // the page's tokens before `start`, from the pool
      mm.add(reinterpret_cast<const uint16_t*>(kd + (t - t0) * kHeadDim)[lane], pl.ks[row0 + (t - t0)]);
  const bool full = lo == t0 && hi == t0 + PG;
  uint32_t a[PG / 4], c[PG / 4];                    // value codes of channels 2l / 2l + 1, 4 tokens a word
  static_assert(PG % 16 == 0, "pages of 16, 32 or 64 tokens");
#pragma unroll
  for (int c0 = 0; c0 < PG; c0 += 16) {             // chunks of 16 rows, all in flight at once
    if (t0 + c0 >= hi || t0 + c0 + 16 <= lo) continue;     // wave-uniform
    uint32_t kw[16], vw[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {                  // rows outside the range re-read row lo
      const int64_t t = t0 + c0 + u;
      const int64_t row = (int64_t)h * count + ((t >= lo && t < hi) ? t : lo) - start;
      kw[u] = k[row * 64 + lane];
      vw[u] = v[row * 64 + lane];
    }
    // the 32 rows' maxima spread over the lanes (chunk_row_maxima), each
    // lane's two rows' scales and brackets computed where they lie
    uint32_t kp[8], vp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kp[i] = pair_max_u16(kw[2 * i], kw[2 * i + 1]);
      vp[i] = pair_max_u16(vw[2 * i], vw[2 * i + 1]);
    }
    const uint32_t m = chunk_row_maxima(kp, vp);
    float s0, lo0, hi0, s1, lo1, hi1;               // rows 2i (low half) and 2i + 1 (high half)
    row_bracket(m & 0xFFFFu, s0, lo0, hi0);
    row_bracket(m >> 16, s1, lo1, hi1);
    {                                               // the scales: one lane of each 4 stores its two rows'
      const int i = 4 * ((lane >> 3) & 1) + fold_row(lane >> 4), r = c0 + 2 * i;
      float* dst = ((lane >> 2) & 1 ? pl.vs : pl.ks) + row0 + r;
      if ((lane & 3) == 0) {
        if (full) {
          *reinterpret_cast<float2*>(dst) = make_float2(s0, s1);
        } else {
          if (t0 + r >= lo && t0 + r < hi) dst[0] = s0;
          if (t0 + r + 1 >= lo && t0 + r + 1 < hi) dst[1] = s1;
        }
      }
    }
    uint32_t vcs[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int64_t t = t0 + c0 + u;
      vcs[u] = 0;
      if (t < lo || t >= hi) continue;              // wave-uniform
      const int lk = fold_lane(false, u >> 1), lv = fold_lane(true, u >> 1);
      const float sl = u & 1 ? s1 : s0, bl = u & 1 ? lo1 : lo0, bh = u & 1 ? hi1 : hi0;
      const uint32_t kc = codes_bracketed(kw[u], lane_value(bl, lk), lane_value(bh, lk), sl, lk);
      const uint32_t vc = codes_bracketed(vw[u], lane_value(bl, lv), lane_value(bh, lv), sl, lv);
      const int r = c0 + u;                         // row in the page
      reinterpret_cast<uint16_t*>(kd + r * kHeadDim)[lane] = (uint16_t)kc;
      vcs[u] = vc;
      if (!full) {
        vd[(2 * lane) * PG + r] = (uint8_t)vc;
        vd[(2 * lane + 1) * PG + r] = (uint8_t)(vc >> 8);
      }
      if (dynamic) mm.add(kc, lane_value(sl, lk));
    }
    if (full) {                                     // 4 rows' codes to one word per channel
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t t01 = __builtin_amdgcn_perm(vcs[4 * g + 1], vcs[4 * g], 0x05010400u);
        const uint32_t t23 = __builtin_amdgcn_perm(vcs[4 * g + 3], vcs[4 * g + 2], 0x05010400u);
        a[c0 / 4 + g] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
        c[c0 / 4 + g] = __builtin_amdgcn_perm(t23, t01, 0x07060302u);
      }
    }
  }
  if (full) {
    uint4* d0 = reinterpret_cast<uint4*>(vd + (2 * lane) * PG);
    uint4* d1 = reinterpret_cast<uint4*>(vd + (2 * lane + 1) * PG);
#pragma unroll
    for (int i = 0; i < PG / 16; ++i) {
      d0[i] = uint4{a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]};
      d1[i] = uint4{c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]};
    }
  }
  if (dynamic) mm.store(pl.summ + summ_page(pl, phys, hsl, lp), lane);
}

// Summaries rebuilt from the pool: grid (pages in range, B * dyn.n), one wave
// per (logical page, dynamic head); lane l takes channels 2l and 2l + 1 of the
// page's valid tokens, each load instruction one 256-byte key row.
template <int PG>
__global__ void __launch_bounds__(64) summary_kernel(PoolArgs pl, BatchArgs bt, HeadList dyn,
                                                     const int32_t* __restrict__ first_pos,
                                                     int32_t max_tokens) {
  const int32_t b = blockIdx.y / dyn.n, k = blockIdx.y % dyn.n, h = dyn.id[k];
  const int32_t hsl = head_slot(pl, h, k, true);     // (the list is in ascending head order)
  const int32_t L = clamp_len(bt, b, pl.P);
  if (L < 1) return;
  int32_t f = first_pos ? first_pos[b] : L - 1;
  if (f < 0) f = 0;
  if (f < L - max_tokens) f = L - max_tokens;      // pages beyond the bound are not refreshed
  if (f >= L) return;
  const int32_t j = f / PG + blockIdx.x;            // logical page to rebuild
  if ((int64_t)j * PG >= L) return;
  const int32_t phys = bt.pt[(int64_t)b * bt.max_pp + j / pl.r];
  if (phys < 0 || phys >= pl.N) return;
  const int32_t lp = j % pl.r;
  const int32_t n = min(PG, L - j * PG);            // valid tokens of the page
  const int lane = threadIdx.x;
  const uint32_t* kr = reinterpret_cast<const uint32_t*>(pl.k + k_row(pl, phys, hsl, lp * PG) * kHeadDim) + lane;
  uint32_t w[PG];
#pragma unroll
  for (int u = 0; u < PG; ++u) w[u] = kr[min(u, n - 1) * 64];   // rows past the valid ones repeat the last
  uint32_t lo0 = 0xFFFFFFFFu, hi0 = 0u, lo1 = 0xFFFFFFFFu, hi1 = 0u;
#pragma unroll
  for (int u = 0; u < PG; ++u) {
    const uint32_t x = order_key((uint16_t)w[u]), y = order_key((uint16_t)(w[u] >> 16));
    lo0 = min(lo0, x); hi0 = max(hi0, x);
    lo1 = min(lo1, y); hi1 = max(hi1, y);
  }
  uint32_t* sp = reinterpret_cast<uint32_t*>(pl.summ + summ_page(pl, phys, hsl, lp));
  sp[lane] = (uint32_t)from_key(lo0) | ((uint32_t)from_key(lo1) << 16);
  sp[kHeadDim / 2 + lane] = (uint32_t)from_key(hi0) | ((uint32_t)from_key(hi1) << 16);
}

// summary_kernel for fp8 pages: min / max of the dequantized keys in position
// order, rounded outward to bf16.
template <int PG>
__global__ void __launch_bounds__(64) summary_kernel_q8(PoolArgs pl, BatchArgs bt, HeadList dyn,
                                                        const int32_t* __restrict__ first_pos,
                                                        int32_t max_tokens) {
  const int32_t b = blockIdx.y / dyn.n, k = blockIdx.y % dyn.n, h = dyn.id[k];
  const int32_t hsl = head_slot(pl, h, k, true);     // (the list is in ascending head order)
  const int32_t L = clamp_len(bt, b, pl.P);
  if (L < 1) return;
  int32_t f = first_pos ? first_pos[b] : L - 1;
  if (f < 0) f = 0;
  if (f < L - max_tokens) f = L - max_tokens;      // pages beyond the bound are not refreshed
  if (f >= L) return;
  const int32_t j = f / PG + blockIdx.x;            // logical page to rebuild
  if ((int64_t)j * PG >= L) return;
  const int32_t phys = bt.pt[(int64_t)b * bt.max_pp + j / pl.r];
  if (phys < 0 || phys >= pl.N) return;
  const int32_t lp = j % pl.r;
  const int32_t n = min(PG, L - j * PG);            // valid tokens of the page
  const int lane = threadIdx.x;
  const int64_t row0 = k_row(pl, phys, hsl, lp * PG);
  const uint8_t* kr = reinterpret_cast<const uint8_t*>(pl.k) + row0 * kHeadDim;
  MinMax2 mm;
  for (int32_t u = 0; u < n; ++u)
    mm.add(reinterpret_cast<const uint16_t*>(kr + (int64_t)u * kHeadDim)[lane], pl.ks[row0 + u]);
  mm.store(pl.summ + summ_page(pl, phys, hsl, lp), lane);
}

}  // namespace

hipError_t launch_append(const PoolArgs& pool, const BatchArgs& batch, const uint16_t* k_new,
                         const uint16_t* v_new, const HeadList* dyn, hipStream_t s) {
  if (batch.B == 0) return hipSuccess;
  HeadList none;
  none.n = 0;
  hipLaunchKernelGGL(append_kernel, dim3(batch.B * pool.hkv), dim3(64), 0, s, pool, batch,
                     reinterpret_cast<const uint32_t*>(k_new), v_new, dyn ? *dyn : none,
                     dyn && dyn->n > 0 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_write(const PoolArgs& pool, const int32_t* pt_row, int64_t start, int64_t count,
                        const uint16_t* k, const uint16_t* v, const HeadList* dyn, int32_t ring_base,
                        int32_t ring_sink, int32_t ring_win, hipStream_t s) {
  if (count == 0) return hipSuccess;
  DynMask m = {};
  if (dyn)
    for (int32_t d = 0; d < dyn->n; ++d) m.w[dyn->id[d] >> 5] |= 1u << (dyn->id[d] & 31);
  const int64_t pages = (start + count - 1) / pool.p - start / pool.p + 1;
  const dim3 grid((unsigned)pages, pool.hkv);
  const uint32_t* k32 = reinterpret_cast<const uint32_t*>(k);
  const uint32_t* v32 = reinterpret_cast<const uint32_t*>(v);
  if (pool.q8) {
    switch (pool.p) {
      case 16: hipLaunchKernelGGL(write_kernel_q8<16>, grid, dim3(64), 0, s, pool, pt_row, start, count, k32, v32, m, ring_base, ring_sink, ring_win); break;
      case 32: hipLaunchKernelGGL(write_kernel_q8<32>, grid, dim3(64), 0, s, pool, pt_row, start, count, k32, v32, m, ring_base, ring_sink, ring_win); break;
      case 64: hipLaunchKernelGGL(write_kernel_q8<64>, grid, dim3(64), 0, s, pool, pt_row, start, count, k32, v32, m, ring_base, ring_sink, ring_win); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (pool.p) {
    case 16: hipLaunchKernelGGL(write_kernel<16>, grid, dim3(64), 0, s, pool, pt_row, start, count, k32, v32, m, ring_base, ring_sink, ring_win); break;
    case 32: hipLaunchKernelGGL(write_kernel<32>, grid, dim3(64), 0, s, pool, pt_row, start, count, k32, v32, m, ring_base, ring_sink, ring_win); break;
    case 64: hipLaunchKernelGGL(write_kernel<64>, grid, dim3(64), 0, s, pool, pt_row, start, count, k32, v32, m, ring_base, ring_sink, ring_win); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_summary(const PoolArgs& pool, const BatchArgs& batch, const HeadList& dyn,
                          const int32_t* first_pos, int32_t max_tokens, hipStream_t s) {
  if (batch.B == 0 || dyn.n == 0 || max_tokens < 1) return hipSuccess;
  // pages overlapping a range of max_tokens positions
  const int32_t pages = (max_tokens + pool.p - 1) / pool.p + 1;
  const dim3 grid(pages, batch.B * dyn.n);
  if (pool.q8) {
    switch (pool.p) {
      case 16: hipLaunchKernelGGL(summary_kernel_q8<16>, grid, dim3(64), 0, s, pool, batch, dyn, first_pos, max_tokens); break;
      case 32: hipLaunchKernelGGL(summary_kernel_q8<32>, grid, dim3(64), 0, s, pool, batch, dyn, first_pos, max_tokens); break;
      case 64: hipLaunchKernelGGL(summary_kernel_q8<64>, grid, dim3(64), 0, s, pool, batch, dyn, first_pos, max_tokens); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (pool.p) {
    case 16: hipLaunchKernelGGL(summary_kernel<16>, grid, dim3(64), 0, s, pool, batch, dyn, first_pos, max_tokens); break;
    case 32: hipLaunchKernelGGL(summary_kernel<32>, grid, dim3(64), 0, s, pool, batch, dyn, first_pos, max_tokens); break;
    case 64: hipLaunchKernelGGL(summary_kernel<64>, grid, dim3(64), 0, s, pool, batch, dyn, first_pos, max_tokens); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace spa
