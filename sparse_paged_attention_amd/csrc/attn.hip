// Unified sparse decode attention over the paged pool.
//
// One launch serves both head kinds (LServe write-up, bqwf.cn, "2.1": a fused
// block-sparse kernel handles static and dynamic sparsity together):
//   streaming head: tokens [0, min(sink, L)) U [max(sink, L - window), L)
//   dynamic head:   tokens of the selected logical pages (positions < L), plus
//                   the tokens appended since the selection, [L_s, L).
// Work is cut into items of a few 16-token blocks; each item runs the online
// softmax over its blocks and writes a partial (running max, running sum,
// unnormalised output), and a second kernel merges the partials of each query
// head (FlashAttention's tiled online softmax, long-context survey
// xllm-io.github.io "2.1"; the row-max / row-sum outputs of the Novita vLLM
// article, "2. 注意力机制修改").
//
// Per 16-token block one wave issues
//   S^T[16 tok][16 q] = K[16][128] . Q^T      4 x v_mfma_f32_16x16x32_bf16
//   O^T[128][16 q]   += V^T[128][16] . P^T    8 x 2 x v_mfma_f32_16x16x16_bf16
// The query group (G <= 16 heads sharing the KV head, grouped-query attention
// of the long-context survey "2.3") fills the 16 query columns; P is split
// into bf16 high and low parts so the products keep ~16 significant bits.
// Keys are stored token-major and values channel-major per logical page, so
// both tiles load straight from HBM into operand registers.
#include "spa_internal.h"

namespace spa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// log2(e) / sqrt(128): scores are kept in the log2 domain
constexpr float kScaleLog2 = 0.12751743074602467f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ int32_t clamp_len(const BatchArgs& bt, int32_t b, int32_t P) {
  int32_t L = bt.lens[b];
  int32_t cap = bt.max_pp * P;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// A 16-token block: absolute positions [t0, t0 + 16), of which [lo, hi) count,
// in physical page `phys` (already validated) at logical slot `lp`.
struct Block {
  int32_t t0, lo, hi, phys, lp;
};

// Operand registers of one block.
struct Tile {
  uint4 k[4];     // K rows: this lane's 64 bytes of token (lane & 15)
  uint2 v[8];     // V^T: channel 16c + (lane & 15), tokens 4*(lane>>4) .. +3
};

// Issues the loads of a block's tile. Empty blocks load from page 0 of the
// pool (always mapped), so the loads never depend on control flow.
template <int PG>
__device__ __forceinline__ void issue_tile(const PoolArgs& pl, int32_t h, const Block& blk, Tile& t) {
  const int lane = threadIdx.x & 63;
  const int row = lane & 15, quad = lane >> 4;
  const int64_t head = (int64_t)blk.phys * pl.hkv + h;
  const int32_t in_page = blk.t0 & (PG - 1);
  const uint4* k4 = reinterpret_cast<const uint4*>(
      pl.k + ((head * pl.P + blk.lp * PG + in_page + row) * kHeadDim + 32 * quad));
#pragma unroll
  for (int i = 0; i < 4; ++i) t.k[i] = k4[i];
  const uint16_t* vp = pl.v + ((head * pl.r + blk.lp) * kHeadDim + row) * PG + in_page + 4 * quad;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) t.v[ch] = *reinterpret_cast<const uint2*>(vp + 16 * ch * PG);
}

struct State {
  float m;          // running max of this lane's query, log2 domain
  float l;          // running sum over this lane's tokens
  f32x4 o[8];       // O^T: channels 16c + 4*quad + r of query (lane & 15)
};

// Cross-lane max over the four 16-lane rows (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float max_over_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// Scores S^T[16 tok][16 q] of one block: 4 chained 16x16x32 MFMAs over D.
__device__ __forceinline__ f32x4 qk_block(const Tile& t, const bf16x8 (&qb)[4]) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16x8 a;
    __builtin_memcpy(&a, &t.k[i], 16);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[i], s, 0, 0, 0);
  }
  return s;
}

// Two blocks (32 tokens) at once. The PV product contracts over 32 tokens
// with one 16x16x32 MFMA per 16 channels: K-slot j of lane row q holds token
// 4q + j of block a (j < 4) or token 4q + j - 4 of block b (j >= 4), which is
// exactly where the QK products left this lane's probabilities.
__device__ __forceinline__ void process_pair(const Block& ba, const Tile& ta, const Block& bb,
                                             const Tile& tb, const bf16x8 (&qb)[4], State& st) {
  const int lane = threadIdx.x & 63;
  const int quad = lane >> 4;
  const f32x4 sa = qk_block(ta, qb);
  const f32x4 sb = qk_block(tb, qb);
  float x[8];
  bool valid[8];
  float bm = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int32_t tka = ba.t0 + 4 * quad + r, tkb = bb.t0 + 4 * quad + r;
    valid[r] = tka >= ba.lo && tka < ba.hi;
    valid[4 + r] = tkb >= bb.lo && tkb < bb.hi;
    x[r] = valid[r] ? sa[r] * kScaleLog2 : -INFINITY;
    x[4 + r] = valid[4 + r] ? sb[r] * kScaleLog2 : -INFINITY;
    bm = fmaxf(bm, fmaxf(x[r], x[4 + r]));
  }
  bm = max_over_rows(bm);
  if (bm == -INFINITY) return;                    // no valid token (same for every lane)
  const float m_new = fmaxf(st.m, bm);
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  float pr[8];
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    pr[r] = __builtin_amdgcn_exp2f(x[r] - m_new);  // 0 for masked tokens
    psum += pr[r];
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) st.o[ch] *= alpha;
  }
  bf16x8 phi, plo;
  {
    uint16_t hb[8], lb[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      hb[r] = bf16_rne(pr[r]);
      lb[r] = bf16_rne(pr[r] - __uint_as_float((uint32_t)hb[r] << 16));
    }
    __builtin_memcpy(&phi, hb, 16);
    __builtin_memcpy(&plo, lb, 16);
  }
  const bool full = ba.lo <= ba.t0 && ba.hi >= ba.t0 + kBlockTokens &&
                    bb.lo <= bb.t0 && bb.hi >= bb.t0 + kBlockTokens;
  uint32_t mk[4];
#pragma unroll
  for (int w = 0; w < 4; ++w)
    mk[w] = (valid[2 * w] ? 0x0000FFFFu : 0u) | (valid[2 * w + 1] ? 0xFFFF0000u : 0u);
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    uint4 w = {ta.v[ch].x, ta.v[ch].y, tb.v[ch].x, tb.v[ch].y};
    if (!full) {                                   // stale pool bytes must not reach the MFMA
      w.x &= mk[0];
      w.y &= mk[1];
      w.z &= mk[2];
      w.w &= mk[3];
    }
    bf16x8 a;
    __builtin_memcpy(&a, &w, 16);
    st.o[ch] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi, st.o[ch], 0, 0, 0);
    st.o[ch] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo, st.o[ch], 0, 0, 0);
  }
}

__device__ __forceinline__ bool page_selected(const int32_t* sel, int32_t cnt, int32_t j) {
  int32_t lo = 0, hi = cnt;                        // ascending ids
  while (lo < hi) {
    const int32_t mid = (lo + hi) >> 1;
    const int32_t x = sel[mid];
    if (x == j) return true;
    if (x < j) lo = mid + 1; else hi = mid;
  }
  return false;
}

// Which blocks an item covers. Blocks are numbered per head:
//   streaming: the sink blocks, then the window blocks;
//   dynamic:   block (i, s) = 16-token block s of the i-th selected page;
//   tail:      16-token blocks of [floor16(L_s), L) outside selected pages.
struct BlockSource {
  int32_t kind;          // 0 streaming, 1 dynamic, 2 tail
  int32_t L;
  int32_t s0, w0, nb_sink, first_w;          // streaming
  const int32_t* sel;
  int32_t cnt, k_max;                        // dynamic / tail
  int32_t ls_floor, ls;                      // tail
};

// Resolves blocks [v0, v0 + BPI) (those at or past v_end are empty) to pool
// locations, then streams them through a ring of DEPTH operand tiles: the
// first DEPTH blocks' loads are issued together, and each tile is refilled
// with block u + DEPTH as soon as block u has been computed. Every lookup
// (selected page ids, page-table entries) is issued unconditionally with a
// clamped index, so each level of the lookup costs one memory round trip for
// the whole item. The kernel has a single call site, so one copy of the
// pipeline serves every kind of item (instruction-cache footprint).
template <int PG, int BPI, int DEPTH>
__device__ __forceinline__ void run_blocks(const PoolArgs& pl, const int32_t* pt_row,
                                           int32_t max_pp, int32_t h, const BlockSource& src,
                                           int32_t v0, int32_t v_end, const bf16x8 (&qb)[4],
                                           State& st) {
  constexpr int SB = PG / kBlockTokens;           // blocks per logical page
  const int32_t L = src.L;
  const int32_t n_pages = (L + PG - 1) / PG;
  Block blk[BPI];
  if (src.kind == 1) {
    int32_t page[BPI];
#pragma unroll
    for (int u = 0; u < BPI; ++u) {
      const int32_t i = min((v0 + u) / SB, src.k_max - 1);
      page[u] = src.sel[i];
    }
#pragma unroll
    for (int u = 0; u < BPI; ++u) {
      const int32_t j = page[u];
      const bool ok = v0 + u < v_end && j >= 0 && j < n_pages;
      const int32_t t0 = ok ? j * PG + ((v0 + u) % SB) * kBlockTokens : 0;
      blk[u] = Block{t0, t0, ok ? min(t0 + kBlockTokens, L) : t0, 0, 0};
    }
  } else if (src.kind == 0) {
#pragma unroll
    for (int u = 0; u < BPI; ++u) {
      const int32_t v = v0 + u;
      int32_t t0, lo, hi;
      if (v < src.nb_sink) {
        t0 = v * kBlockTokens; lo = t0; hi = min(t0 + kBlockTokens, src.s0);
      } else {
        t0 = (src.first_w + v - src.nb_sink) * kBlockTokens; lo = max(t0, src.w0); hi = min(t0 + kBlockTokens, L);
      }
      if (v >= v_end) { t0 = 0; lo = 0; hi = 0; }
      blk[u] = Block{t0, lo, hi, 0, 0};
    }
  } else {
#pragma unroll
    for (int u = 0; u < BPI; ++u) {
      const int32_t t0 = src.ls_floor + (v0 + u) * kBlockTokens;
      int32_t lo = max(t0, src.ls), hi = min(t0 + kBlockTokens, L);
      if (v0 + u >= v_end || page_selected(src.sel, src.cnt, t0 / PG)) hi = lo;
      blk[u] = Block{hi > lo ? t0 : 0, lo, hi, 0, 0};
    }
  }
  int32_t ptv[BPI];
#pragma unroll
  for (int u = 0; u < BPI; ++u) {
    const int32_t slot = min((blk[u].t0 / PG) / (pl.P / PG), max_pp - 1);
    ptv[u] = pt_row[slot];
  }
#pragma unroll
  for (int u = 0; u < BPI; ++u) {
    const int32_t j = blk[u].t0 / PG;
    int32_t phys = ptv[u];
    if (phys < 0 || phys >= pl.N || blk[u].hi <= blk[u].lo) { phys = 0; blk[u].hi = blk[u].lo; blk[u].t0 = 0; }
    blk[u].phys = phys;
    blk[u].lp = blk[u].hi > blk[u].lo ? j % (pl.P / PG) : 0;
  }
  // blocks go in pairs; DEPTH (even) tiles are in flight
  static_assert(BPI % 2 == 0 && DEPTH % 2 == 0, "blocks are processed in pairs");
  constexpr int D = DEPTH < BPI ? DEPTH : BPI;
  Tile t[D];
#pragma unroll
  for (int u = 0; u < D; ++u) issue_tile<PG>(pl, h, blk[u], t[u]);
#pragma unroll
  for (int u = 0; u < BPI; u += 2) {
    if (blk[u].lo < blk[u].hi || blk[u + 1].lo < blk[u + 1].hi)
      process_pair(blk[u], t[u % D], blk[u + 1], t[(u + 1) % D], qb, st);
    if (u + D < BPI) {
      issue_tile<PG>(pl, h, blk[u + D], t[u % D]);
      issue_tile<PG>(pl, h, blk[u + 1 + D], t[(u + 1) % D]);
    }
  }
}

// One item of one (sequence, KV head): the online softmax over its blocks and
// a partial (max, sum, unnormalised output) per query head. Items are laid
// out as [streaming: B x n_stream x items_stream][dynamic: B x n_dyn x items_dyn].
template <int PG, int BPI, int DEPTH>
__global__ void __launch_bounds__(64) attn_kernel(PoolArgs pl, BatchArgs bt, AttnPlan plan, int32_t G,
                                                  const uint16_t* __restrict__ q,
                                                  const int32_t* __restrict__ sel_pages,
                                                  const int32_t* __restrict__ sel_count,
                                                  const int32_t* __restrict__ sel_len,
                                                  float* __restrict__ part_o,
                                                  float* __restrict__ part_ml) {
  int32_t idx = blockIdx.x;
  const int32_t n_stream_items = bt.B * plan.n_stream * plan.items_stream;
  const bool dynamic = idx >= n_stream_items;
  int32_t b, h, it;
  if (!dynamic) {
    const int32_t per_b = plan.n_stream * plan.items_stream;
    b = idx / per_b;
    const int32_t r = idx % per_b;
    h = plan.stream_ids[r / plan.items_stream];
    it = r % plan.items_stream;
  } else {
    idx -= n_stream_items;
    const int32_t per_b = plan.n_dyn * plan.items_dyn;
    b = idx / per_b;
    const int32_t r = idx % per_b;
    h = plan.dyn_ids[r / plan.items_dyn];
    it = r % plan.items_dyn;
  }
  const int32_t n_items = dynamic ? plan.items_dyn : plan.items_stream;
  // independent loads first: length, selection count / length, query
  const int32_t L = clamp_len(bt, b, pl.P);
  int32_t cnt = 0, ls = 0;
  if (dynamic) {
    cnt = min(max(sel_count[(int64_t)b * pl.hkv + h], 0), plan.k_max);
    ls = sel_len[b];
  }
  const int lane = threadIdx.x & 63;
  const int g = lane & 15, quad = lane >> 4;
  const int32_t* pt_row = bt.pt + (int64_t)b * bt.max_pp;

  // query operand: Q[g][32*quad + 8*i .. +8], zero for g >= G
  bf16x8 qb[4];
  const int32_t hq = pl.hkv * G;
  {
    const int32_t gq = g < G ? g : 0;
    const uint4* q4 = reinterpret_cast<const uint4*>(q + ((int64_t)b * hq + h * G + gq) * kHeadDim + 32 * quad);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 w = q4[i];
      if (g >= G) w = uint4{0, 0, 0, 0};
      __builtin_memcpy(&qb[i], &w, 16);
    }
  }

  State st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) st.o[ch] = f32x4{0.f, 0.f, 0.f, 0.f};

  BlockSource src;
  src.L = L;
  src.sel = sel_pages + ((int64_t)b * pl.hkv + h) * plan.k_max;
  src.cnt = cnt;
  src.k_max = plan.k_max;
  if (L > 0) {
    int32_t v_begin = it * BPI, v_end;
    if (!dynamic) {
      src.kind = 0;
      src.s0 = min(plan.sink, L);
      src.w0 = max(plan.sink, L - plan.window);
      src.nb_sink = (src.s0 + kBlockTokens - 1) / kBlockTokens;
      src.first_w = src.w0 / kBlockTokens;
      const int32_t nb_win = L > src.w0 ? (L - 1) / kBlockTokens - src.first_w + 1 : 0;
      v_end = min(src.nb_sink + nb_win, v_begin + BPI);
    } else if (it < n_items - 1) {
      src.kind = 1;
      v_end = min(cnt * (PG / kBlockTokens), v_begin + BPI);
    } else {
      src.kind = 2;
      src.ls = min(max(ls, 0), L);
      src.ls_floor = (src.ls / kBlockTokens) * kBlockTokens;
      v_begin = 0;
      v_end = (L - src.ls_floor + kBlockTokens - 1) / kBlockTokens;   // any length: chunks of BPI
    }
    for (int32_t v0 = v_begin; v0 < v_end; v0 += BPI)
      run_blocks<PG, BPI, DEPTH>(pl, pt_row, bt.max_pp, h, src, v0, v_end, qb, st);
  }

  // fold the four token quads of the running sum, store the partial
  st.l += __shfl_xor(st.l, 16, 64);
  st.l += __shfl_xor(st.l, 32, 64);
  const int64_t slot0 = ((int64_t)b * pl.hkv + h) * plan.item_stride * G;
  if (g < G) {
    const int64_t slot = slot0 + (int64_t)it * G + g;
    float* o = part_o + slot * kHeadDim + 4 * quad;
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) *reinterpret_cast<f32x4*>(o + 16 * ch) = st.o[ch];
    if (quad == 0) {
      part_ml[slot * 2 + 0] = st.m;
      part_ml[slot * 2 + 1] = st.l;
    }
  }

}

// Merge of the item partials of one (sequence, KV head): the running-max /
// running-sum rule of online softmax applied across items. Thread (g, d) owns
// channel d of query g; the items' (max, sum) pairs are staged in LDS first so
// every output channel's loads are independent and in flight together.
constexpr int kCombineThreads = 512;
constexpr int kMaxItemsLds = kMaxPartialsPerHead;

__global__ void __launch_bounds__(kCombineThreads) combine_kernel(int32_t hkv, AttnPlan plan, int32_t G,
                                                                  const float* __restrict__ part_o,
                                                                  const float* __restrict__ part_ml,
                                                                  float* __restrict__ out,
                                                                  float* __restrict__ lse) {
  __shared__ float sm[kMaxItemsLds], sl[kMaxItemsLds];
  __shared__ float sM[16];
  const int32_t b = blockIdx.x / hkv, h = blockIdx.x % hkv;
  const int32_t n_items = plan.kind[h] ? plan.items_dyn : plan.items_stream;
  const int64_t slot0 = ((int64_t)b * hkv + h) * plan.item_stride * G;   // slot(i, g) = slot0 + i*G + g
  const int32_t n_ml = n_items * G;                                     // <= kMaxItemsLds (host check)
  for (int32_t k = threadIdx.x; k < n_ml; k += kCombineThreads) {
    sm[k] = part_ml[(slot0 + k) * 2];
    sl[k] = part_ml[(slot0 + k) * 2 + 1];
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float M = -INFINITY;
    for (int32_t i = 0; i < n_items; ++i) M = fmaxf(M, sm[i * G + threadIdx.x]);
    sM[threadIdx.x] = M;
  }
  __syncthreads();
  const int32_t hq = hkv * G;
  for (int32_t gd = threadIdx.x; gd < G * kHeadDim; gd += kCombineThreads) {
    const int32_t g = gd / kHeadDim, d = gd % kHeadDim;
    const float M = sM[g];
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll 8
      for (int32_t i = 0; i < n_items; ++i) {
        const float w = __builtin_amdgcn_exp2f(sm[i * G + g] - M);
        den += w * sl[i * G + g];
        num += w * part_o[(slot0 + (int64_t)i * G + g) * kHeadDim + d];
      }
    }
    const int64_t oi = (int64_t)b * hq + h * G + g;
    out[oi * kHeadDim + d] = M == -INFINITY ? 0.f : num / den;
    if (lse && d == 0) lse[oi] = M == -INFINITY ? -INFINITY : (M + log2f(den)) * kLn2;
  }
}

template <int PG, int BPI, int DEPTH = 4>
hipError_t launch_attn_t(const PoolArgs& pool, const BatchArgs& batch, const AttnPlan& plan, int32_t G,
                         const uint16_t* q, const int32_t* sel_pages, const int32_t* sel_count,
                         const int32_t* sel_len, float* part_o, float* part_ml, int32_t* tickets,
                         float* out, float* lse, hipStream_t s) {
  const int64_t grid = (int64_t)batch.B * (plan.n_stream * plan.items_stream + plan.n_dyn * plan.items_dyn);
  hipLaunchKernelGGL((attn_kernel<PG, BPI, DEPTH>), dim3((unsigned)grid), dim3(64), 0, s, pool, batch, plan, G, q,
                     sel_pages, sel_count, sel_len, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(batch.B * pool.hkv), dim3(kCombineThreads), 0, s, pool.hkv, plan, G,
                     part_o, part_ml, out, lse);
  return hipGetLastError();
}

template <int PG>
hipError_t launch_attn_p(const PoolArgs& pool, const BatchArgs& batch, const AttnPlan& plan, int32_t G,
                         const uint16_t* q, const int32_t* sel_pages, const int32_t* sel_count,
                         const int32_t* sel_len, float* part_o, float* part_ml, int32_t* tickets,
                         float* out, float* lse, hipStream_t s) {
  switch (plan.blocks_per_item) {
    case 4: return launch_attn_t<PG, 4>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, tickets, out, lse, s);
    case 8: return launch_attn_t<PG, 8>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, tickets, out, lse, s);
    case 16: return launch_attn_t<PG, 16>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, tickets, out, lse, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn(const PoolArgs& pool, const BatchArgs& batch, const AttnPlan& plan, int32_t G,
                       const uint16_t* q, const int32_t* sel_pages, const int32_t* sel_count,
                       const int32_t* sel_len, float* out, float* lse, float* part_o,
                       float* part_ml, int32_t* tickets, hipStream_t s) {
  if (batch.B == 0) return hipSuccess;
  switch (pool.p) {
    case 16: return launch_attn_p<16>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, tickets, out, lse, s);
    case 32: return launch_attn_p<32>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, tickets, out, lse, s);
    case 64: return launch_attn_p<64>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, part_o, part_ml, tickets, out, lse, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spa
