// Device-side addressing of the page pool and the one-token append, shared by
// the pool kernels and the attention kernel (which can run the append in its
// own launch).
//
// LServe write-up (bqwf.cn), "2.2 分层分页KV缓存": tokens live in logical
// pages (the selection unit) packed inside physical pages (the allocation
// unit); "2.1 混合稀疏注意力机制": each logical page of a dynamic head is
// summarised by the channel-wise min and max of its keys.
//
// In-page layout: keys token-major [P][D] per (physical page, head); values
// channel-major [D][p] per logical page; summaries [2][D] (min row, max row)
// per logical page.
#pragma once
#include "spa_internal.h"

namespace spa {
namespace {

// hsl: the head's slot in its physical page (head_slot)
__device__ __forceinline__ int64_t k_row(const PoolArgs& pl, int32_t phys, int32_t hsl, int32_t row) {
  return ((int64_t)phys * pl.hs + hsl) * pl.P + row;                  // row of D elements
}
__device__ __forceinline__ int64_t v_page(const PoolArgs& pl, int32_t phys, int32_t hsl, int32_t lp) {
  return (((int64_t)phys * pl.hs + hsl) * pl.r + lp) * (int64_t)kHeadDim * pl.p;
}
__device__ __forceinline__ int64_t summ_page(const PoolArgs& pl, int32_t phys, int32_t hsl, int32_t lp) {
  return (((int64_t)phys * pl.hs + hsl) * pl.r + lp) * (int64_t)(2 * kHeadDim);
}
// Slot of KV head h in its physical page: h, or, when pages hold fewer slots
// than heads (compact layout), its rank among the heads of its kind.
// dyn_below: dynamic heads with an index below h.
__device__ __forceinline__ int32_t head_slot(const PoolArgs& pl, int32_t h, int32_t dyn_below, bool dynamic) {
  return pl.hs == pl.hkv ? h : (dynamic ? dyn_below : h - dyn_below);
}
// Dynamic heads below h in an ascending head list.
__device__ __forceinline__ int32_t dyn_rank(const HeadList& dyn, int32_t h) {
  int32_t n = 0;
  for (int32_t d = 0; d < dyn.n; ++d) n += dyn.id[d] < h;
  return n;
}
__device__ __forceinline__ int32_t clamp_len(const BatchArgs& bt, int32_t b, int32_t P) {
  int32_t L = bt.lens[b];
  int32_t cap = bt.max_pp * P;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// Physical page of position t of a streaming head in the ring that starts at
// `base` (the sink's pages, then the window's pages reused in turn: the
// window spans at most ring_win pages, so the pages it covers never share a
// slot), or -1 when the ring does not lie inside the pool.
__device__ __forceinline__ int32_t ring_page(const BatchArgs& bt, int32_t base, int32_t t, int32_t P, int32_t N) {
  const int32_t pg = t / P;
  const int32_t slot = pg < bt.ring_sink ? pg : bt.ring_sink + (pg - bt.ring_sink) % bt.ring_win;
  return base >= 0 && base <= N - (bt.ring_sink + bt.ring_win) ? base + slot : -1;
}

// bf16 bit pattern -> unsigned key that orders like IEEE totalOrder (finite
// values; -0 below +0), and back.
__device__ __forceinline__ uint32_t order_key(uint16_t x) {
  return (x & 0x8000u) ? (uint32_t)(~x & 0xFFFFu) : (uint32_t)(x | 0x8000u);
}
__device__ __forceinline__ uint16_t from_key(uint32_t k) {
  return (k & 0x8000u) ? (uint16_t)(k & 0x7FFFu) : (uint16_t)(~k & 0xFFFFu);
}

// ---- fp8 pages -------------------------------------------------------------
// OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest
// finite 448). A row is quantized with one fp32 scale, amax / 448; each code
// is the nearest E4M3 value of x / scale, ties to even.

// Code of a finite fp32 value, from its bit pattern: nearest, ties to even,
// saturating at 448.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u, a = u & 0x7FFFFFFFu;
  uint32_t c;
  if (a >= 0x43E00000u) {                          // |y| >= 448
    c = 0x7Eu;
  } else if (a < 0x3C800000u) {                    // |y| < 2^-6: multiples of 2^-9 (8 * 2^-9 is code 8)
    c = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.f);
  } else {                                         // exponent field 1..15, 3 mantissa bits kept
    const uint32_t m = (a >> 20) & 7u, rest = a & 0xFFFFFu;
    c = ((((a >> 23) - 120u)) << 3) | m;
    if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) c += 1;   // a carry moves into the exponent
    c = c > 0x7Eu ? 0x7Eu : c;
  }
  return sign | c;
}

// Value of a code (never one of the NaN codes), exact in fp32.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return (c & 0x80u) ? -v : v;
}

// Largest bf16 <= x and smallest bf16 >= x, as bit patterns.
__device__ __forceinline__ uint32_t bf16_down(double x) {
  const uint32_t u = __float_as_uint(__double2float_rd(x));   // largest fp32 <= x
  uint32_t b = u >> 16;                                         // toward zero
  if ((u & 0xFFFFu) && (u >> 31)) b += 1;                       // negative: one step further down
  return b;
}
__device__ __forceinline__ uint32_t bf16_up(double x) { return bf16_down(-x) ^ 0x8000u; }

// Quantizes one D = 128 row held by a wave as bf16 pairs (lane l: channels 2l
// and 2l + 1, in w). Returns the lane's two codes (bits 0-7 and 8-15) and sets
// the row's scale. Every lane of the wave must take part (cross-lane max).
__device__ __forceinline__ uint32_t quantize_pair(uint32_t w, float& scale) {
  const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xFFFF0000u);
  float a = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
  for (int o = 32; o; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
  scale = a / 448.f;
  if (scale == 0.f) return 0;
  return e4m3_code(x0 / scale) | (e4m3_code(x1 / scale) << 8);
}

// Running min / max in IEEE totalOrder (-0 below +0, the order of the bf16
// summaries) of the dequantized values of the lane's two channels (codes in
// bits 0-7 / 8-15 of c2).
struct MinMax2 {
  double lo0 = INFINITY, hi0 = -INFINITY, lo1 = INFINITY, hi1 = -INFINITY;
  __device__ __forceinline__ static void fold(double v, double& lo, double& hi) {
    if (v < lo || (v == lo && __signbit(v))) lo = v;
    if (v > hi || (v == hi && !__signbit(v))) hi = v;
  }
  __device__ __forceinline__ void add(uint32_t c2, float scale) {
    fold((double)e4m3_value(c2 & 0xFFu) * (double)scale, lo0, hi0);     // products exact in fp64
    fold((double)e4m3_value((c2 >> 8) & 0xFFu) * (double)scale, lo1, hi1);
  }
  // the summary rows of the page, rounded outward to bf16
  __device__ __forceinline__ void store(uint16_t* summ_page_base, int lane) const {
    uint32_t* sp = reinterpret_cast<uint32_t*>(summ_page_base);
    sp[lane] = bf16_down(lo0) | (bf16_down(lo1) << 16);
    sp[kHeadDim / 2 + lane] = bf16_up(hi0) | (bf16_up(hi1) << 16);
  }
};

// The outward-rounded bf16 min / max words (channels 2 lane and 2 lane + 1)
// of one quantized key row merged into a stored summary record: channel-wise
// totalOrder min of the stored minimum and the new key rounded down, max of
// the stored maximum and the new key rounded up; the new key alone when it
// opens the page. Rounding outward is monotone, so this equals the rebuild
// over all of the page's keys.
__device__ __forceinline__ void merge_q8_summary(uint16_t* summ_rec, int lane, uint32_t c2, float scale,
                                                 bool opens) {
  uint32_t* sp = reinterpret_cast<uint32_t*>(summ_rec);
  const double v0 = (double)e4m3_value(c2 & 0xFFu) * (double)scale;
  const double v1 = (double)e4m3_value((c2 >> 8) & 0xFFu) * (double)scale;
  const uint32_t dn0 = bf16_down(v0), dn1 = bf16_down(v1), up0 = bf16_up(v0), up1 = bf16_up(v1);
  uint32_t lo = dn0 | (dn1 << 16), hi = up0 | (up1 << 16);
  if (!opens) {
    const uint32_t smin = sp[lane], smax = sp[kHeadDim / 2 + lane];
    uint32_t l2 = 0, h2 = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t a = order_key((uint16_t)(smin >> (16 * half))), n = order_key((uint16_t)(lo >> (16 * half)));
      const uint32_t c = order_key((uint16_t)(smax >> (16 * half))), m = order_key((uint16_t)(hi >> (16 * half)));
      l2 |= (uint32_t)from_key(min(a, n)) << (16 * half);
      h2 |= (uint32_t)from_key(max(c, m)) << (16 * half);
    }
    lo = l2;
    hi = h2;
  }
  sp[lane] = lo;
  sp[kHeadDim / 2 + lane] = hi;
}

// Writes token L-1 of sequence b, KV head h into an fp8 pool from its
// quantized rows (lane l: the codes of channels 2l, 2l + 1 in bits 0-15 of kc
// / vc; ks / vs the row scales); with `summary`, the new key is merged into
// the stored summary of its logical page (merge_q8_summary), so the page's
// earlier rows are not read again.
__device__ __forceinline__ void store_token_q8(const PoolArgs& pl, const BatchArgs& bt, int32_t b, int32_t hsl,
                                               uint32_t kc, float ks, uint32_t vc, float vs, bool summary,
                                               bool in_ring) {
  const int lane = threadIdx.x & 63;
  const int32_t L = clamp_len(bt, b, pl.P);
  if (L < 1) return;
  const int32_t t = L - 1;
  const int32_t phys = in_ring ? ring_page(bt, bt.ring[b], t, pl.P, pl.N) : bt.pt[(int64_t)b * bt.max_pp + t / pl.P];
  if (phys < 0 || phys >= pl.N) return;
  const int32_t slot = t % pl.P, lp = slot / pl.p, i = slot % pl.p;
  const int64_t row0 = k_row(pl, phys, hsl, lp * pl.p);               // the page's first token row
  uint8_t* krow0 = reinterpret_cast<uint8_t*>(pl.k) + row0 * kHeadDim;
  reinterpret_cast<uint16_t*>(krow0 + (int64_t)i * kHeadDim)[lane] = (uint16_t)kc;
  uint8_t* vp = reinterpret_cast<uint8_t*>(pl.v) + v_page(pl, phys, hsl, lp);
  vp[(2 * lane) * pl.p + i] = (uint8_t)vc;
  vp[(2 * lane + 1) * pl.p + i] = (uint8_t)(vc >> 8);
  if (lane == 0) {
    pl.ks[row0 + i] = ks;
    pl.vs[row0 + i] = vs;
  }
  if (summary) merge_q8_summary(pl.summ + summ_page(pl, phys, hsl, lp), lane, kc, ks, i == 0);
}

// append_token for fp8 pages: the key and value rows are quantized (one scale
// each) and stored (store_token_q8). k_new / v_new: bf16 [B][H_kv][D] as
// 32-bit pairs.
__device__ __forceinline__ void append_token_q8(const PoolArgs& pl, const BatchArgs& bt, int32_t b, int32_t h,
                                                int32_t hsl, const uint32_t* __restrict__ k_new,
                                                const uint32_t* __restrict__ v_new, bool summary, bool in_ring) {
  const int lane = threadIdx.x & 63;
  const int64_t src = ((int64_t)b * pl.hkv + h) * (kHeadDim / 2);
  const uint32_t kin = k_new[src + lane], vin = v_new[src + lane];
  float ks, vs;
  const uint32_t kc = quantize_pair(kin, ks);     // every lane takes part (cross-lane max)
  const uint32_t vc = quantize_pair(vin, vs);
  store_token_q8(pl, bt, b, hsl, kc, ks, vc, vs, summary, in_ring);
}

// One wave writes token L-1 of sequence b, KV head h into its pool slot; lane
// l owns channels 2l and 2l+1. With `summary`, the same wave rebuilds the
// summary of the logical page receiving the token: min and max over the
// page's earlier tokens (read from the pool, 16 rows per batch of loads) and
// the new key. `in_ring`: a streaming head kept in the sequence's ring; hsl:
// the head's slot in its page. k_new / v_new: bf16 [B][H_kv][D].
__device__ __forceinline__ void append_token(const PoolArgs& pl, const BatchArgs& bt, int32_t b, int32_t h,
                                             int32_t hsl, const uint32_t* __restrict__ k_new,
                                             const uint16_t* __restrict__ v_new, bool summary, bool in_ring) {
  const int32_t L = clamp_len(bt, b, pl.P);
  if (L < 1) return;
  const int32_t t = L - 1;
  const int32_t phys = in_ring ? ring_page(bt, bt.ring[b], t, pl.P, pl.N) : bt.pt[(int64_t)b * bt.max_pp + t / pl.P];
  if (phys < 0 || phys >= pl.N) return;
  const int32_t slot = t % pl.P, lp = slot / pl.p, i = slot % pl.p;
  const int lane = threadIdx.x & 63;
  const int64_t src = ((int64_t)b * pl.hkv + h) * kHeadDim;
  const uint32_t kw = k_new[src / 2 + lane];
  uint16_t* krow0 = pl.k + k_row(pl, phys, hsl, lp * pl.p) * kHeadDim;   // first token of the page
  reinterpret_cast<uint32_t*>(krow0 + (int64_t)i * kHeadDim)[lane] = kw;
  uint16_t* vp = pl.v + v_page(pl, phys, hsl, lp);
  vp[(2 * lane) * pl.p + i] = v_new[src + 2 * lane];
  vp[(2 * lane + 1) * pl.p + i] = v_new[src + 2 * lane + 1];
  if (!summary) return;
  uint32_t lo0 = order_key((uint16_t)kw), hi0 = lo0;
  uint32_t lo1 = order_key((uint16_t)(kw >> 16)), hi1 = lo1;
  for (int32_t r0 = 0; r0 < i; r0 += 16) {           // the page's earlier tokens
    uint32_t w[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)                      // rows past i-1 re-read row i (the new key)
      w[u] = reinterpret_cast<const uint32_t*>(krow0 + (int64_t)min(r0 + u, i) * kHeadDim)[lane];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint32_t a = order_key((uint16_t)w[u]), c = order_key((uint16_t)(w[u] >> 16));
      lo0 = min(lo0, a); hi0 = max(hi0, a);
      lo1 = min(lo1, c); hi1 = max(hi1, c);
    }
  }
  uint32_t* sp = reinterpret_cast<uint32_t*>(pl.summ + summ_page(pl, phys, hsl, lp));
  sp[lane] = (uint32_t)from_key(lo0) | ((uint32_t)from_key(lo1) << 16);
  sp[kHeadDim / 2 + lane] = (uint32_t)from_key(hi0) | ((uint32_t)from_key(hi1) << 16);
}

}  // namespace
}  // namespace spa
