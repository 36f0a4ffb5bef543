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
