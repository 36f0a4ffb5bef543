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
#include "spa_internal.h"

namespace spa {
namespace {

__device__ __forceinline__ int64_t k_row(const PoolArgs& pl, int32_t phys, int32_t h, int32_t slot) {
  return ((int64_t)phys * pl.hkv + h) * pl.P + slot;                 // row of D elements
}
__device__ __forceinline__ int64_t v_page(const PoolArgs& pl, int32_t phys, int32_t h, int32_t lp) {
  return (((int64_t)phys * pl.hkv + h) * pl.r + lp) * (int64_t)kHeadDim * pl.p;
}
__device__ __forceinline__ int64_t summ_page(const PoolArgs& pl, int32_t phys, int32_t h, int32_t lp) {
  return (((int64_t)phys * pl.hkv + h) * pl.r + lp) * (int64_t)(2 * kHeadDim);
}
__device__ __forceinline__ int32_t clamp_len(const BatchArgs& bt, int32_t b, int32_t P) {
  int32_t L = bt.lens[b];
  int32_t cap = bt.max_pp * P;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// bf16 bit pattern -> unsigned key that orders like IEEE totalOrder (finite
// values; -0 below +0), and back.
__device__ __forceinline__ uint32_t order_key(uint16_t x) {
  return (x & 0x8000u) ? (uint32_t)(~x & 0xFFFFu) : (uint32_t)(x | 0x8000u);
}
__device__ __forceinline__ uint16_t from_key(uint32_t k) {
  return (k & 0x8000u) ? (uint16_t)(k & 0x7FFFu) : (uint16_t)(~k & 0xFFFFu);
}

// One wave per (sequence, KV head): writes token L-1. Lane l owns channels
// 2l and 2l+1. When h is one of the dynamic heads, the same wave also rebuilds
// the summary of the logical page receiving the token: min and max over the
// page's earlier tokens (read from the pool, 16 rows per batch of loads) and
// the new key.
__global__ void __launch_bounds__(64) append_kernel(PoolArgs pl, BatchArgs bt,
                                                    const uint32_t* __restrict__ k_new,
                                                    const uint16_t* __restrict__ v_new,
                                                    HeadList dyn, int32_t with_summary) {
  const int32_t b = blockIdx.x / pl.hkv, h = blockIdx.x % pl.hkv;
  const int32_t L = clamp_len(bt, b, pl.P);
  if (L < 1) return;
  const int32_t t = L - 1;
  const int32_t phys = bt.pt[(int64_t)b * bt.max_pp + t / pl.P];
  if (phys < 0 || phys >= pl.N) return;
  const int32_t slot = t % pl.P, lp = slot / pl.p, i = slot % pl.p;
  const int lane = threadIdx.x;
  const int64_t src = ((int64_t)b * pl.hkv + h) * kHeadDim;
  const uint32_t kw = k_new[src / 2 + lane];
  uint16_t* krow0 = pl.k + k_row(pl, phys, h, lp * pl.p) * kHeadDim;   // first token of the page
  reinterpret_cast<uint32_t*>(krow0 + (int64_t)i * kHeadDim)[lane] = kw;
  uint16_t* vp = pl.v + v_page(pl, phys, h, lp);
  vp[(2 * lane) * pl.p + i] = v_new[src + 2 * lane];
  vp[(2 * lane + 1) * pl.p + i] = v_new[src + 2 * lane + 1];
  if (!with_summary) return;
  bool is_dyn = false;
  for (int32_t d = 0; d < dyn.n; ++d) is_dyn |= dyn.id[d] == h;
  if (!is_dyn) return;
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
  uint32_t* sp = reinterpret_cast<uint32_t*>(pl.summ + summ_page(pl, phys, h, lp));
  sp[lane] = (uint32_t)from_key(lo0) | ((uint32_t)from_key(lo1) << 16);
  sp[kHeadDim / 2 + lane] = (uint32_t)from_key(hi0) | ((uint32_t)from_key(hi1) << 16);
}

// Bulk write of one sequence: grid (ceil(count / 4), hkv), 256 threads =
// 4 tokens x 64 lanes of 2 channels.
__global__ void __launch_bounds__(256) write_kernel(PoolArgs pl, const int32_t* __restrict__ pt,
                                                    int32_t max_pp, int64_t start, int64_t count,
                                                    const uint32_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v) {
  const int32_t h = blockIdx.y;
  const int64_t n = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  if (n >= count) return;
  const int64_t t = start + n;
  const int32_t phys = pt[t / pl.P];
  if (phys < 0 || phys >= pl.N) return;
  const int32_t slot = (int32_t)(t % pl.P), lp = slot / pl.p, i = slot % pl.p;
  const int lane = threadIdx.x % 64;
  const int64_t src = ((int64_t)h * count + n) * kHeadDim;
  reinterpret_cast<uint32_t*>(pl.k + k_row(pl, phys, h, slot) * kHeadDim)[lane] = k[src / 2 + lane];
  uint16_t* vp = pl.v + v_page(pl, phys, h, lp);
  vp[(2 * lane) * pl.p + i] = v[src + 2 * lane];
  vp[(2 * lane + 1) * pl.p + i] = v[src + 2 * lane + 1];
}

// grid (pages in range, B * dyn.n), 128 threads = one channel each.
__global__ void __launch_bounds__(128) summary_kernel(PoolArgs pl, BatchArgs bt, HeadList dyn,
                                                      const int32_t* __restrict__ first_pos,
                                                      int32_t max_tokens) {
  const int32_t b = blockIdx.y / dyn.n, h = dyn.id[blockIdx.y % dyn.n];
  const int32_t L = clamp_len(bt, b, pl.P);
  if (L < 1) return;
  int32_t f = first_pos ? first_pos[b] : L - 1;
  if (f < 0) f = 0;
  if (f < L - max_tokens) f = L - max_tokens;      // pages beyond the bound are not refreshed
  if (f >= L) return;
  const int32_t j = f / pl.p + blockIdx.x;          // logical page to rebuild
  if ((int64_t)j * pl.p >= L) return;
  const int32_t phys = bt.pt[(int64_t)b * bt.max_pp + j / pl.r];
  if (phys < 0 || phys >= pl.N) return;
  const int32_t lp = j % pl.r;
  const int32_t t0 = j * pl.p, t1 = min(t0 + pl.p, L);
  const int c = threadIdx.x;
  const uint16_t* kr = pl.k + k_row(pl, phys, h, lp * pl.p) * kHeadDim + c;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int32_t t = 0; t < t1 - t0; ++t) {
    const uint32_t key = order_key(kr[(int64_t)t * kHeadDim]);
    lo = min(lo, key);
    hi = max(hi, key);
  }
  uint16_t* s = pl.summ + summ_page(pl, phys, h, lp);
  s[c] = from_key(lo);
  s[kHeadDim + c] = from_key(hi);
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

hipError_t launch_write(const PoolArgs& pool, const int32_t* pt_row, int32_t max_pp, int64_t start,
                        int64_t count, const uint16_t* k, const uint16_t* v, hipStream_t s) {
  if (count == 0) return hipSuccess;
  dim3 grid((unsigned)((count + 3) / 4), pool.hkv);
  hipLaunchKernelGGL(write_kernel, grid, dim3(256), 0, s, pool, pt_row, max_pp, start, count,
                     reinterpret_cast<const uint32_t*>(k), v);
  return hipGetLastError();
}

hipError_t launch_summary(const PoolArgs& pool, const BatchArgs& batch, const HeadList& dyn,
                          const int32_t* first_pos, int32_t max_tokens, hipStream_t s) {
  if (batch.B == 0 || dyn.n == 0 || max_tokens < 1) return hipSuccess;
  // pages overlapping a range of max_tokens positions
  const int32_t pages = (max_tokens + pool.p - 1) / pool.p + 1;
  dim3 grid(pages, batch.B * dyn.n);
  hipLaunchKernelGGL(summary_kernel, grid, dim3(128), 0, s, pool, batch, dyn, first_pos, max_tokens);
  return hipGetLastError();
}

}  // namespace spa
