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
  append_token(pl, bt, b, h, k_new, v_new, with_summary && is_dyn);
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
