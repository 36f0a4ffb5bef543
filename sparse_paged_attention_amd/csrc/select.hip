// Query-aware page selection for dynamic heads.
//
// LServe write-up (bqwf.cn), "2.1 混合稀疏注意力机制": at decode time a
// dynamic head scores each block by the similarity of the query to the
// block's min-max pooled keys and keeps the most relevant blocks under a token
// budget; "3.2 解码阶段加速" sets the budget to min(4096, L/32) and reruns the
// selection only every few tokens. The score used here is the largest q.k a
// key inside the page's [kmin, kmax] box can reach,
//     s_j = max_g RN32( sum_c max(q_gc * kmax_jc, q_gc * kmin_jc) )
//         = max_g RN32( q_g+ . kmax_j + q_g- . kmin_j ),
// the query-aware block bound of the Quest row in the sparse-method table of
// the long-context survey (xllm-io.github.io). Products of two bf16 values are
// exact in fp64 and the 128-term sum is accumulated in fp64, so the fp32
// result is the correctly rounded exact sum except in vanishingly rare
// double-rounding cases -- independent of the reduction tree.
//
// Top-k keeps the first k pages in (score descending, page id ascending)
// order by an exact bucket select on unique 64-bit keys
//     key = order(score) << 32 | (0xFFFFFFFF - page id),
// then writes the kept ids in ascending order.
#include "spa_internal.h"

namespace spa {
namespace {

__device__ __forceinline__ int32_t clamp_len(const BatchArgs& bt, int32_t b, int32_t P) {
  int32_t L = bt.lens[b];
  int32_t cap = bt.max_pp * P;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- scoring
//
// A group of LPP lanes scores NP pages; each lane owns CPL = 128 / LPP
// channels of every page, so its q+ / q- values stay in registers (fp64) and
// its summary loads are contiguous. The V = NP * G partial sums of a group
// are reduce-scattered over the group's lanes (R = LPP / V lanes end up
// sharing each total), rounded to fp32 and max-reduced over the query group.
template <int G>
struct ScoreShape {
  static constexpr int LPP = G <= 4 ? 16 : 4 * G;   // lanes per page
  static constexpr int CPL = kHeadDim / LPP;        // channels per lane
  static constexpr int NP = 4;                      // pages per group per pass
  static constexpr int V = NP * G;                  // partial sums per lane
  static constexpr int R = LPP / V;                 // lanes holding each total
  static constexpr int GPW = 64 / LPP;              // groups per wave
  static constexpr int GPB = 4 * GPW;               // groups per 256-thread block
  static constexpr int PAGES = GPB * NP;            // pages per block
};

template <int CPL>
__device__ __forceinline__ void load_chunk(const uint16_t* p, double (&out)[CPL]) {
  if constexpr (CPL == 8) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x); out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
    out[4] = bf16_lo(w.z); out[5] = bf16_hi(w.z); out[6] = bf16_lo(w.w); out[7] = bf16_hi(w.w);
  } else if constexpr (CPL == 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x); out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    out[0] = bf16_lo(w); out[1] = bf16_hi(w);
  }
}

template <int G>
__global__ void __launch_bounds__(256) score_kernel(PoolArgs pl, BatchArgs bt, HeadList dyn,
                                                    const uint16_t* __restrict__ q,
                                                    float* __restrict__ scores, int32_t n_max) {
  using S = ScoreShape<G>;
  const int32_t b = blockIdx.y / dyn.n, h = dyn.id[blockIdx.y % dyn.n];
  const int32_t L = clamp_len(bt, b, pl.P);
  const int32_t n = (L + pl.p - 1) / pl.p;
  const int32_t base = blockIdx.x * S::PAGES;
  if (base >= n) return;

  const int lane = threadIdx.x & 63;
  const int sub = lane % S::LPP;                          // position inside the group
  const int group = (threadIdx.x >> 6) * S::GPW + lane / S::LPP;
  const int c0 = sub * S::CPL;

  // q+ and q- of this lane's channels, fp64 (exact for bf16)
  double qp[G][S::CPL], qn[G][S::CPL];
  const int32_t hq = pl.hkv * G;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    double qv[S::CPL];
    load_chunk<S::CPL>(q + ((int64_t)b * hq + h * G + g) * kHeadDim + c0, qv);
#pragma unroll
    for (int i = 0; i < S::CPL; ++i) {
      qp[g][i] = qv[i] > 0.0 ? qv[i] : 0.0;
      qn[g][i] = qv[i] < 0.0 ? qv[i] : 0.0;
    }
  }

  double v[S::V];                                         // [page slot][query]
#pragma unroll
  for (int pp = 0; pp < S::NP; ++pp) {
    const int32_t j = base + pp * S::GPB + group;
    double kmin[S::CPL], kmax[S::CPL];
    bool ok = j < n;
    int32_t phys = 0;
    if (ok) {
      phys = bt.pt[(int64_t)b * bt.max_pp + j / pl.r];
      ok = phys >= 0 && phys < pl.N;
    }
    if (ok) {
      const uint16_t* s = pl.summ + ((((int64_t)phys * pl.hkv + h) * pl.r + j % pl.r) * 2) * kHeadDim + c0;
      load_chunk<S::CPL>(s, kmin);
      load_chunk<S::CPL>(s + kHeadDim, kmax);
    } else {
#pragma unroll
      for (int i = 0; i < S::CPL; ++i) { kmin[i] = 0.0; kmax[i] = 0.0; }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      double acc = 0.0;
#pragma unroll
      for (int i = 0; i < S::CPL; ++i) {
        acc = fma(qp[g][i], kmax[i], acc);
        acc = fma(qn[g][i], kmin[i], acc);
      }
      v[pp * G + g] = acc;
    }
  }

  // reduce-scatter over the high lane bits of the group, then sum over the
  // R lanes that share a total
#pragma unroll
  for (int m = S::LPP / 2; m >= 1; m /= 2) {
    if (m >= S::R) {
      const bool upper = (sub & m) != 0;
      const int half = m / S::R;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const double send = upper ? v[i] : v[i + half];
        const double keep = upper ? v[i + half] : v[i];
        v[i] = keep + __shfl_xor(send, m, 64);
      }
    } else {
      v[0] += __shfl_xor(v[0], m, 64);
    }
  }
  // lane `sub` now holds the total of index sub / R = page_slot * G + query
  float s = (float)v[0];
  s = s == 0.0f ? 0.0f : s;                               // one zero: +0
#pragma unroll
  for (int m = 1; m < G; m *= 2) s = fmaxf(s, __shfl_xor(s, m * S::R, 64));
  const int idx = sub / S::R;
  const int pp = idx / G;
  const int32_t j = base + pp * S::GPB + group;
  if (sub % (S::R * G) == 0 && j < n) {
    bool ok = true;
    const int32_t phys = bt.pt[(int64_t)b * bt.max_pp + j / pl.r];
    ok = phys >= 0 && phys < pl.N;
    scores[((int64_t)b * pl.hkv + h) * n_max + j] = ok ? s : -INFINITY;
  }
}

// ------------------------------------------------------------------ top-k

constexpr int kTopkThreads = 1024;
constexpr int kBins = 1024;

__device__ __forceinline__ uint64_t page_key(const float* s, int32_t j) {
  const uint32_t u = __float_as_uint(s[j]);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

// Inclusive sum over the block of one value per thread; every thread gets its
// own inclusive prefix and `total`.
__device__ int32_t block_inclusive_scan(int32_t x, int32_t* sh_wave, int32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const int32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) sh_wave[wave] = x;
  __syncthreads();
  int32_t before = 0, all = 0;
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    const int32_t t = sh_wave[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();
  total = all;
  return x + before;
}

__global__ void __launch_bounds__(kTopkThreads) topk_kernel(BatchArgs bt, int32_t p, int32_t P,
                                                            int32_t hkv, HeadList dyn,
                                                            const float* __restrict__ scores,
                                                            int32_t n_max,
                                                            const int32_t* __restrict__ budget,
                                                            int32_t k_max, int32_t* sel_pages,
                                                            int32_t* sel_count, int32_t* sel_len) {
  __shared__ int32_t hist[kBins];
  __shared__ int32_t sh_wave[kTopkThreads / 64];
  __shared__ uint64_t sh_min[kTopkThreads / 64], sh_max[kTopkThreads / 64];
  __shared__ int32_t sh_pick[2];

  const int32_t b = blockIdx.x / dyn.n, h = dyn.id[blockIdx.x % dyn.n];
  const int32_t L = clamp_len(bt, b, P);
  const int32_t n = (L + p - 1) / p;
  int32_t k = budget[b] / p;
  k = k < 1 ? 1 : k;
  k = k > n ? n : k;
  k = k > k_max ? k_max : k;
  const float* s = scores + ((int64_t)b * hkv + h) * n_max;
  const int tid = threadIdx.x;
  const int32_t per = (n + kTopkThreads - 1) / kTopkThreads;   // <= kMaxPerThread
  const int32_t first = tid * per;
  const int32_t mine = max(0, min(per, n - first));

  uint64_t cand = mine >= 64 ? ~0ull : ((1ull << mine) - 1);
  uint64_t sel = 0;
  int32_t need = k;

  for (int round = 0; round < 16 && need > 0; ++round) {
    // candidate count and key range
    int32_t total;
    block_inclusive_scan(__popcll(cand), sh_wave, total);
    if (total <= need) { sel |= cand; cand = 0; break; }
    uint64_t lo = ~0ull, hi = 0;
    for (int32_t e = 0; e < mine; ++e)
      if (cand >> e & 1) {
        const uint64_t key = page_key(s, first + e);
        lo = key < lo ? key : lo;
        hi = key > hi ? key : hi;
      }
    for (int d = 32; d >= 1; d /= 2) {
      const uint64_t l2 = __shfl_xor(lo, d, 64), h2 = __shfl_xor(hi, d, 64);
      lo = l2 < lo ? l2 : lo;
      hi = h2 > hi ? h2 : hi;
    }
    if ((tid & 63) == 0) { sh_min[tid >> 6] = lo; sh_max[tid >> 6] = hi; }
    hist[tid] = 0;
    __syncthreads();
    lo = ~0ull;
    hi = 0;
    for (int w = 0; w < kTopkThreads / 64; ++w) {
      lo = sh_min[w] < lo ? sh_min[w] : lo;
      hi = sh_max[w] > hi ? sh_max[w] : hi;
    }
    const uint64_t span = hi - lo;
    const int bits = span == 0 ? 0 : 64 - __clzll((long long)span);
    const int shift = bits > 10 ? bits - 10 : 0;               // (span >> shift) < kBins
    for (int32_t e = 0; e < mine; ++e)
      if (cand >> e & 1) atomicAdd(&hist[(page_key(s, first + e) - lo) >> shift], 1);
    __syncthreads();
    // bins in descending order: thread t looks at bin kBins-1-t
    const int32_t cnt = hist[kBins - 1 - tid];
    int32_t tot2;
    const int32_t incl = block_inclusive_scan(cnt, sh_wave, tot2);
    if (incl - cnt < need && incl >= need) { sh_pick[0] = kBins - 1 - tid; sh_pick[1] = incl - cnt; }
    __syncthreads();
    const int32_t pick = sh_pick[0], above = sh_pick[1];
    for (int32_t e = 0; e < mine; ++e)
      if (cand >> e & 1) {
        const int32_t bin = (int32_t)((page_key(s, first + e) - lo) >> shift);
        if (bin > pick) { sel |= 1ull << e; cand &= ~(1ull << e); }
        else if (bin < pick) cand &= ~(1ull << e);
      }
    need -= above;
    __syncthreads();
  }

  // compaction in id order
  int32_t total;
  const int32_t cnt = __popcll(sel);
  const int32_t at = block_inclusive_scan(cnt, sh_wave, total) - cnt;
  int32_t* out = sel_pages + ((int64_t)b * hkv + h) * k_max;
  int32_t w = at;
  for (int32_t e = 0; e < mine; ++e)
    if (sel >> e & 1) out[w++] = first + e;
  if (tid == 0) {
    sel_count[(int64_t)b * hkv + h] = total;
    sel_len[b] = L;
  }
}

template <int G>
hipError_t launch_score_g(const PoolArgs& pool, const BatchArgs& batch, const HeadList& dyn,
                          const uint16_t* q, float* scores, int32_t n_max, hipStream_t s) {
  using S = ScoreShape<G>;
  dim3 grid((n_max + S::PAGES - 1) / S::PAGES, batch.B * dyn.n);
  hipLaunchKernelGGL(score_kernel<G>, grid, dim3(256), 0, s, pool, batch, dyn, q, scores, n_max);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const PoolArgs& pool, const BatchArgs& batch, const HeadList& dyn,
                         int32_t G, const uint16_t* q, const int32_t* budget, int32_t k_max,
                         int32_t* sel_pages, int32_t* sel_count, int32_t* sel_len, float* scores,
                         int32_t n_max, hipStream_t s) {
  if (batch.B == 0 || dyn.n == 0) return hipSuccess;
  hipError_t e;
  switch (G) {
    case 1: e = launch_score_g<1>(pool, batch, dyn, q, scores, n_max, s); break;
    case 2: e = launch_score_g<2>(pool, batch, dyn, q, scores, n_max, s); break;
    case 4: e = launch_score_g<4>(pool, batch, dyn, q, scores, n_max, s); break;
    case 8: e = launch_score_g<8>(pool, batch, dyn, q, scores, n_max, s); break;
    case 16: e = launch_score_g<16>(pool, batch, dyn, q, scores, n_max, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_kernel, dim3(batch.B * dyn.n), dim3(kTopkThreads), 0, s, batch, pool.p,
                     pool.P, pool.hkv, dyn, scores, n_max, budget, k_max, sel_pages, sel_count,
                     sel_len);
  return hipGetLastError();
}

}  // namespace spa
