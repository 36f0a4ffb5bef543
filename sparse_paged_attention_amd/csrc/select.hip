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
#include "pool_rows.h"

namespace spa {
namespace {


__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- scoring
//
// One wave scores a range of consecutive logical pages of one (sequence,
// dynamic head). Inside the wave, a group of LPP lanes scores NP pages at a
// time; each lane owns CPL = 128 / LPP channels of every page, so its q+ / q-
// values stay in registers (fp64) and its summary loads are contiguous. The
// V = NP * G partial sums of a group are reduce-scattered over the group's
// lanes (R = LPP / V lanes end up sharing each total), rounded to fp32 and
// max-reduced over the query group. The pool offset of each page of the
// range's summary is computed once into LDS; summary loads run one pass ahead
// of the arithmetic and are issued unconditionally (an invalid page reads
// page 0 and is masked).
// Exchange with the partner lane of butterfly level M (M < 16: inside each
// 16-lane row). DPP pairings stand in for lane ^ M: row_mirror (i <-> 15 - i)
// for M = 8, row_half_mirror (i <-> 7 - i in each half row) for M = 4,
// quad_perm for M = 2, 1. Each partner differs from the lane in bit M and in
// no higher bit, which is all a reduce-scatter over the bits M, M/2, ... 1
// needs: the halves kept and the lane that ends with each total are those of
// lane ^ M. The moves need no LDS round trip (the score kernel runs one wave
// per SIMD, so such latency is not hidden).
template <int M>
__device__ __forceinline__ uint32_t xchg32(uint32_t x) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M >= 16, "butterfly level");
  if constexpr (M >= 16) {
    return (uint32_t)__shfl_xor((int)x, M, 64);
  } else {
    constexpr int ctrl = M == 8 ? 0x140 : M == 4 ? 0x141 : M == 2 ? 0x4E : 0xB1;
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, ctrl, 0xF, 0xF, false);
  }
}
template <int M>
__device__ __forceinline__ double xchg(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint64_t lo = xchg32<M>((uint32_t)u), hi = xchg32<M>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, lo | (hi << 32));
}
template <int M>
__device__ __forceinline__ float xchg(float x) {
  return __uint_as_float(xchg32<M>(__float_as_uint(x)));
}

template <int G_>
struct ScoreShape {
  static constexpr int G = G_;
  // lanes per page: 32 for G <= 4 (4 channels per lane: the lane's q+ / q-
  // in fp64 take 64 registers, and the kernel fits three waves per SIMD; with
  // 16 lanes per page it needed 282 registers and ran one wave per SIMD)
  static constexpr int LPP = G <= 4 ? 32 : 4 * G;
  static constexpr int CPL = kHeadDim / LPP;        // channels per lane
  static constexpr int NP = 4;                      // pages per group per pass
  static constexpr int V = NP * G;                  // partial sums per lane
  static constexpr int R = LPP / V;                 // lanes holding each total
  static constexpr int GPW = 64 / LPP;              // groups per wave
  static constexpr int PASS = GPW * NP;             // pages per pass
  // most passes per wave: for G <= 4 (three waves per SIMD) 6, so that a
  // 128K row's ranges (2736 waves for 16 heads) are still all resident at
  // once and each wave's chain of dependent load rounds is shorter (20.3
  // against 21.2 us for 8 passes at the 128K benchmark shape; 7 passes: 21.0
  // us). Launches with fewer pages take fewer passes per wave (launch_score_g).
  static constexpr int PASSES = G <= 4 ? 6 : 8;
  static constexpr int RING = 2;                    // passes in flight
  // waves a launch can keep resident with room to spare (three per SIMD for
  // G <= 4, one or two above)
  static constexpr int WAVES = G <= 4 ? 2048 : 1024;
  // the last range of a head takes up to one pass more, so that a length just
  // past a multiple of the range needs no extra wave (which would wait for a
  // free slot until every other wave of the launch has finished); not for
  // G > 4, whose registers the extra pass would push past two waves per SIMD
  static constexpr int XPASS = G <= 4 ? 1 : 0;
  static constexpr int MAXP = PASSES + XPASS;
  static constexpr int OFFS = PASS * MAXP;          // pages of the longest range
};

template <int CPL>
struct Raw {
  uint32_t w[CPL / 2];
};

template <int CPL>
__device__ __forceinline__ void load_raw(const uint16_t* p, Raw<CPL>& r) {
  if constexpr (CPL == 8) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    r.w[0] = w.x; r.w[1] = w.y; r.w[2] = w.z; r.w[3] = w.w;
  } else if constexpr (CPL == 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    r.w[0] = w.x; r.w[1] = w.y;
  } else {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

template <int CPL>
__device__ __forceinline__ void widen(const Raw<CPL>& r, double (&out)[CPL]) {
#pragma unroll
  for (int i = 0; i < CPL / 2; ++i) {
    out[2 * i] = bf16_lo(r.w[i]);
    out[2 * i + 1] = bf16_hi(r.w[i]);
  }
}

// The summary of the page receiving a token appended in the same launch, as
// the append leaves it: the channel-wise min / max of the stored summary and
// the new key (on fp8 pages the key as quantized, rounded outward: kn_lo down,
// kn_hi up; on bf16 pages both are the key), or the new key alone when it
// opens the page. Taking min / max with the new key again changes nothing, so
// the stored record may be read before or after the append wave rewrites it.
template <int CPL>
__device__ __forceinline__ void merge_new_key(Raw<CPL>& mn, Raw<CPL>& mx, const Raw<CPL>& kn_lo,
                                              const Raw<CPL>& kn_hi, bool opens) {
#pragma unroll
  for (int w = 0; w < CPL / 2; ++w) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint16_t a = (uint16_t)(mn.w[w] >> (16 * half)), c = (uint16_t)(mx.w[w] >> (16 * half));
      const uint16_t kl = (uint16_t)(kn_lo.w[w] >> (16 * half)), kh = (uint16_t)(kn_hi.w[w] >> (16 * half));
      const uint32_t ka = order_key(a), kc = order_key(c);
      const uint16_t l = opens ? kl : from_key(min(ka, order_key(kl)));
      const uint16_t u = opens ? kh : from_key(max(kc, order_key(kh)));
      lo |= (uint32_t)l << (16 * half);
      hi |= (uint32_t)u << (16 * half);
    }
    mn.w[w] = lo;
    mx.w[w] = hi;
  }
}

// The exchange used by the score reduction: DPP moves, except for groups of a
// whole wave (G = 16), whose kernel has no register room for them.
template <class S, int M, class T>
__device__ __forceinline__ T exch(T x) {
  if constexpr (S::LPP >= 64) return __shfl_xor(x, M, 64);
  else return xchg<M>(x);
}

// One butterfly level M of the reduce-scatter of the V partial sums over the
// LPP lanes of a group (levels M >= R halve the values kept; below R the R
// lanes sharing a total add it up), then the next level.
template <class S, int M>
__device__ __forceinline__ void reduce_level(double (&v)[S::V], int sub) {
  if constexpr (M >= 1) {
    if constexpr (M >= S::R) {
      const bool upper = (sub & M) != 0;
      constexpr int half = M / S::R;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const double send = upper ? v[i] : v[i + half];
        const double keep = upper ? v[i + half] : v[i];
        v[i] = keep + exch<S, M>(send);
      }
    } else {
      v[0] += exch<S, M>(v[0]);
    }
    reduce_level<S, M / 2>(v, sub);
  }
}

// Max over the G query totals of a page slot (lanes M * R apart).
template <class S, int M>
__device__ __forceinline__ void max_over_group(float& sc) {
  if constexpr (M < S::G) {
    sc = fmaxf(sc, exch<S, M * S::R>(sc));
    max_over_group<S, M * 2>(sc);
  }
}

// FRESH: the step's token is appended in this launch (k_new / v_new given):
// B * H_kv extra work-groups in rows past the heads' rows write it into the
// pool and rebuild its page summary, and the waves scoring that page use the
// summary with the new key merged in.
template <int G, bool FRESH>
__global__ void __launch_bounds__(64) score_kernel(PoolArgs pl, BatchArgs bt, HeadList dyn,
                                                   const uint16_t* __restrict__ q,
                                                   float* __restrict__ scores, int32_t n_max,
                                                   int32_t passes, int32_t gq,
                                                   const uint32_t* __restrict__ k_new,
                                                   const uint16_t* __restrict__ v_new) {
  // G: the group size the kernel is built for; gq <= G the heads of the
  // caller's group (query columns g >= gq repeat query gq - 1: a page's score
  // is the maximum over the group, which a repeated query leaves unchanged)
  using S = ScoreShape<G>;
  if (FRESH && (int32_t)blockIdx.y >= bt.B * dyn.n) {
    const int32_t w = ((int32_t)blockIdx.y - bt.B * dyn.n) * (int32_t)gridDim.x + (int32_t)blockIdx.x;
    if (w >= bt.B * pl.hkv) return;
    const int32_t ab = w / pl.hkv, ah = w - ab * pl.hkv;
    bool is_dyn = false;
    for (int32_t d = 0; d < dyn.n; ++d) is_dyn |= dyn.id[d] == ah;
    const int32_t hsl_a = head_slot(pl, ah, dyn_rank(dyn, ah), is_dyn);
    if (pl.q8)
      append_token_q8(pl, bt, ab, ah, hsl_a, k_new, reinterpret_cast<const uint32_t*>(v_new), is_dyn,
                      bt.ring != nullptr && !is_dyn);
    else
      append_token(pl, bt, ab, ah, hsl_a, k_new, v_new, is_dyn, bt.ring != nullptr && !is_dyn);
    return;
  }
  static_assert(S::OFFS <= 192, "three page offsets per lane");
  __shared__ uint32_t offs[S::OFFS];
  const int32_t b = blockIdx.y / dyn.n, h = dyn.id[blockIdx.y % dyn.n];
  const int32_t hsl = head_slot(pl, h, blockIdx.y % dyn.n, true);   // (the list is in ascending head order)
  const int32_t L = clamp_len(bt, b, pl.P);
  const int32_t n = (L + pl.p - 1) / pl.p;
  const int32_t base = blockIdx.x * passes * S::PASS;    // a range of `passes` passes
  if (base >= n) return;

  const int lane = threadIdx.x & 63;
  const int sub = lane % S::LPP;                          // position inside the group
  const int group = lane / S::LPP;
  const int c0 = sub * S::CPL;

  // summary record (512 B) of every page of the range through the page
  // table, or ~0 for pages past the length or unmapped
  const int32_t* pt_row = bt.pt + (int64_t)b * bt.max_pp;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int32_t i = lane + 64 * k, j = base + i;
    if (i < S::OFFS) {
      const int32_t phys = pt_row[min(j / pl.r, bt.max_pp - 1)];
      const bool ok = j < n && phys >= 0 && phys < pl.N;
      offs[i] = ok ? (uint32_t)(((int64_t)phys * pl.hs + hsl) * pl.r + j % pl.r) : ~0u;
    }
  }

  // q+ and q- of this lane's channels, fp64 (exact for bf16)
  double qp[G][S::CPL], qn[G][S::CPL];
  const int32_t hq = pl.hkv * gq;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    Raw<S::CPL> rq;
    load_raw<S::CPL>(q + ((int64_t)b * hq + h * gq + min(g, gq - 1)) * kHeadDim + c0, rq);
    double qv[S::CPL];
    widen<S::CPL>(rq, qv);
#pragma unroll
    for (int i = 0; i < S::CPL; ++i) {
      qp[g][i] = qv[i] > 0.0 ? qv[i] : 0.0;
      qn[g][i] = qv[i] < 0.0 ? qv[i] : 0.0;
    }
  }
  // where the step's token lands (its key is taken below, by the one wave
  // whose range holds that page, once the first summary loads are out)
  Raw<S::CPL> kn = {}, kn_hi = {};
  const int32_t j_new = FRESH && L >= 1 ? (L - 1) / pl.p : -1;
  const bool opens = FRESH && L >= 1 && (L - 1) % pl.p == 0;
  __syncthreads();

  // summary location of page slot pp of pass it (page 0 of the pool if invalid)
  auto locate = [&](int it, int pp, bool& ok) -> const uint16_t* {
    const uint32_t o = offs[it * S::PASS + pp * S::GPW + group];
    ok = o != ~0u;
    return pl.summ + (uint64_t)(ok ? o : 0u) * (2 * kHeadDim) + c0;
  };

  // one pass worth of loaded summaries
  struct Pass {
    Raw<S::CPL> mn[S::NP], mx[S::NP];
    bool ok[S::NP];
  };
  auto issue = [&](int it, Pass& ps) {
#pragma unroll
    for (int pp = 0; pp < S::NP; ++pp) {
      const uint16_t* sp = locate(it, pp, ps.ok[pp]);
      load_raw<S::CPL>(sp, ps.mn[pp]);
      load_raw<S::CPL>(sp + kHeadDim, ps.mx[pp]);
    }
  };
  float* out_row = scores + ((int64_t)b * pl.hkv + h) * n_max;
  auto compute = [&](int it, Pass& ps) {
    if (FRESH && j_new >= base + it * S::PASS && j_new < base + (it + 1) * S::PASS) {
#pragma unroll
      for (int pp = 0; pp < S::NP; ++pp)
        if (base + it * S::PASS + pp * S::GPW + group == j_new)
          merge_new_key<S::CPL>(ps.mn[pp], ps.mx[pp], kn, kn_hi, opens);
    }
    double v[S::V];                                       // [page slot][query]
#pragma unroll
    for (int pp = 0; pp < S::NP; ++pp) {
      double kmin[S::CPL], kmax[S::CPL];
      widen<S::CPL>(ps.mn[pp], kmin);
      widen<S::CPL>(ps.mx[pp], kmax);
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
    reduce_level<S, S::LPP / 2>(v, sub);
    // lane `sub` now holds the total of index sub / R = page_slot * G + query
    float sc = (float)v[0];
    sc = sc == 0.0f ? 0.0f : sc;                          // one zero: +0
    max_over_group<S, 1>(sc);
    const int pp = (sub / S::R) / G;
    bool ok = false;
#pragma unroll
    for (int k = 0; k < S::NP; ++k) ok = k == pp ? ps.ok[k] : ok;
    const int32_t j = base + it * S::PASS + pp * S::GPW + group;
    if (sub % (S::R * G) == 0 && j < n) out_row[j] = ok ? sc : -INFINITY;
  };

  // a ring of S::RING passes in flight: the loads of pass it + 1 run under
  // the arithmetic of pass it (fully unrolled, so the ring is never indexed
  // at run time; deeper rings measured slower)
  // Passes past the head's last page are skipped (wave-uniform): the last
  // range of a head is often nearly empty.
  const int32_t cap = blockIdx.x + 1 == gridDim.x ? passes + S::XPASS : passes;
  const int32_t live = min(cap, (n - base + S::PASS - 1) / S::PASS);
  Pass ring[S::RING];
#pragma unroll
  for (int it = 0; it < S::RING; ++it)
    if (it < live) issue(it, ring[it]);
  // the new key's channels of this lane (on fp8 pages as the append
  // quantizes it, rounded outward), for the wave whose range holds its page
  if (FRESH && j_new >= base && j_new < base + live * S::PASS) {   // wave-uniform
    load_raw<S::CPL>(reinterpret_cast<const uint16_t*>(k_new) + ((int64_t)b * pl.hkv + h) * kHeadDim + c0, kn);
    kn_hi = kn;
    if (pl.q8) {          // the key as the append quantizes it (the group's lanes hold the whole row), rounded outward
      float x[S::CPL];
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < S::CPL / 2; ++i) {
        x[2 * i] = bf16_lo(kn.w[i]);
        x[2 * i + 1] = bf16_hi(kn.w[i]);
        amax = fmaxf(amax, fmaxf(fabsf(x[2 * i]), fabsf(x[2 * i + 1])));
      }
#pragma unroll
      for (int o = 1; o < S::LPP; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      const float scale = amax / 448.f;
#pragma unroll
      for (int i = 0; i < S::CPL / 2; ++i) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t code = scale == 0.f ? 0u : e4m3_code(x[2 * i + e] / scale);
          const double v = (double)e4m3_value(code) * (double)scale;
          lo |= bf16_down(v) << (16 * e);
          hi |= bf16_up(v) << (16 * e);
        }
        kn.w[i] = lo;
        kn_hi.w[i] = hi;
      }
    }
  }
#pragma unroll
  for (int it = 0; it < S::PASSES; ++it) {
    if (it >= live) break;
    compute(it, ring[it % S::RING]);
    if (it + S::RING < live) issue(it + S::RING, ring[it % S::RING]);
  }
  // the extra pass of a head's last range when it follows S::PASSES passes
  // (issued by the loop above; after fewer passes the loop computes it)
  if constexpr (S::XPASS > 0)
    if (live > S::PASSES) compute(S::PASSES, ring[S::PASSES % S::RING]);
}

// ------------------------------------------------------------------ top-k
//
// One 1024-thread block per (sequence, dynamic head). Element e of thread t is
// page e * 1024 + t (coalesced loads), held in a register as the 32-bit
// order-preserving image of its fp32 score. Rounds of a 4096-bin histogram
// over the remaining candidates' key range find the bin holding the k-th
// largest key: keys above it are kept, keys below dropped, the bin's keys stay
// candidates. Once at most kMaxCand candidates are left they are ranked
// exactly by (key descending, page id ascending); if more share one key, the
// ones with the lowest page ids are kept (ties go to the lower page id). Kept
// ids are written in ascending order: a block-wide prefix sum over
// per-(element, wave) counts gives each its position; the ids are also staged
// in LDS so the physical-page look-ups go out as one coalesced round.

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kHistBins = 4096;                     // 4 per thread
constexpr int kMaxCand = 128;
constexpr int kOutStage = 4096;                     // kept ids staged in LDS

__device__ __forceinline__ uint32_t order32(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide reductions on the VALU: DPP within each 16-lane row (swap
// neighbours, pairs, then mirror halves and rows), then the cross-row lane
// swaps; every lane ends with the result.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));   // row_mirror
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(a[0], a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(c[0], c[1]);
}

// Sum over the 8-lane group holding this lane (lanes 8m .. 8m + 7).
__device__ __forceinline__ int32_t group8_sum(int32_t v) {
  v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
  return v;
}

// Exclusive prefix over the block (thread order) of one value per thread.
// The caller puts a barrier between this call's reads of sh_wave and the next
// call (the pick that follows each use does).
__device__ int32_t block_exclusive_scan(int32_t x, int32_t* sh_wave, int32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t incl = x;
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const int32_t y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) {
    // the slot's address formed here: left to itself the compiler computes it
    // before the rounds and, with 16 scores per thread, parks it in scratch
    int32_t w = wave;
    asm volatile("" : "+v"(w));
    sh_wave[w] = incl;
  }
  __syncthreads();
  int32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int32_t t = sh_wave[w];
    before += w < wave ? t : 0;
    all += t;
  }
  total = all;
  return incl - x + before;
}

// For a per-thread element mask: the position of every set element among all
// set elements in page-id order (ids e * kTopkThreads + thread); returns the
// number of set elements. The E * waves per-(element, wave) counts are
// scanned by wave 0 alone (a few per lane), between two barriers; `again`:
// the block calls it once more later (block-uniform).
template <int E>
__device__ int32_t id_order_ranks(uint32_t mask, int32_t (&rank)[E], int32_t* table, int32_t* sh_total,
                                  bool again) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t ball = __ballot((mask >> e) & 1);
    if (lane == 0) table[e * kTopkWaves + wave] = __popcll(ball);
  }
  __syncthreads();
  constexpr int N = E * kTopkWaves, PL = (N + 63) / 64;   // entries, entries per lane of wave 0
  if (wave == 0) {
    int32_t sum = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int idx = lane * PL + i;
      sum += idx < N ? table[idx] : 0;
    }
    int32_t incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
      const int32_t y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    int32_t run = incl - sum;
#pragma unroll
    for (int i = 0; i < PL; ++i) {                  // (the lane's entries read again: fewer live registers)
      const int idx = lane * PL + i;
      if (idx < N) {
        const int32_t c = table[idx];
        table[idx] = run;
        run += c;
      }
    }
    if (lane == 63) *sh_total = incl;
  }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t ball = __ballot((mask >> e) & 1);
    rank[e] = table[e * kTopkWaves + wave] + __popcll(ball & below);
  }
  const int32_t total = *sh_total;
  if (again) __syncthreads();                       // table and sh_total free for the next call
  return total;
}

template <int E>   // elements per thread: n_max <= E * kTopkThreads
__global__ void __launch_bounds__(kTopkThreads) topk_kernel(BatchArgs bt, int32_t p, int32_t P,
                                                            int32_t hkv, HeadList dyn,
                                                            const float* __restrict__ scores,
                                                            int32_t n_max,
                                                            const int32_t* __restrict__ budget,
                                                            int32_t k_max, int32_t* sel_pages,
                                                            int32_t* sel_count, int32_t* sel_len,
                                                            int32_t* sel_phys) {
  static_assert(E <= 32, "32-bit element masks");
  constexpr int BINS = kHistBins, PER = BINS / kTopkThreads;
  __shared__ int32_t hist[BINS];
  __shared__ int32_t sh_wave[kTopkWaves];
  __shared__ uint32_t sh_min[kTopkWaves], sh_max[kTopkWaves];
  __shared__ int32_t sh_cnt[kTopkWaves];
  __shared__ int32_t sh_pick[3];
  __shared__ int32_t sh_nc, sh_total;
  __shared__ uint64_t cand_key[kMaxCand];
  __shared__ uint32_t sel_bits[kTopkThreads];
  __shared__ int32_t table[E * kTopkWaves];
  __shared__ int32_t staged[kOutStage];

  const int32_t b = blockIdx.x / dyn.n, h = dyn.id[blockIdx.x % dyn.n];
  const int32_t L = clamp_len(bt, b, P);
  const int32_t n = (L + p - 1) / p;
  int32_t k = budget[b] / p;
  k = k < 1 ? 1 : k;
  k = k > n ? n : k;
  k = k > k_max ? k_max : k;
  const float* s = scores + ((int64_t)b * hkv + h) * n_max;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  uint32_t ord[E];
  uint32_t cand = 0, sel = 0;                       // bit e: element e
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int32_t j = e * kTopkThreads + tid;
    ord[e] = order32(s[min(j, n_max - 1)]);
    if (j < n) cand |= 1u << e;
  }
  int32_t need = k;
  int32_t rank[E];
  int32_t known = -1;       // candidates left by the previous round's pick (its bin's count)

  for (int round = 0; round < 8 && need > 0; ++round) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0;
    int32_t total = known;
    // when the candidates the last pick left are all kept, or few enough to
    // rank exactly, their key range is not needed (block-uniform)
    if (!(known >= 0 && (known <= need || known <= kMaxCand))) {
      // candidate count and key range; the histogram is cleared meanwhile
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (cand >> e & 1) { lo = min(lo, ord[e]); hi = max(hi, ord[e]); }
      lo = wave_reduce(lo, [](uint32_t x, uint32_t y) { return min(x, y); });
      hi = wave_reduce(hi, [](uint32_t x, uint32_t y) { return max(x, y); });
      const int32_t c = (int32_t)wave_reduce((uint32_t)__popc(cand), [](uint32_t x, uint32_t y) { return x + y; });
      if (lane == 0) { sh_min[wave] = lo; sh_max[wave] = hi; sh_cnt[wave] = c; }
#pragma unroll
      for (int i = 0; i < PER; ++i) hist[tid * PER + i] = 0;
      sel_bits[tid] = 0;                             // (untouched until the exact ranking)
      if (tid == 0) sh_nc = 0;
      __syncthreads();
      lo = 0xFFFFFFFFu;
      hi = 0;
      total = 0;
#pragma unroll
      for (int w = 0; w < kTopkWaves; ++w) { lo = min(lo, sh_min[w]); hi = max(hi, sh_max[w]); total += sh_cnt[w]; }
    }
    if (total <= need) { sel |= cand; cand = 0; break; }
    if (total <= kMaxCand) {
      // exact ranks by (key descending, page id ascending) among the few left
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (cand >> e & 1) {
          const int32_t at = atomicAdd(&sh_nc, 1);
          cand_key[at] = ((uint64_t)ord[e] << 32) | (0xFFFFFFFFu - (uint32_t)(e * kTopkThreads + tid));
        }
      __syncthreads();
      // thread (i, part): how many of candidates part*16 .. +15 outrank
      // candidate i; the 8 parts are summed within the 8-lane group
      const int32_t nc = sh_nc;
      const int32_t i = tid >> 3, part = tid & 7;
      int32_t r = 0;
      if (i < nc) {
        const uint64_t key = cand_key[i];
#pragma unroll
        for (int x = 0; x < kMaxCand / 8; ++x) {
          const int32_t jj = part * (kMaxCand / 8) + x;
          r += jj < nc && cand_key[jj] > key;
        }
      }
      r = group8_sum(r);
      if (part == 0 && i < nc && r < need) {
        const uint32_t id = 0xFFFFFFFFu - (uint32_t)cand_key[i];
        atomicOr(&sel_bits[id % kTopkThreads], 1u << (id / kTopkThreads));
      }
      __syncthreads();
      sel |= sel_bits[tid];
      cand = 0;
      break;
    }
    if (lo == hi) {
      // more than kMaxCand candidates share one key: keep the `need` lowest page ids
      id_order_ranks<E>(cand, rank, table, &sh_total, true);
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((cand >> e & 1) && rank[e] < need) sel |= 1u << e;
      cand = 0;
      break;
    }
    const uint32_t span = hi - lo;
    const int bits = 32 - __clz((int)span);
    const int shift = bits > 12 ? bits - 12 : 0;    // (span >> shift) < BINS
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (cand >> e & 1) atomicAdd(&hist[(ord[e] - lo) >> shift], 1);
    __syncthreads();
    // bins in descending order: thread t owns bins BINS-1-t*PER .. BINS-PER-t*PER
    int32_t cnt[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) { cnt[i] = hist[BINS - 1 - (tid * PER + i)]; sum += cnt[i]; }
    int32_t tot2;
    int32_t run = block_exclusive_scan(sum, sh_wave, tot2);       // keys in higher bins
    int32_t hit = -1, hit_run = 0, hit_cnt = 0;   // the owned bin where the count reaches `need`
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool here = run < need && run + cnt[i] >= need;
      hit = here ? i : hit;
      hit_run = here ? run : hit_run;
      hit_cnt = here ? cnt[i] : hit_cnt;
      run += cnt[i];
    }
    if (hit >= 0) {
      // recomputed here: left to itself the compiler keeps the bin numbers in
      // registers from the start, spills them, and this one thread then waits
      // on a scratch load before the barrier
      int32_t t = tid;
      asm volatile("" : "+v"(t));
      sh_pick[0] = BINS - 1 - (t * PER + hit);
      sh_pick[1] = hit_run;
      sh_pick[2] = hit_cnt;
    }
    __syncthreads();
    const uint32_t pick = (uint32_t)sh_pick[0];
    const int32_t above = sh_pick[1];
    known = sh_pick[2];
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (cand >> e & 1) {
        const uint32_t bin = (ord[e] - lo) >> shift;
        if (bin > pick) { sel |= 1u << e; cand &= ~(1u << e); }
        else if (bin < pick) cand &= ~(1u << e);
      }
    need -= above;
  }

  // kept ids in ascending order
  const int32_t total = id_order_ranks<E>(sel, rank, table, &sh_total, false);
  int32_t* out = sel_pages + ((int64_t)b * hkv + h) * k_max;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((sel >> e) & 1) {
      const int32_t id = e * kTopkThreads + tid;
      out[rank[e]] = id;
      if (rank[e] < kOutStage) staged[rank[e]] = id;
    }
  if (tid == 0) {
    sel_count[(int64_t)b * hkv + h] = total;
    sel_len[b] = L;
  }
  if (sel_phys) {                                 // physical page of each kept page, through the page table
    __syncthreads();
    int32_t* ph = sel_phys + ((int64_t)b * hkv + h) * k_max;
    const int32_t* pt_row = bt.pt + (int64_t)b * bt.max_pp;
    const int32_t r = P / p;
    for (int32_t i = tid; i < min(total, kOutStage); i += kTopkThreads) ph[i] = pt_row[staged[i] / r];
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (((sel >> e) & 1) && rank[e] >= kOutStage) ph[rank[e]] = pt_row[(e * kTopkThreads + tid) / r];
  }
}

template <int G>
hipError_t launch_score_g(const PoolArgs& pool, const BatchArgs& batch, const HeadList& dyn, int32_t gq,
                          const uint16_t* q, float* scores, int32_t n_max, const uint16_t* k_new,
                          const uint16_t* v_new, hipStream_t s) {
  using S = ScoreShape<G>;
  // passes per wave: S::PASSES when the rows fill the GPU, fewer when there
  // are few pages in all (small batches), so that about S::WAVES waves share
  // them and each wave's chain of dependent load rounds is short
  const int64_t pages = (int64_t)batch.B * dyn.n * n_max;
  const int64_t per = (int64_t)S::WAVES * S::PASS;
  const int32_t passes = (int32_t)std::min<int64_t>(S::PASSES, std::max<int64_t>(1, (pages + per - 1) / per));
  // ranges of passes * PASS pages; the last one also takes up to PASS more
  const int32_t range = passes * S::PASS;
  const int32_t ranges = std::max(1, (n_max - S::XPASS * S::PASS + range - 1) / range);
  if (k_new) {          // extra rows for the append waves
    const int32_t rows = (batch.B * pool.hkv + ranges - 1) / ranges;
    hipLaunchKernelGGL((score_kernel<G, true>), dim3(ranges, batch.B * dyn.n + rows), dim3(64), 0, s, pool, batch,
                       dyn, q, scores, n_max, passes, gq, reinterpret_cast<const uint32_t*>(k_new), v_new);
  } else {
    hipLaunchKernelGGL((score_kernel<G, false>), dim3(ranges, batch.B * dyn.n), dim3(64), 0, s, pool, batch, dyn,
                       q, scores, n_max, passes, gq, nullptr, nullptr);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const PoolArgs& pool, const BatchArgs& batch, const HeadList& dyn,
                         int32_t G, const uint16_t* q, const int32_t* budget, int32_t k_max,
                         int32_t* sel_pages, int32_t* sel_count, int32_t* sel_len, int32_t* sel_phys,
                         float* scores, int32_t n_max, const uint16_t* k_new, const uint16_t* v_new,
                         hipStream_t s) {
  if (batch.B == 0) return hipSuccess;
  if (dyn.n == 0) return k_new ? launch_append(pool, batch, k_new, v_new, nullptr, s) : hipSuccess;
  hipError_t e;
  // the scoring kernel built for the next power of two holds the group
  const int32_t gk = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16;
  if (G > 16) return hipErrorInvalidValue;
  if (k_new && gk >= 8) {     // no room in those scoring kernels' registers: append first
    if ((e = launch_append(pool, batch, k_new, v_new, &dyn, s)) != hipSuccess) return e;
    k_new = v_new = nullptr;
  }
  switch (gk) {
    case 1: e = launch_score_g<1>(pool, batch, dyn, G, q, scores, n_max, k_new, v_new, s); break;
    case 2: e = launch_score_g<2>(pool, batch, dyn, G, q, scores, n_max, k_new, v_new, s); break;
    case 4: e = launch_score_g<4>(pool, batch, dyn, G, q, scores, n_max, k_new, v_new, s); break;
    case 8: e = launch_score_g<8>(pool, batch, dyn, G, q, scores, n_max, k_new, v_new, s); break;
    default: e = launch_score_g<16>(pool, batch, dyn, G, q, scores, n_max, k_new, v_new, s); break;
  }
  if (e != hipSuccess) return e;
#define SPA_TOPK(E)                                                                                     \
  hipLaunchKernelGGL(topk_kernel<E>, dim3(batch.B * dyn.n), dim3(kTopkThreads), 0, s, batch, pool.p, pool.P, \
                     pool.hkv, dyn, scores, n_max, budget, k_max, sel_pages, sel_count, sel_len, sel_phys)
  // the fewest scores per thread that hold the row: each phase of the
  // selection costs VALU work per element, on one compute unit per problem
  if (n_max <= 8 * kTopkThreads) SPA_TOPK(8);
  else if (n_max <= 9 * kTopkThreads) SPA_TOPK(9);
  else if (n_max <= 12 * kTopkThreads) SPA_TOPK(12);
  else if (n_max <= 16 * kTopkThreads) SPA_TOPK(16);
  else if (n_max <= 24 * kTopkThreads) SPA_TOPK(24);
  else SPA_TOPK(32);
#undef SPA_TOPK
  return hipGetLastError();
}

}  // namespace spa
