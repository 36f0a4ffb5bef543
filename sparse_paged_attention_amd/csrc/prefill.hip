// Prefill block-sparse attention.
//
// LServe write-up (bqwf.cn), "3.1 预填充阶段优化": during prefill the
// importance of each block of the prompt is estimated from a low-rank
// approximation of the attention logits, Score(Q, K_i) ~ (Q W_q)(K_i W_k)^T /
// sqrt(d) with W_q, W_k projecting d dimensions down to d/8; exact attention
// then runs only on the most important blocks (first the approximate scores
// of all blocks, then the selected blocks); below 32K tokens the dynamic heads
// attend densely. Streaming heads keep the sink and the local window ("2.1").
//
// Three launches:
//   pool_kernel    per (block, KV head, side): the block's mean query over
//                  the KV head's G query heads (side 0) or mean key (side 1),
//                  projected to r = d/8 dimensions, in fp64;
//   select_kernel  per (query block j, dynamic KV head): the score of every
//                  earlier block, RN32((qbar_j W_q).(kbar_i W_k) / sqrt(d)) in
//                  fp64, and the best kb - 1 of them (score descending, block
//                  id ascending) plus block j itself, ascending;
//   attn_kernel    per (query block, KV head, group of up to 4 query heads):
//                  exact causal attention over the block's key blocks (the
//                  selection; every earlier block in dense mode; the sink and
//                  window blocks of streaming heads), online softmax, K and V
//                  of each key block staged once in LDS for all of the
//                  group's heads, S^T = K Q^T and O^T += V^T P^T on
//                  v_mfma_f32_16x16x32_bf16 (P split into bf16 high and low
//                  parts, as in the decode kernel).
#include "psplit.h"
#include "spa_internal.h"

namespace spa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kB = kPrefillBlock;          // 64 tokens per block
constexpr int kR = kHeadDim / 8;           // 16: rank of the projections
constexpr float kScaleLog2 = 0.12751743074602467f;   // log2(e) / sqrt(128)
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kRescaleSlack = 8.f;

__device__ __forceinline__ double bfd(uint32_t w16) { return (double)__uint_as_float(w16 << 16); }

template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* as_scalar(const T* p) {
  return (const __attribute__((address_space(4))) T*)p;
}

// ------------------------------------------------------------ pooling
//
// One wave per (block j, KV head h, side): lane l sums channels 2l and 2l + 1
// over the block's rows (and, for queries, over the G heads) in fp64, divides
// by the row count, then contributes x[2l] W[2l][r] + x[2l+1] W[2l+1][r] to
// each of the r = 16 projections, summed over the wave.
__global__ void __launch_bounds__(64) pool_kernel(PrefillArgs a) {
  const int32_t j = blockIdx.x, h = blockIdx.y, side = blockIdx.z;
  if (!((a.dyn_mask[h >> 5] >> (h & 31)) & 1u)) return;
  const int lane = threadIdx.x;
  const int64_t t0 = (int64_t)j * kB, t1 = min(t0 + kB, a.L);
  const int32_t heads = side == 0 ? a.G : 1;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(side == 0 ? a.q : a.k);
  double s0 = 0.0, s1 = 0.0;
  for (int32_t g = 0; g < heads; ++g) {
    const int64_t head = side == 0 ? (int64_t)h * a.G + g : h;
    const uint32_t* rows = src + (head * a.L) * (kHeadDim / 2) + lane;
    // rows summed in order; the loads of 32 rows go out together
    double u0 = 0.0, u1 = 0.0;
    int64_t t = t0;
    for (; t + 32 <= t1; t += 32) {
      uint32_t w[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) w[i] = rows[(t + i) * (kHeadDim / 2)];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        u0 += bfd(w[i] & 0xFFFFu);
        u1 += bfd(w[i] >> 16);
      }
    }
    for (; t < t1; ++t) {
      const uint32_t w = rows[t * (kHeadDim / 2)];
      u0 += bfd(w & 0xFFFFu);
      u1 += bfd(w >> 16);
    }
    s0 += u0 / (double)(t1 - t0);
    s1 += u1 / (double)(t1 - t0);
  }
  s0 /= (double)heads;
  s1 /= (double)heads;
  const uint16_t* W = side == 0 ? a.wq : a.wk;
  double y[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r)
    y[r] = s0 * bfd(W[(2 * lane) * kR + r]) + s1 * bfd(W[(2 * lane + 1) * kR + r]);
#pragma unroll
  for (int r = 0; r < kR; ++r)
#pragma unroll
    for (int o = 32; o; o >>= 1) y[r] += __shfl_xor(y[r], o, 64);
  double* dst = (side == 0 ? a.qp : a.kp) + ((int64_t)h * a.nb + j) * kR;
  if (lane < kR) {
    double v = y[0];
#pragma unroll
    for (int r = 1; r < kR; ++r) v = lane == r ? y[r] : v;
    dst[lane] = v;
  }
}

// ---------------------------------------------------------- selection

__device__ __forceinline__ uint32_t order32(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide reduction on the VALU (DPP inside each 16-lane row: swap
// neighbours, pairs, then mirror halves and rows; then the cross-row lane
// swaps); every lane ends with the result.
template <class Op>
__device__ __forceinline__ uint32_t wave_all(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));   // row_mirror
  auto x = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(x[0], x[1]);
  auto y = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(y[0], y[1]);
}

__device__ __forceinline__ int32_t wave_sum(int32_t v) {
  return (int32_t)wave_all((uint32_t)v, [](uint32_t p, uint32_t q) { return p + q; });
}

// One wave per (query block j, dynamic KV head h). Lane l holds the scores of
// blocks l, l + 64, ... below j (M slots per lane, the first mv of them in
// use). The k-th largest order key T is found bit by bit from the top (the
// largest T with at least k keys >= T), starting below the leading bits that
// the smallest and the largest key share (T lies between them); keys above T
// are kept, and of those equal to T the ones with the lowest block ids. Kept
// ids go out ascending, then j itself.
template <int M>
__global__ void __launch_bounds__(64) select_kernel(PrefillArgs a) {
  const int32_t j = blockIdx.x, h = blockIdx.y;
  if (!((a.dyn_mask[h >> 5] >> (h & 31)) & 1u)) return;
  const int lane = threadIdx.x;
  int32_t* sel = a.sel + ((int64_t)h * a.nb + j) * a.kb;
  const int32_t k = min(j, a.kb - 1);
  const int32_t mv = (j + 63) >> 6;
  const double* qp = a.qp + ((int64_t)h * a.nb + j) * kR;
  const double* kbase = a.kp + (int64_t)h * a.nb * kR;
  double qv[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) qv[r] = qp[r];
  const double scale = 0.088388347648318440550;   // 1 / sqrt(128)
  uint32_t key[M];
#pragma unroll
  for (int m = 0; m < M; ++m) key[m] = 0;
  // the loads of two slots go out together; a lane past j reads block
  // j - 1 and drops the result. The dot product is a chain of fused
  // multiply-adds in fp64
#pragma unroll
  for (int m = 0; m < M; m += 2) {
    if (m < mv) {
      double kv[2][kR];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const double* kp = kbase + (int64_t)min(lane + 64 * (m + u), j - 1) * kR;
#pragma unroll
        for (int r = 0; r < kR; ++r) kv[u][r] = kp[r];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int32_t i = lane + 64 * (m + u);
        double s = 0.0;
#pragma unroll
        for (int r = 0; r < kR; ++r) s = __builtin_fma(qv[r], kv[u][r], s);
        const float sc = (float)(s * scale);
        if (i < j) {
          key[m + u] = order32(sc);
          if (a.scores) a.scores[((int64_t)h * a.nb + j) * a.nb + i] = sc;
        }
      }
    }
  }
  if (k == j) {                                   // every earlier block is kept
    for (int32_t i = lane; i <= j; i += 64) sel[i] = i;
    if (lane == 0) a.cnt[(int64_t)h * a.nb + j] = j + 1;
    return;
  }
  // the k-th largest key among the j valid ones (order keys of real scores are
  // never 0, so 0 marks the invalid slots); with k = 0 nothing is kept
  uint32_t T = 0xFFFFFFFFu;
  if (k > 0) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      lo = key[m] != 0 ? min(lo, key[m]) : lo;
      hi = max(hi, key[m]);
    }
    lo = wave_all(lo, [](uint32_t p, uint32_t q) { return min(p, q); });
    hi = wave_all(hi, [](uint32_t p, uint32_t q) { return max(p, q); });
    T = hi;
    const uint32_t diff = lo ^ hi;
    if (diff != 0) {
      const int top = 31 - __builtin_clz(diff);
      T = hi & ~((2u << top) - 1u);
      for (int bit = top; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        int32_t c = 0;
#pragma unroll
        for (int m = 0; m < M; ++m) c += key[m] >= cand;     // unused slots hold 0 < cand
        if (wave_sum(c) >= k) T = cand;
      }
    }
  }
  int32_t gt = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) gt += key[m] > T;
  const int32_t need_eq = k - wave_sum(gt);       // keys equal to T still to keep, lowest ids first
  const uint64_t below = (1ull << lane) - 1;
  int32_t eq_seen = 0, kept = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const bool eq = key[m] == T && key[m] != 0;
    const uint64_t eqb = __ballot(eq);
    const bool keep = key[m] > T || (eq && eq_seen + __popcll(eqb & below) < need_eq);
    eq_seen += __popcll(eqb);
    const uint64_t kb = __ballot(keep);
    if (keep) sel[kept + __popcll(kb & below)] = lane + 64 * m;
    kept += __popcll(kb);
  }
  if (lane == 0) {
    sel[k] = j;
    a.cnt[(int64_t)h * a.nb + j] = k + 1;
  }
}

// ---------------------------------------------------------- attention
//
// Work-group: (query block j, KV head h, heads g0 .. g0 + NH - 1 of its group);
// 2 * NH waves, wave w handles query head g0 + w / 2, rows 32 (w % 2) .. +32 of
// the block as two 16-row column tiles of the MFMAs. Per key block, every
// thread stages part of K (row-major, rows padded to 272 bytes) and of V^T
// (channel-major, rows padded to 144 bytes) into one of four LDS block
// buffers. In a V^T row the keys of each 32-key half of the block are
// interleaved in groups of four: keys 4q .. 4q + 3 and 16 + 4q .. 19 + 4q
// (q = 0 .. 3) sit side by side, the eight keys one lane of the P V MFMAs
// takes, so it reads them as one 16-byte piece. Key blocks go in pairs: the
// next pair's global loads are in flight while the current pair is computed,
// one barrier per pair.
constexpr int kKStride = 136;              // bf16 per K row in LDS
constexpr int kVStride = 72;               // bf16 per V^T row in LDS (144 B: 16-byte aligned; 16 rows read as 16-byte pieces fall on distinct banks)
constexpr int kKBytes = kB * kKStride * 2;
constexpr int kVBytes = kHeadDim * kVStride * 2;
constexpr int kBufBytes = kKBytes + kVBytes;

template <int NT>
struct Stage {
  static constexpr int KP = 1024 / NT;   // 16-byte pieces of K per thread
  static constexpr int VU = 512 / NT;    // V units (channel pair x 8 keys) per thread
  uint32_t k[KP][4];                     // (32-bit words: held as 16-byte vectors, the pieces
  uint32_t v[VU][8];                     // went to scratch memory, whose store waited for the loads)
};

// Which key blocks a query block attends: [0, n1) then [w0, j] (the second
// range empty when n1 > j).
struct KeyList {
  int32_t count, n1, w0;
  __device__ __forceinline__ int32_t at(int32_t e, const __attribute__((address_space(4))) int32_t* sel) const {
    if (sel) return sel[e];
    return e < n1 ? e : w0 + (e - n1);
  }
};

template <int NH>
__global__ void __launch_bounds__(NH * 128) attn_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kBufBytes];
  constexpr int NT = NH * 128;                 // threads
  const int32_t j = (int32_t)(gridDim.x - 1 - blockIdx.x);   // longest key lists first
  const int32_t h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t g = blockIdx.z * NH + (w >> 1);
  const int rh = w & 1;
  const int quad = lane >> 4, col = lane & 15;
  const bool dynamic = (a.dyn_mask[h >> 5] >> (h & 31)) & 1u;
  const int64_t L = a.L;

  // key blocks of this query block
  KeyList kl;
  const __attribute__((address_space(4))) int32_t* sel_list = nullptr;
  if (dynamic && !a.dense) {
    kl.count = as_scalar(a.cnt)[(int64_t)h * a.nb + j];
    kl.n1 = kl.w0 = 0;
    sel_list = as_scalar(a.sel) + ((int64_t)h * a.nb + j) * a.kb;
  } else if (dynamic) {
    kl.n1 = j + 1;
    kl.w0 = j + 1;
    kl.count = j + 1;
  } else {
    const int32_t sink_blocks = min((a.sink + kB - 1) / kB, j + 1);
    const int64_t first_win = max((int64_t)0, (int64_t)j * kB + 1 - a.window) / kB;
    kl.n1 = sink_blocks;
    kl.w0 = (int32_t)max((int64_t)sink_blocks, first_win);
    kl.count = sink_blocks + (j + 1 - kl.w0);
  }

  // the query operand of the wave's two column tiles: Q[row][32 quad + 8 i .. +8]
  const int64_t qhead = (int64_t)h * a.G + g;
  bf16x8 qb[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int64_t row = min((int64_t)j * kB + 32 * rh + 16 * qt + col, L - 1);
    const uint4* q4 = reinterpret_cast<const uint4*>(a.q + (qhead * L + row) * kHeadDim + 32 * quad);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = q4[i];
      __builtin_memcpy(&qb[qt][i], &v, 16);
    }
  }

  // staging assignment: K piece p (of 1024 16-byte pieces) = row p / 16, cols
  // 8 (p % 16) .. +8; V unit u (of 512) = channel pair u % 64, keys 8 (u / 64) .. +8
  using St = Stage<NT>;
  // byte offsets of this thread's staged pieces inside a key block
  const uint32_t kcol = 16u * (tid % 16), vcol = 4u * (tid % 64);
  uint32_t koff[St::KP], voff[St::VU];
#pragma unroll
  for (int x = 0; x < St::KP; ++x) koff[x] = (uint32_t)((tid + NT * x) / 16) * 256u + kcol;
#pragma unroll
  for (int x = 0; x < St::VU; ++x) voff[x] = (uint32_t)(8 * ((tid + NT * x) / 64)) * 256u + vcol;
  auto load_block = [&](int32_t kbk, St& st) {
    const int64_t base = (int64_t)kbk * kB;
    const char* kb = reinterpret_cast<const char*>(a.k + ((int64_t)h * L + base) * kHeadDim);
    const char* vb = reinterpret_cast<const char*>(a.v + ((int64_t)h * L + base) * kHeadDim);
    if (base + kB <= L) {                               // block-uniform
#pragma unroll
      for (int x = 0; x < St::KP; ++x) {
        const uint4 kv4 = *reinterpret_cast<const uint4*>(kb + koff[x]);
        st.k[x][0] = kv4.x; st.k[x][1] = kv4.y; st.k[x][2] = kv4.z; st.k[x][3] = kv4.w;
      }
#pragma unroll
      for (int x = 0; x < St::VU; ++x)
#pragma unroll
        for (int u = 0; u < 8; ++u) st.v[x][u] = *reinterpret_cast<const uint32_t*>(vb + voff[x] + 256u * u);
    } else {
      // the prompt's last block: rows past its end repeat its last row (no
      // query attends them)
      asm volatile("");                                 // a real branch: the loads above need no clamp
      const uint32_t last = (uint32_t)(L - 1 - base) * 256u;
#pragma unroll
      for (int x = 0; x < St::KP; ++x) {
        const uint4 kv4 = *reinterpret_cast<const uint4*>(kb + min(koff[x] - kcol, last) + kcol);
        st.k[x][0] = kv4.x; st.k[x][1] = kv4.y; st.k[x][2] = kv4.z; st.k[x][3] = kv4.w;
      }
#pragma unroll
      for (int x = 0; x < St::VU; ++x)
#pragma unroll
        for (int u = 0; u < 8; ++u)
          st.v[x][u] = *reinterpret_cast<const uint32_t*>(vb + min(voff[x] - vcol + 256u * u, last) + vcol);
    }
  };
  auto store_block = [&](int buf, const St& st) {
    uint8_t* kl_ = lds + buf * kBufBytes;
    uint8_t* vl = kl_ + kKBytes;
#pragma unroll
    for (int x = 0; x < St::KP; ++x) {
      const int p = tid + NT * x;
      *reinterpret_cast<uint4*>(kl_ + ((p / 16) * kKStride + 8 * (p % 16)) * 2) = uint4{st.k[x][0], st.k[x][1], st.k[x][2], st.k[x][3]};
    }
#pragma unroll
    for (int x = 0; x < St::VU; ++x) {
      const int un = tid + NT * x;
      const int cp = un % 64, kg = un / 64;
      const uint32_t* v = st.v[x];
      uint4 lo, hi;                 // channel 2cp / 2cp + 1, keys 8kg .. +8: the low / high halves of pairs of words
      lo.x = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);
      lo.y = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);
      lo.z = __builtin_amdgcn_perm(v[5], v[4], 0x05040100u);
      lo.w = __builtin_amdgcn_perm(v[7], v[6], 0x05040100u);
      hi.x = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);
      hi.y = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);
      hi.z = __builtin_amdgcn_perm(v[5], v[4], 0x07060302u);
      hi.w = __builtin_amdgcn_perm(v[7], v[6], 0x07060302u);
      // keys 8kg .. 8kg + 3 and 8kg + 4 .. 8kg + 7 in the interleaved order
      const int c0 = 32 * (kg / 4) + 16 * (kg % 2) + 4 * ((kg % 4) / 2);
      uint8_t* r0 = vl + (2 * cp) * kVStride * 2;
      uint8_t* r1 = vl + (2 * cp + 1) * kVStride * 2;
      *reinterpret_cast<uint2*>(r0 + c0 * 2) = uint2{lo.x, lo.y};
      *reinterpret_cast<uint2*>(r0 + (c0 + 8) * 2) = uint2{lo.z, lo.w};
      *reinterpret_cast<uint2*>(r1 + c0 * 2) = uint2{hi.x, hi.y};
      *reinterpret_cast<uint2*>(r1 + (c0 + 8) * 2) = uint2{hi.z, hi.w};
    }
  };

  // running reference per query column (log2 units) and the value subtracted
  // before exponentiation (0 while the column has no key yet)
  float m_ref[2] = {-INFINITY, -INFINITY}, m_sub[2] = {0.f, 0.f}, l_sum[2] = {0.f, 0.f};
  f32x4 o[2][8];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int c = 0; c < 8; ++c) o[qt][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one key block staged in LDS buffer buf: scores, mask, online softmax, P V
  auto block = [&](int32_t kbk, int buf) {
    const uint8_t* kl_ = lds + buf * kBufBytes;
    const uint8_t* vl = kl_ + kKBytes;

    // S^T = K Q^T: 4 key tiles x 2 query tiles, 4 MFMAs each over d
    f32x4 s[2][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8 ka[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ka[i] = *reinterpret_cast<const bf16x8*>(kl_ + ((16 * t + col) * kKStride + 32 * quad + 8 * i) * 2);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[i], qb[qt][i], acc, 0, 0, 0);
        s[qt][t] = acc;
      }
    }

    // mask: causal, the sequence's end, and the streaming pattern. A key
    // block below the diagonal needs none when the head is dynamic, or when
    // it lies wholly in the sink or wholly inside every row's window (its
    // first key at or after the last row's window start)
    const int32_t kpos0 = kbk * kB + 4 * quad;      // positions fit 32 bits (L <= 2^24)
    const bool full = kbk < j && (dynamic || (kbk + 1) * kB <= a.sink ||
                                  (int64_t)kbk * kB >= (int64_t)(j + 1) * kB - a.window);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int32_t tq = j * kB + 32 * rh + 16 * qt + col;
      if (!full) {
        int32_t kp0 = kpos0;
        asm volatile("" : "+v"(kp0));      // keeps the comparisons inside this branch
        const int32_t Li = (int32_t)L, sink = a.sink, wlo = tq + 1 - a.window;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int32_t sp = kp0 + 16 * t + r;
            const bool ok = (sp <= tq) & (sp < Li) & (dynamic | (sp < sink) | (sp >= wlo));   // no branches
            s[qt][t][r] = ok ? s[qt][t][r] : -INFINITY;
          }
      }
      // online softmax over the 64 keys of the block for this query column.
      // A column's reference rises only when the block's maximum passes it
      // by the slack. Scaling is monotone, so that happens for some column
      // exactly when some lane's own maximum passes its column's reference:
      // the cross-lane reduction runs only then, with the same outcome
      float bm = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) bm = fmaxf(bm, s[qt][t][r]);
      if (__any(bm * kScaleLog2 > m_ref[qt] + kRescaleSlack)) {
        auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
        bm = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
        auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
        bm = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
        bm *= kScaleLog2;
        // a column with nothing of this block (bm = -inf) keeps its reference;
        // its scores are -inf and their probabilities come out 0 against any
        // finite reference (0 while the column has none yet)
        const bool first = m_ref[qt] == -INFINITY;
        const bool raise = bm > m_ref[qt] + kRescaleSlack;
        const float mn = raise ? bm : m_ref[qt];
        if (__any(raise && !first)) {
          const float alpha = raise && !first ? __builtin_amdgcn_exp2f(m_ref[qt] - mn) : 1.f;
          l_sum[qt] *= alpha;
#pragma unroll
          for (int c = 0; c < 8; ++c) o[qt][c] *= alpha;
        }
        m_ref[qt] = mn;
        m_sub[qt] = mn == -INFINITY ? 0.f : mn;
      }
      const float mx = m_sub[qt];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qt][t][r], kScaleLog2, -mx));
          l_sum[qt] += p;
          s[qt][t][r] = p;
        }
    }

    // O^T += V^T P^T over the two 32-key pairs (tiles 0,1 and 2,3)
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      bf16x8 ph[2], pl[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int x = 0; x < 8; x += 2) {
          const int t = 2 * pr + x / 4, r = x % 4;
          bf16x2 hv, lv;
          split_pair(s[qt][t][r], s[qt][t][r + 1], hv, lv);
          ph[qt][x] = hv[0]; ph[qt][x + 1] = hv[1];
          pl[qt][x] = lv[0]; pl[qt][x + 1] = lv[1];
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        // keys 32pr + 4quad .. +3, then 32pr + 16 + 4quad .. +3 (the interleaved order)
        const uint4 vv = *reinterpret_cast<const uint4*>(vl + ((16 * c + col) * kVStride + 32 * pr + 8 * quad) * 2);
        bf16x8 av;
        __builtin_memcpy(&av, &vv, 16);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          o[qt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ph[qt], o[qt][c], 0, 0, 0);
          o[qt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pl[qt], o[qt][c], 0, 0, 0);
        }
      }
    }
  };

  // two key blocks per barrier: pair q sits in buffers 2 (q & 1) and
  // 2 (q & 1) + 1 while the next pair's global loads are in flight (the
  // buffers it overwrites were last read two pairs before, behind the last
  // barrier)
  St st0, st1;
  const int32_t nk = kl.count;
  if (nk > 0) load_block(kl.at(0, sel_list), st0);
  if (nk > 1) load_block(kl.at(1, sel_list), st1);
  for (int32_t e = 0; e < nk; e += 2) {
    const int buf = 2 * ((e >> 1) & 1);
    store_block(buf, st0);
    if (e + 1 < nk) store_block(buf + 1, st1);
    __syncthreads();
    if (e + 2 < nk) load_block(kl.at(e + 2, sel_list), st0);
    if (e + 3 < nk) load_block(kl.at(e + 3, sel_list), st1);
    block(kl.at(e, sel_list), buf);
    if (e + 1 < nk) block(kl.at(e + 1, sel_list), buf + 1);
  }

  // normalise and store the wave's rows
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float l = l_sum[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int64_t row = (int64_t)j * kB + 32 * rh + 16 * qt + col;
    if (row >= L) continue;
    float* orow = a.out + (qhead * L + row) * kHeadDim + 4 * quad;
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<f32x4*>(orow + 16 * c) = o[qt][c] / l;
    if (a.lse && quad == 0) a.lse[qhead * L + row] = (m_ref[qt] + __log2f(l)) * kLn2;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  hipError_t e;
  if (a.any_dynamic && !a.dense) {
    hipLaunchKernelGGL(pool_kernel, dim3(a.nb, a.hkv, 2), dim3(64), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 grid(a.nb, a.hkv);
    if (a.nb <= 8 * 64) hipLaunchKernelGGL(select_kernel<8>, grid, dim3(64), 0, s, a);
    else if (a.nb <= 16 * 64) hipLaunchKernelGGL(select_kernel<16>, grid, dim3(64), 0, s, a);
    else if (a.nb <= 32 * 64) hipLaunchKernelGGL(select_kernel<32>, grid, dim3(64), 0, s, a);
    else if (a.nb <= 64 * 64) hipLaunchKernelGGL(select_kernel<64>, grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL(select_kernel<128>, grid, dim3(64), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // query heads per work-group: the largest of 4, 2, 1 that divides G
  const int nh = a.G % 4 == 0 ? 4 : a.G % 2 == 0 ? 2 : 1;
  const dim3 grid(a.nb, a.hkv, a.G / nh);
  switch (nh) {
    case 1: hipLaunchKernelGGL(attn_kernel<1>, grid, dim3(128), 0, s, a); break;
    case 2: hipLaunchKernelGGL(attn_kernel<2>, grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(attn_kernel<4>, grid, dim3(512), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace spa
