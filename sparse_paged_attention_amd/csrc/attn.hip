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
#include <atomic>

#include "pool_rows.h"
#include "psplit.h"

namespace spa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// log2(e) / sqrt(128): scores are kept in the log2 domain
constexpr float kScaleLog2 = 0.12751743074602467f;
constexpr float kLn2 = 0.69314718055994531f;

// The same memory seen through the constant address space: wave-uniform
// loads from it are scalar loads. Only for data no kernel of the launch
// writes (lengths, selections, page table).
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* as_scalar(const T* p) {
  return (const __attribute__((address_space(4))) T*)p;
}

// A 16-token block: absolute positions [t0, t0 + 16), of which [lo, hi) count,
// in physical page `phys` (already validated) at logical slot `lp`.
struct Block {
  int32_t t0, lo, hi, phys, lp;
};

// Operand registers of a pair of blocks (a, b). V is kept the way the PV
// MFMA consumes it: v[c] = {block a's 4 tokens, block b's 4 tokens} of
// channel 16c + (lane & 15), so the loads land in place.
struct PairTile {
  uint4 ka[4], kb[4];   // K rows: this lane's 64 bytes of token (lane & 15) of a / b
  uint4 v[8];
};

// Issues the loads of block `blk` into the a (half = 0) or b (half = 1) half
// of a pair tile. Empty blocks load from page 0 of the pool (always mapped),
// so the loads never depend on control flow; the padding slot of an odd
// item loads nothing and is zero. The block base is wave-uniform and each
// lane adds a fixed 32-bit offset (scalar base + vector offset addressing).
template <int PG>
__device__ __forceinline__ void issue_half(const PoolArgs& pl, int32_t h, const Block& blk, PairTile& t,
                                           int half, bool real) {
  uint4* kd = half ? t.kb : t.ka;
  if (!real) {
#pragma unroll
    for (int i = 0; i < 4; ++i) kd[i] = uint4{0, 0, 0, 0};
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
      if (half) { t.v[ch].z = 0; t.v[ch].w = 0; } else { t.v[ch].x = 0; t.v[ch].y = 0; }
    }
    return;
  }
  const int lane = threadIdx.x & 63;
  const int row = lane & 15, quad = lane >> 4;
  const int64_t head = (int64_t)blk.phys * pl.hs + h;     // h: the head's slot in its page
  const int32_t in_page = blk.t0 & (PG - 1);
  const uint16_t* kbase = pl.k + (head * pl.P + blk.lp * PG + in_page) * kHeadDim;
  const uint16_t* vbase = pl.v + (head * pl.r + blk.lp) * (int64_t)(kHeadDim * PG) + in_page;
  const uint32_t koff = row * kHeadDim + 32 * quad, voff = row * PG + 4 * quad;
#pragma unroll
  for (int i = 0; i < 4; ++i) kd[i] = *reinterpret_cast<const uint4*>(kbase + koff + 8 * i);
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    const uint2 w = *reinterpret_cast<const uint2*>(vbase + voff + 16 * ch * PG);
    if (half) { t.v[ch].z = w.x; t.v[ch].w = w.y; } else { t.v[ch].x = w.x; t.v[ch].y = w.y; }
  }
}

// fp8 pages: the same tiles as E4M3 codes (half the bytes), with each
// token's key and value scale. A lane's four score rows (tokens 4*quad .. +3
// of a block) are also the four tokens of its probabilities, so one f32x4 of
// key scales and one of value scales per block cover both uses.
struct PairTile8 {
  uint4 ka[2], kb[2];       // K codes: this lane's 32 bytes of token (lane & 15) of a / b
  uint32_t va[8], vb[8];    // V codes: tokens 4*quad .. +3 of channel 16c + (lane & 15), block a / b
  f32x4 ksa, ksb, vsa, vsb; // key / value scales of tokens 4*quad .. +3 of block a / b
};

template <int PG>
__device__ __forceinline__ void issue_half8(const PoolArgs& pl, int32_t h, const Block& blk, PairTile8& t,
                                            int half, bool real) {
  uint4* kd = half ? t.kb : t.ka;
  uint32_t* vd = half ? t.vb : t.va;
  f32x4& ks = half ? t.ksb : t.ksa;
  f32x4& vs = half ? t.vsb : t.vsa;
  if (!real) {
#pragma unroll
    for (int i = 0; i < 2; ++i) kd[i] = uint4{0, 0, 0, 0};
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) vd[ch] = 0;
    ks = f32x4{0.f, 0.f, 0.f, 0.f};
    vs = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  const int lane = threadIdx.x & 63;
  const int row = lane & 15, quad = lane >> 4;
  const int64_t head = (int64_t)blk.phys * pl.hs + h;     // h: the head's slot in its page
  const int32_t in_page = blk.t0 & (PG - 1);
  const int64_t row0 = head * pl.P + blk.lp * PG + in_page; // the block's first token row
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(pl.k) + row0 * kHeadDim;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(pl.v) + (head * pl.r + blk.lp) * (int64_t)(kHeadDim * PG) + in_page;
  const uint32_t koff = row * kHeadDim + 32 * quad, voff = row * PG + 4 * quad;
#pragma unroll
  for (int i = 0; i < 2; ++i) kd[i] = *reinterpret_cast<const uint4*>(kbase + koff + 16 * i);
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) vd[ch] = *reinterpret_cast<const uint32_t*>(vbase + voff + 16 * ch * PG);
  ks = *reinterpret_cast<const f32x4*>(pl.ks + row0 + 4 * quad);
  vs = *reinterpret_cast<const f32x4*>(pl.vs + row0 + 4 * quad);
}

struct State {
  float m;          // running reference (near the maximum) of this lane's query, log2 units
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

// Cross-lane sum over the four 16-lane rows.
__device__ __forceinline__ float sum_over_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Scores S^T[16 tok][16 q] of one block: 4 chained 16x16x32 MFMAs over D.
__device__ __forceinline__ f32x4 qk_block(const uint4 (&k)[4], const bf16x8 (&qb)[4]) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16x8 a;
    __builtin_memcpy(&a, &k[i], 16);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[i], s, 0, 0, 0);
  }
  return s;
}

// qk_block over E4M3 key codes: the codes become bf16 operands exactly; the
// key scale is applied to the scores afterwards.
__device__ __forceinline__ f32x4 qk_block8(const uint4 (&k)[2], const bf16x8 (&qb)[4]) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4& w = k[i / 2];
    const uint2 lo = codes_bf16x4(i % 2 ? w.z : w.x), hi = codes_bf16x4(i % 2 ? w.w : w.y);
    const uint4 u = {lo.x, lo.y, hi.x, hi.y};
    bf16x8 a;
    __builtin_memcpy(&a, &u, 16);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[i], s, 0, 0, 0);
  }
  return s;
}

// The running reference of the online softmax is raised only when a block's
// maximum exceeds it by more than this (log2 units): probabilities then stay
// below 2^kRescaleSlack, and the rescale of the accumulators (which live in
// accumulation registers) is rare instead of happening on most blocks.
// out = o / l and lse = ref + log2(l) are unchanged by the choice of reference.
constexpr float kRescaleSlack = 8.f;

// Probabilities of a pair of blocks, in the form the PV MFMA consumes.
struct PairProbs {
  bf16x8 hi, lo;       // P split into bf16 high and low parts
  uint32_t mk[4];      // V masks (token validity) when the pair is not full
  bool full, any;      // every token valid / at least one valid token
};

// Online-softmax step for two blocks (32 tokens) given their scores: updates
// the running reference and sum, rescales the accumulators when the
// reference rises, and returns this lane's 8 probabilities (K-slot j of lane
// row q: token 4q + j of block a for j < 4, token 4q + j - 4 of block b).
// Q8 (fp8 pages): the scores are multiplied by their key scales first, and
// the probabilities by their value scales after the running sum has taken
// them (the sum is over softmax weights, the value scale belongs to V).
template <bool Q8 = false>
__device__ __forceinline__ PairProbs softmax_pair(const Block& ba, const Block& bb, const f32x4& sa,
                                                  const f32x4& sb, State& st, const f32x4* ksa = nullptr,
                                                  const f32x4* ksb = nullptr, const f32x4* vsa = nullptr,
                                                  const f32x4* vsb = nullptr) {
  PairProbs pp;
  const int quad = (threadIdx.x & 63) >> 4;
  pp.full = ba.lo <= ba.t0 && ba.hi >= ba.t0 + kBlockTokens && bb.lo <= bb.t0 && bb.hi >= bb.t0 + kBlockTokens;
  float s[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s[r] = Q8 ? sa[r] * (*ksa)[r] : sa[r];
    s[4 + r] = Q8 ? sb[r] * (*ksb)[r] : sb[r];
  }
  if (!pp.full) {                                  // mask the invalid tokens (uniform branch)
    bool valid[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int32_t tka = ba.t0 + 4 * quad + r, tkb = bb.t0 + 4 * quad + r;
      valid[r] = tka >= ba.lo && tka < ba.hi;
      valid[4 + r] = tkb >= bb.lo && tkb < bb.hi;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) s[r] = valid[r] ? s[r] : -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pp.mk[i] = (valid[2 * i] ? 0x0000FFFFu : 0u) | (valid[2 * i + 1] ? 0xFFFF0000u : 0u);
  }
  float bm = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
  bm = max_over_rows(bm) * kScaleLog2;            // this query's maximum over the pair, log2 units
  pp.any = bm != -INFINITY;                       // same for every lane
  if (!pp.any) return pp;
  const bool first = st.m == -INFINITY;
  const bool raise = bm > st.m + kRescaleSlack;   // always true on the first block
  const float m_new = raise ? bm : st.m;
  if (__any(raise && !first)) {                   // o and l are still zero before the first block
    const float alpha = raise && !first ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.f;
    st.l *= alpha;
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) st.o[ch] *= alpha;
  }
  st.m = m_new;
  float pr[8];
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], kScaleLog2, -m_new));   // 0 for masked tokens
    psum += pr[r];
  }
  st.l += psum;
  if (Q8) {                                       // masked tokens keep 0 whatever their (stale) scale
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = pr[r] != 0.f ? pr[r] * (*vsa)[r] : 0.f;
      pr[4 + r] = pr[4 + r] != 0.f ? pr[4 + r] * (*vsb)[r] : 0.f;
    }
  }
#pragma unroll
  for (int r = 0; r < 8; r += 2) {
    bf16x2 h, lo;
    split_pair(pr[r], pr[r + 1], h, lo);
    pp.hi[r] = h[0]; pp.hi[r + 1] = h[1];
    pp.lo[r] = lo[0]; pp.lo[r + 1] = lo[1];
  }
  return pp;
}

// O^T[128][16 q] += V^T[128][32 tok] . P^T: one 16x16x32 MFMA per 16
// channels for each of the two parts of P.
__device__ __forceinline__ void pv_pair(const PairTile& t, const PairProbs& pp, State& st) {
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    uint4 w = t.v[ch];
    if (!pp.full) {                                // stale pool bytes must not reach the MFMA
      w.x &= pp.mk[0];
      w.y &= pp.mk[1];
      w.z &= pp.mk[2];
      w.w &= pp.mk[3];
    }
    bf16x8 a;
    __builtin_memcpy(&a, &w, 16);
    st.o[ch] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pp.hi, st.o[ch], 0, 0, 0);
    st.o[ch] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pp.lo, st.o[ch], 0, 0, 0);
  }
}

// pv_pair over E4M3 value codes (the value scales are already in P).
__device__ __forceinline__ void pv_pair8(const PairTile8& t, const PairProbs& pp, State& st) {
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    const uint2 a2 = codes_bf16x4(t.va[ch]), b2 = codes_bf16x4(t.vb[ch]);
    uint4 w = {a2.x, a2.y, b2.x, b2.y};
    if (!pp.full) {                                // stale pool bytes must not reach the MFMA
      w.x &= pp.mk[0];
      w.y &= pp.mk[1];
      w.z &= pp.mk[2];
      w.w &= pp.mk[3];
    }
    bf16x8 a;
    __builtin_memcpy(&a, &w, 16);
    st.o[ch] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pp.hi, st.o[ch], 0, 0, 0);
    st.o[ch] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pp.lo, st.o[ch], 0, 0, 0);
  }
}

// The partial of the token appended in the same launch, taken from the
// caller's buffers (the pool row is being written by this very wave): for
// each query g of the group, reference = its score q_g . k / sqrt(D) (log2
// units), sum = 1, output = the value row; an empty partial when the token
// has no pool slot (no token, or an unmapped page: such a token is not
// attended). Written to slot `it` of the head like an item's partial. Lane
// (g, quad) covers q channels 32*quad .. +32 and output channels
// 16c + 4*quad + r, as in the items.
__device__ __forceinline__ void token_partial(const PoolArgs& pl, const BatchArgs& bt, int32_t b, int32_t h,
                                              int32_t G, int32_t item_stride, int32_t it, const uint16_t* q,
                                              const uint16_t* k_new, const uint16_t* v_new, float* part_o,
                                              float* part_ml, bool in_ring) {
  const int lane = threadIdx.x & 63, g = lane & 15, quad = lane >> 4;
  const int32_t L = clamp_len(bt, b, pl.P);
  bool valid = L >= 1;
  if (valid) {
    const int32_t phys = in_ring ? ring_page(bt, bt.ring[b], L - 1, pl.P, pl.N)
                                 : bt.pt[(int64_t)b * bt.max_pp + (L - 1) / pl.P];
    valid = phys >= 0 && phys < pl.N;
  }
  const int64_t bh = (int64_t)b * pl.hkv + h;
  const int32_t gq = g < G ? g : 0;
  const uint4* q4 = reinterpret_cast<const uint4*>(q + (bh * G + gq) * kHeadDim + 32 * quad);
  const uint4* k4 = reinterpret_cast<const uint4*>(k_new + bh * kHeadDim + 32 * quad);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 qw = q4[i], kw = k4[i];
    bf16x8 qv, kv;
    __builtin_memcpy(&qv, &qw, 16);
    __builtin_memcpy(&kv, &kw, 16);
#pragma unroll
    for (int j = 0; j < 8; ++j) s = __builtin_fmaf((float)qv[j], (float)kv[j], s);
  }
  const float t = sum_over_rows(s) * kScaleLog2;
  if (g >= G) return;
  const int64_t slot = (bh * item_stride + it) * G + g;
  float* o = part_o + slot * kHeadDim + 4 * quad;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint2 w = *reinterpret_cast<const uint2*>(v_new + bh * kHeadDim + 16 * c + 4 * quad);
    f32x4 v = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
               __uint_as_float(w.y & 0xFFFF0000u)};
    if (!valid) v = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(o + 16 * c) = v;
  }
  if (quad == 0) {
    part_ml[slot * 2 + 0] = valid ? t : -INFINITY;
    part_ml[slot * 2 + 1] = valid ? 1.f : 0.f;
  }
}

// token_partial on fp8 pages, from the token's rows as the append quantizes
// them (kc / vc: lane l holds the codes of channels 2l and 2l + 1; ks / vs the
// row scales; the same codes the pool receives): the score over the key codes
// times the key scale, the output the dequantized value row -- the arithmetic
// the items apply to every stored token. Each lane fetches the codes of its
// channels from the lanes that quantized them.
__device__ __forceinline__ void token_partial_q8(const PoolArgs& pl, const BatchArgs& bt, int32_t b, int32_t h,
                                                 int32_t G, int32_t item_stride, int32_t it, const uint16_t* q,
                                                 uint32_t kc, float ks, uint32_t vc, float vs, float* part_o,
                                                 float* part_ml, bool in_ring) {
  const int lane = threadIdx.x & 63, g = lane & 15, quad = lane >> 4;
  const int32_t L = clamp_len(bt, b, pl.P);
  bool valid = L >= 1;
  if (valid) {
    const int32_t phys = in_ring ? ring_page(bt, bt.ring[b], L - 1, pl.P, pl.N)
                                 : bt.pt[(int64_t)b * bt.max_pp + (L - 1) / pl.P];
    valid = phys >= 0 && phys < pl.N;
  }
  const int64_t bh = (int64_t)b * pl.hkv + h;
  const int32_t gq = g < G ? g : 0;
  const uint4* q4 = reinterpret_cast<const uint4*>(q + (bh * G + gq) * kHeadDim + 32 * quad);
  // q channels 32 quad + 8 i + j; their key codes sit in lane 16 quad + 4 i + j / 2
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 qw = q4[i];
    bf16x8 qv;
    __builtin_memcpy(&qv, &qw, 16);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t c2 = (uint32_t)__shfl((int)kc, 16 * quad + 4 * i + m, 64);
      s = __builtin_fmaf((float)qv[2 * m], e4m3_value(c2 & 0xFFu), s);
      s = __builtin_fmaf((float)qv[2 * m + 1], e4m3_value((c2 >> 8) & 0xFFu), s);
    }
  }
  const float t = sum_over_rows(s) * ks * kScaleLog2;
  // output channels 16 c + 4 quad + r; their value codes sit in lane 8 c + 2 quad + r / 2
  f32x4 v[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint32_t c2 = (uint32_t)__shfl((int)vc, 8 * c + 2 * quad + m, 64);
      v[c][2 * m] = e4m3_value(c2 & 0xFFu) * vs;
      v[c][2 * m + 1] = e4m3_value((c2 >> 8) & 0xFFu) * vs;
    }
  if (g >= G) return;
  const int64_t slot = (bh * item_stride + it) * G + g;
  float* o = part_o + slot * kHeadDim + 4 * quad;
#pragma unroll
  for (int c = 0; c < 8; ++c)
    *reinterpret_cast<f32x4*>(o + 16 * c) = valid ? v[c] : f32x4{0.f, 0.f, 0.f, 0.f};
  if (quad == 0) {
    part_ml[slot * 2 + 0] = valid ? t : -INFINITY;
    part_ml[slot * 2 + 1] = valid ? 1.f : 0.f;
  }
}

// Which blocks an item covers. Blocks are numbered per head:
//   streaming: the sink blocks, then the window blocks;
//   dynamic:   block (i, s) = 16-token block s of the i-th selected page,
//              limited to positions below L_s (the length at selection);
//   tail:      16-token blocks of [floor16(L_s), L), limited to [L_s, L).
// Selected pages below L_s plus all of [L_s, L) is the same token set as
// selected pages below L plus the part of [L_s, L) outside them, and needs
// no membership test.
struct BlockSource {
  int32_t kind;          // 0 streaming, 1 dynamic, 2 tail
  int32_t L, ls;         // ls: L_s clamped to [0, lim]
  int32_t lim;           // pool rows below lim are read (L, or L - 1 when the last token is appended in this launch)
  int32_t s0, w0, nb_sink, first_w;          // streaming
  int32_t ring_base;                         // streaming: first page of the sequence's ring, if kept in one
  int32_t ls_floor;                          // tail
};

// Resolves blocks [v0, v0 + BPI) (those at or past v_end are empty) to pool
// locations, then streams them through a ring of DEPTH operand tiles: the
// first DEPTH blocks' loads are issued together, and each tile is refilled
// with block u + DEPTH as soon as block u has been computed. The look-ups
// (selected page ids, page-table entries) are wave-uniform scalar loads:
// they travel on the scalar-memory path, so they never queue behind the
// tile loads other waves of the compute unit have in flight, and every
// level of look-up costs one round trip for the whole item. For selected
// pages the page-table entry depends only on the page id (`page`, loaded by
// the caller before the lengths arrive). The kernel has a single call site,
// so one copy of the pipeline serves every kind of item (instruction-cache
// footprint).
template <bool Q8> struct TileOf { using T = PairTile; };
template <> struct TileOf<true> { using T = PairTile8; };

template <int PG, int BPI, int DEPTH, bool RING, bool Q8>
__device__ __forceinline__ void run_blocks(const PoolArgs& pl, const BatchArgs& bt, const int32_t* pt_row,
                                           int32_t max_pp, int32_t h, const BlockSource& src,
                                           const int32_t (&page)[(BPI + 1) & ~1],
                                           const int32_t (&page_phys)[(BPI + 1) & ~1], bool use_phys,
                                           int32_t v0, int32_t v_end, const bf16x8 (&qb)[4], State& st) {
  constexpr int SB = PG / kBlockTokens;           // blocks per logical page
  constexpr int NB = (BPI + 1) & ~1;              // pipeline slots: BPI rounded up to pairs
  const int32_t r = pl.P / PG;
  const auto pt = as_scalar(pt_row);
  Block blk[NB];
  int32_t ptv[NB];
  if (src.kind == 1) {
    if (use_phys) {                                // resolved when the pages were selected
#pragma unroll
      for (int u = 0; u < NB; ++u) ptv[u] = page_phys[u];
    } else {
#pragma unroll
      for (int u = 0; u < NB; ++u) ptv[u] = pt[min(max(page[u], 0) / r, max_pp - 1)];
    }
    const int32_t n_pages_s = (src.ls + PG - 1) / PG;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int32_t j = page[u];
      const bool ok = v0 + u < v_end && j >= 0 && j < n_pages_s;
      const int32_t t0 = ok ? j * PG + ((v0 + u) % SB) * kBlockTokens : 0;
      blk[u] = Block{t0, t0, ok ? min(t0 + kBlockTokens, src.ls) : t0, 0, 0};
    }
  } else {
    if (src.kind == 0) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int32_t v = v0 + u;
        int32_t t0, lo, hi;
        if (v < src.nb_sink) {
          t0 = v * kBlockTokens; lo = t0; hi = min(t0 + kBlockTokens, min(src.s0, src.lim));
        } else {
          t0 = (src.first_w + v - src.nb_sink) * kBlockTokens; lo = max(t0, src.w0);
          hi = min(t0 + kBlockTokens, src.lim);
        }
        if (v >= v_end) { t0 = 0; lo = 0; hi = 0; }
        blk[u] = Block{t0, lo, hi, 0, 0};
      }
    } else {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int32_t t0 = src.ls_floor + (v0 + u) * kBlockTokens;
        const int32_t lo = max(t0, src.ls), hi = v0 + u < v_end ? min(t0 + kBlockTokens, src.lim) : lo;
        blk[u] = Block{hi > lo ? t0 : 0, lo, hi, 0, 0};
      }
    }
    if (RING && src.kind == 0) {               // the ring's pages follow from the position alone
#pragma unroll
      for (int u = 0; u < NB; ++u) ptv[u] = ring_page(bt, src.ring_base, blk[u].t0, pl.P, pl.N);
    } else {
#pragma unroll
      for (int u = 0; u < NB; ++u) ptv[u] = pt[min(blk[u].t0 / pl.P, max_pp - 1)];
    }
  }
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int32_t j = blk[u].t0 / PG;
    int32_t phys = ptv[u];
    if (phys < 0 || phys >= pl.N || blk[u].hi <= blk[u].lo) { phys = 0; blk[u].hi = blk[u].lo; blk[u].t0 = 0; }
    blk[u].phys = phys;
    blk[u].lp = blk[u].hi > blk[u].lo ? j % r : 0;
  }
  // Blocks go in pairs through a ring of DEPTH / 2 pair tiles. The scores of
  // the next pair are computed before the current pair's PV product, so its
  // MFMAs queue behind the current ones while the VALU works on the softmax.
  static_assert(DEPTH % 2 == 0, "blocks are processed in pairs");
  constexpr int D = DEPTH < NB ? DEPTH : NB;
  constexpr int NT = D / 2;
  using Tile = typename TileOf<Q8>::T;
  Tile t[NT];
  auto issue = [&](const Block& bk, Tile& tile, int half, bool real) {
    if constexpr (Q8) issue_half8<PG>(pl, h, bk, tile, half, real);
    else issue_half<PG>(pl, h, bk, tile, half, real);
  };
  auto qk = [&](const Tile& tile, int half) {
    if constexpr (Q8) return qk_block8(half ? tile.kb : tile.ka, qb);
    else return qk_block(half ? tile.kb : tile.ka, qb);
  };
#pragma unroll
  for (int u = 0; u < D; u += 2) {
    issue(blk[u], t[u / 2], 0, u < BPI);
    issue(blk[u + 1], t[u / 2], 1, u + 1 < BPI);
  }
  f32x4 sa = qk(t[0], 0), sb = qk(t[0], 1);
#pragma unroll
  for (int u = 0; u < NB; u += 2) {
    const Tile& tc = t[(u / 2) % NT];
    PairProbs pp;
    if constexpr (Q8) pp = softmax_pair<true>(blk[u], blk[u + 1], sa, sb, st, &tc.ksa, &tc.ksb, &tc.vsa, &tc.vsb);
    else pp = softmax_pair(blk[u], blk[u + 1], sa, sb, st);
    if (u + 2 < NB) {
      const Tile& tn = t[((u + 2) / 2) % NT];
      sa = qk(tn, 0);
      sb = qk(tn, 1);
    }
    if (pp.any) {
      if constexpr (Q8) pv_pair8(tc, pp, st);
      else pv_pair(tc, pp, st);
    }
    if (u + D < NB) {
      issue(blk[u + D], t[(u / 2) % NT], 0, u + D < BPI);
      issue(blk[u + 1 + D], t[(u / 2) % NT], 1, u + 1 + D < BPI);
    }
  }
}

// The dynamic-head mask as opaque register values, so that nothing below
// turns into an indexed reload of the launch arguments (one more memory
// round trip).
struct HeadMask {
  uint32_t w0, w1, w2, w3;
  __device__ __forceinline__ explicit HeadMask(const AttnPlan& plan)
      : w0(plan.dyn_mask[0]), w1(plan.dyn_mask[1]), w2(plan.dyn_mask[2]), w3(plan.dyn_mask[3]) {
    asm volatile("" : "+s"(w0), "+s"(w1), "+s"(w2), "+s"(w3));
  }
  // (written with counts only: a select among the words gets turned back
  // into an indexed array read)
  __device__ __forceinline__ bool dynamic(int32_t h) const { return below(h + 1) != below(h); }
  // dynamic heads among [0, h)
  __device__ __forceinline__ int32_t below(int32_t h) const {
    return part(w0, h) + part(w1, h - 32) + part(w2, h - 64) + part(w3, h - 96);
  }
  __device__ __forceinline__ static int32_t part(uint32_t w, int32_t k) {
    return k <= 0 ? 0 : __popc(k >= 32 ? w : w & ((1u << k) - 1u));
  }
};

// One item of one (sequence, KV head): the online softmax over its blocks and
// a partial (max, sum, unnormalised output) per query head.
// FRESH: the step's token is appended in this launch (k_new / v_new given);
// a separate instantiation, so plain attention carries none of its code.
template <int PG, int BPI, int DEPTH, bool FRESH, bool RING, bool Q8 = false>
__global__ void __launch_bounds__(64) attn_kernel(PoolArgs pl, BatchArgs bt, AttnPlan plan, int32_t G,
                                                  const uint16_t* q, const int32_t* sel_pages,
                                                  const int32_t* sel_count, const int32_t* sel_len,
                                                  const int32_t* sel_phys, float* part_o, float* part_ml,
                                                  const uint32_t* k_new, const uint16_t* v_new,
                                                  int32_t n_append) {
  constexpr int SB = PG / kBlockTokens;
  // Every launch argument the kernel uses, read into registers in one round:
  // left to itself the compiler fetches each argument just before its first
  // use, one dependent scalar-memory round trip at a time.
  asm volatile("" ::"s"(pl.hkv), "s"(pl.hs), "s"(pl.P), "s"(pl.N), "s"(bt.max_pp), "s"(plan.items_stream),
               "s"(plan.items_dyn), "s"(plan.item_stride), "s"(plan.items_per_seq), "s"(plan.sink),
               "s"(plan.window), "s"(plan.k_max),
               "s"(G), "s"(plan.dyn_mask[0]), "s"(plan.dyn_mask[1]), "s"(plan.dyn_mask[2]),
               "s"(plan.dyn_mask[3]), "s"(plan.sel_mask), "s"(plan.use_phys));
  asm volatile("" ::"s"(pl.k), "s"(pl.v), "s"(bt.pt), "s"(bt.lens), "s"(sel_pages), "s"(sel_count),
               "s"(sel_len), "s"(sel_phys), "s"(q), "s"(part_o), "s"(part_ml),
               "s"(k_new), "s"(v_new), "s"(n_append), "s"(bt.B));
  if (RING) asm volatile("" ::"s"(bt.ring), "s"(bt.ring_sink), "s"(bt.ring_win));
  if (Q8) asm volatile("" ::"s"(pl.ks), "s"(pl.vs));
  // work-group -> (sequence, head, item): head h's first item within the
  // sequence is h * items_stream + (dynamic heads below h) * (items_dyn - items_stream)
  const HeadMask mask(plan);
  // the last n_append work-groups (after every item, so the items keep their
  // places on the compute units) write the step's token into the pool, one
  // per sequence and KV head, and its partial; no item reads that row
  const int32_t n_items_all = bt.B * plan.items_per_seq;
  if (FRESH && (int32_t)blockIdx.x >= n_items_all) {
    const int32_t w = (int32_t)blockIdx.x - n_items_all;
    const int32_t ab = w / pl.hkv, ah = w - ab * pl.hkv;
    const int32_t n_it = mask.dynamic(ah) ? plan.items_dyn : plan.items_stream;
    const int32_t hsl_a = head_slot(pl, ah, mask.below(ah), mask.dynamic(ah));
    if constexpr (Q8) {                 // the rows quantized once, shared by the partial and the append
      const int lane = threadIdx.x & 63;
      const int64_t src = ((int64_t)ab * pl.hkv + ah) * (kHeadDim / 2);
      const uint32_t kin = k_new[src + lane], vin = reinterpret_cast<const uint32_t*>(v_new)[src + lane];
      float ks, vs;
      const uint32_t kc = quantize_pair(kin, ks), vc = quantize_pair(vin, vs);
      token_partial_q8(pl, bt, ab, ah, G, plan.item_stride, n_it, q, kc, ks, vc, vs, part_o, part_ml,
                       RING && !mask.dynamic(ah));
      store_token_q8(pl, bt, ab, hsl_a, kc, ks, vc, vs, mask.dynamic(ah), RING && !mask.dynamic(ah));
    } else {
      token_partial(pl, bt, ab, ah, G, plan.item_stride, n_it, q, reinterpret_cast<const uint16_t*>(k_new), v_new,
                    part_o, part_ml, RING && !mask.dynamic(ah));
      append_token(pl, bt, ab, ah, hsl_a, k_new, v_new, mask.dynamic(ah), RING && !mask.dynamic(ah));
    }
    return;
  }
  const int32_t item = (int32_t)blockIdx.x;
  const int32_t b = item / plan.items_per_seq;
  const int32_t rem = item - b * plan.items_per_seq;
  const int32_t extra = plan.items_dyn - plan.items_stream;
  int32_t h = 0;
  for (int32_t hi = pl.hkv; hi - h > 1;) {
    const int32_t mid = (h + hi) >> 1;
    if (mid * plan.items_stream + mask.below(mid) * extra <= rem) h = mid; else hi = mid;
  }
  const int32_t it = rem - (h * plan.items_stream + mask.below(h) * extra);
  const bool dynamic = mask.dynamic(h);
  const int32_t n_items = dynamic ? plan.items_dyn : plan.items_stream;
  const int32_t kind = !dynamic ? 0 : (it < n_items - 1 ? 1 : 2);
  const int lane = threadIdx.x & 63;
  const int g = lane & 15, quad = lane >> 4;

  // one round of independent loads: length, selection count and length, the
  // selected page ids of the item's blocks, the query
  const int64_t bh = (int64_t)b * pl.hkv + h;
  // (sel_mask is 0 when no head is dynamic: the selection pointers then
  // alias the lengths and every index collapses to 0)
  constexpr int NB = (BPI + 1) & ~1;
  const int32_t L_raw = as_scalar(bt.lens)[b];
  const int32_t cnt_raw = as_scalar(sel_count)[bh & plan.sel_mask];
  const int32_t ls_raw = as_scalar(sel_len)[b & plan.sel_mask];
  const int32_t ring_raw = RING ? as_scalar(bt.ring)[b] : -1;
  int32_t page[NB], page_phys[NB];
  {
    const auto sp = as_scalar(sel_pages);
    const auto sq = as_scalar(sel_phys);          // aliases sel_pages when not in use
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int64_t i = (bh * plan.k_max + min((it * BPI + u) / SB, plan.k_max - 1)) & plan.sel_mask;
      page[u] = sp[i];
      page_phys[u] = sq[i];
    }
  }
  // all of the round in flight together, waited for once (the compiler would
  // otherwise sink each load to its first use, behind the branches)
  asm volatile("" ::"s"(L_raw), "s"(cnt_raw), "s"(ls_raw), "s"(ring_raw));
#pragma unroll
  for (int u = 0; u < NB; ++u) asm volatile("" ::"s"(page[u]), "s"(page_phys[u]));
  const int32_t* pt_row = bt.pt + (int64_t)b * bt.max_pp;

  // query operand: Q[g][32*quad + 8*i .. +8]. Columns g >= G carry a copy of
  // query 0: every column of the scores, of the softmax (its reductions run
  // over tokens, within a column) and of the PV product is independent of the
  // others, and those columns are never stored, so they need no zeroing --
  // zeroing them would make the wave wait for this load before issuing any
  // tile load.
  bf16x8 qb[4];
  const int32_t hq = pl.hkv * G;
  {
    const int32_t gq = g < G ? g : 0;
    const uint4* q4 = reinterpret_cast<const uint4*>(q + ((int64_t)b * hq + h * G + gq) * kHeadDim + 32 * quad);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = q4[i];
      __builtin_memcpy(&qb[i], &w, 16);
    }
  }

  State st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) st.o[ch] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t cap = bt.max_pp * pl.P;
  const int32_t L = L_raw < 0 ? 0 : (L_raw > cap ? cap : L_raw);
  // with the step's token appended in this launch, pool rows are read below
  // L - 1 only (the token has a partial of its own)
  BlockSource src;
  src.kind = kind;
  src.L = L;
  src.lim = FRESH ? max(L - 1, 0) : L;
  src.ls = min(max(ls_raw, 0), src.lim);
  src.ring_base = ring_raw;
  int32_t v_begin = it * BPI, v_end = 0;
  if (kind == 0) {
    src.s0 = min(plan.sink, L);
    src.w0 = max(plan.sink, L - plan.window);
    src.nb_sink = (src.s0 + kBlockTokens - 1) / kBlockTokens;
    src.first_w = src.w0 / kBlockTokens;
    const int32_t nb_win = L > src.w0 ? (L - 1) / kBlockTokens - src.first_w + 1 : 0;
    v_end = min(src.nb_sink + nb_win, v_begin + BPI);
  } else if (kind == 1) {
    const int32_t cnt = min(max(cnt_raw, 0), plan.k_max);
    v_end = min(cnt * SB, v_begin + BPI);
  } else {
    src.ls_floor = (src.ls / kBlockTokens) * kBlockTokens;
    v_begin = 0;
    v_end = (L - src.ls_floor + kBlockTokens - 1) / kBlockTokens;   // any length: chunks of BPI
  }
  for (int32_t v0 = v_begin; v0 < v_end; v0 += BPI)
    run_blocks<PG, BPI, DEPTH, RING, Q8>(pl, bt, pt_row, bt.max_pp, head_slot(pl, h, mask.below(h), dynamic), src, page, page_phys, plan.use_phys != 0, v0, v_end,
                               qb, st);

  // fold the four token quads of the running sum, store the partial
  st.l += __shfl_xor(st.l, 16, 64);
  st.l += __shfl_xor(st.l, 32, 64);
  if (g < G) {
    const int64_t slot = (bh * plan.item_stride + it) * G + g;
    float* o = part_o + slot * kHeadDim + 4 * quad;
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) *reinterpret_cast<f32x4*>(o + 16 * ch) = st.o[ch];
    if (quad == 0) {
      part_ml[slot * 2 + 0] = st.m;
      part_ml[slot * 2 + 1] = st.l;
    }
  }
}

// Merge of the item partials of one query head: the running-max /
// running-sum rule of online softmax applied across items (long-context
// survey "2.1"; Novita article "2."). One wave per (sequence, query head,
// quarter of the channels): lane (slice, c4) folds channels
// 32*quarter + 4*c4 .. +3 over items slice, slice + 8, ..., all of a chunk's
// loads issued before any is used; the eight slices are then folded across
// lanes.
constexpr int kCombineSlices = 8;
constexpr int kCombineChunk = 8;

__device__ __forceinline__ void fold_partial(float m_i, float l_i, const f32x4& o_i, float& M, float& l,
                                             f32x4& o) {
  if (m_i == -INFINITY) return;                  // empty item
  const float Mn = fmaxf(M, m_i);
  const float a = __builtin_amdgcn_exp2f(M - Mn), c = __builtin_amdgcn_exp2f(m_i - Mn);
  l = l * a + l_i * c;
  o = o * a + o_i * c;
  M = Mn;
}

__global__ void __launch_bounds__(64) combine_kernel(int32_t hkv, AttnPlan plan, int32_t G,
                                                     const float* __restrict__ part_o,
                                                     const float* __restrict__ part_ml, float* __restrict__ out,
                                                     float* __restrict__ lse) {
  // all launch arguments in one scalar-memory round trip (see attn_kernel)
  asm volatile("" ::"s"(hkv), "s"(G), "s"(plan.items_stream), "s"(plan.items_dyn), "s"(plan.item_stride),
               "s"(plan.extra_partial),
               "s"(plan.dyn_mask[0]), "s"(plan.dyn_mask[1]), "s"(plan.dyn_mask[2]), "s"(plan.dyn_mask[3]),
               "s"(part_o), "s"(part_ml), "s"(out), "s"(lse));
  const HeadMask mask(plan);
  const int32_t quarter = blockIdx.x & 3, oi = blockIdx.x >> 2;    // oi = b * H_q + h * G + g
  const int32_t bh = oi / G, g = oi - bh * G;
  const int32_t h = bh % hkv;
  // (+1: the partial of a token appended in the attention launch)
  const int32_t n_items = (mask.dynamic(h) ? plan.items_dyn : plan.items_stream) + plan.extra_partial;
  const int lane = threadIdx.x, slice = lane >> 3, c4 = lane & 7;
  const int32_t ch = 32 * quarter + 4 * c4;
  const int64_t slot0 = (int64_t)bh * plan.item_stride * G + g;     // slot(i) = slot0 + i * G
  float M = -INFINITY, l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int32_t i0 = slice; i0 < n_items; i0 += kCombineSlices * kCombineChunk) {
    f32x4 ov[kCombineChunk];
    float2 mlv[kCombineChunk];
#pragma unroll
    for (int k = 0; k < kCombineChunk; ++k) {
      const int64_t slot = slot0 + (int64_t)min(i0 + k * kCombineSlices, n_items - 1) * G;
      ov[k] = *reinterpret_cast<const f32x4*>(part_o + slot * kHeadDim + ch);
      mlv[k] = *reinterpret_cast<const float2*>(part_ml + slot * 2);
    }
#pragma unroll
    for (int k = 0; k < kCombineChunk; ++k)
      if (i0 + k * kCombineSlices < n_items) fold_partial(mlv[k].x, mlv[k].y, ov[k], M, l, o);
  }
#pragma unroll
  for (int x = 8; x < 64; x <<= 1) {
    const float M2 = __shfl_xor(M, x, 64), l2 = __shfl_xor(l, x, 64);
    f32x4 o2;
#pragma unroll
    for (int r = 0; r < 4; ++r) o2[r] = __shfl_xor(o[r], x, 64);
    fold_partial(M2, l2, o2, M, l, o);
  }
  if (slice != 0) return;
  f32x4 res = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) res = o / l;
  *reinterpret_cast<f32x4*>(out + (int64_t)oi * kHeadDim + ch) = res;
  if (lse && lane == 0 && quarter == 0) lse[oi] = M == -INFINITY ? -INFINITY : (M + log2f(l)) * kLn2;
}

template <int PG, int BPI, int DEPTH = 4>
hipError_t launch_attn_t(const PoolArgs& pool, const BatchArgs& batch, const AttnPlan& plan, int32_t G,
                         const uint16_t* q, const int32_t* sel_pages, const int32_t* sel_count,
                         const int32_t* sel_len, const int32_t* sel_phys, float* part_o, float* part_ml,
                         float* out, float* lse, const uint16_t* k_new, const uint16_t* v_new, hipStream_t s) {
  const int32_t n_append = k_new ? batch.B * pool.hkv : 0;
  const int64_t grid = n_append + (int64_t)batch.B * plan.items_per_seq;
  // kernel variants: the token appended in the launch (FRESH) and streaming
  // heads kept in rings (RING) are template flags, so launches without them
  // carry none of their code
#define SPA_ATTN_LAUNCH(FRESH, RING, ...)                                                                    \
  hipLaunchKernelGGL((attn_kernel<PG, BPI, DEPTH, FRESH, RING, ##__VA_ARGS__>), dim3((unsigned)grid), dim3(64), \
                     0, s, pool, batch, plan, G, q, sel_pages, sel_count, sel_len, sel_phys, part_o, part_ml,  \
                     reinterpret_cast<const uint32_t*>(k_new), v_new, n_append)
  const bool ring = batch.ring != nullptr;
  if (pool.q8) {
    if (k_new) {
      if (ring) SPA_ATTN_LAUNCH(true, true, true); else SPA_ATTN_LAUNCH(true, false, true);
    } else {
      if (ring) SPA_ATTN_LAUNCH(false, true, true); else SPA_ATTN_LAUNCH(false, false, true);
    }
  } else if (k_new) {
    if (ring) SPA_ATTN_LAUNCH(true, true); else SPA_ATTN_LAUNCH(true, false);
  } else {
    if (ring) SPA_ATTN_LAUNCH(false, true); else SPA_ATTN_LAUNCH(false, false);
  }
#undef SPA_ATTN_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AttnPlan cplan = plan;
  cplan.extra_partial = k_new ? 1 : 0;
  hipLaunchKernelGGL(combine_kernel, dim3(batch.B * pool.hkv * G * 4), dim3(64), 0, s, pool.hkv, cplan, G,
                     part_o, part_ml, out, lse);
  return hipGetLastError();
}

template <int PG>
hipError_t launch_attn_p(const PoolArgs& pool, const BatchArgs& batch, const AttnPlan& plan, int32_t G,
                         const uint16_t* q, const int32_t* sel_pages, const int32_t* sel_count,
                         const int32_t* sel_len, const int32_t* sel_phys, float* part_o, float* part_ml,
                         float* out, float* lse, const uint16_t* k_new, const uint16_t* v_new, hipStream_t s) {
  switch (plan.blocks_per_item) {
#define SPA_BPI_CASE(n) \
    case n: return launch_attn_t<PG, n>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, sel_phys, part_o, part_ml, out, lse, k_new, v_new, s);
    SPA_BPI_CASE(4) SPA_BPI_CASE(5) SPA_BPI_CASE(6) SPA_BPI_CASE(7) SPA_BPI_CASE(8) SPA_BPI_CASE(9)
    SPA_BPI_CASE(10) SPA_BPI_CASE(12) SPA_BPI_CASE(16)
#undef SPA_BPI_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Scratch of spa_sparse_decode_attn_noalloc, for callers that cannot
// allocate: the split partials of one call live in this array instead of a
// caller's workspace. One copy per GPU, held until the process ends; calls
// that overlap on one GPU share it and race.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_area(void** ptr, size_t* bytes) {
  // The array's name is a host-side stand-in, not a device address: the
  // device address comes from the runtime, once per device (each GPU holds
  // its own copy at its own address), with that device current.
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    cache[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  *bytes = kScratchBytes;
  return hipSuccess;
}

hipError_t launch_attn(const PoolArgs& pool, const BatchArgs& batch, const AttnPlan& plan, int32_t G,
                       const uint16_t* q, const int32_t* sel_pages, const int32_t* sel_count,
                       const int32_t* sel_len, const int32_t* sel_phys, float* out, float* lse,
                       float* part_o, float* part_ml, const uint16_t* k_new, const uint16_t* v_new,
                       hipStream_t s) {
  if (batch.B == 0) return hipSuccess;
  switch (pool.p) {
    case 16: return launch_attn_p<16>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, sel_phys, part_o, part_ml, out, lse, k_new, v_new, s);
    case 32: return launch_attn_p<32>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, sel_phys, part_o, part_ml, out, lse, k_new, v_new, s);
    case 64: return launch_attn_p<64>(pool, batch, plan, G, q, sel_pages, sel_count, sel_len, sel_phys, part_o, part_ml, out, lse, k_new, v_new, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spa
