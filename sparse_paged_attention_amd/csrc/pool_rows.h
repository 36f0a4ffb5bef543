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

// Codes of two fp32 values with |y| <= 464 (bits 0-7: y0, bits 8-15: y1) by
// the hardware conversion, which on this GPU writes OCP E4M3 rounded to
// nearest, ties to even: for every such fp32 value its code equals
// e4m3_code's (checked over all of them, both signs).
__device__ __forceinline__ uint32_t e4m3_code2(float y0, float y1) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false) & 0xFFFFu;
}

// Value of a code (never one of the NaN codes), exact in fp32.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return (c & 0x80u) ? -v : v;
}

// fp32 bit pattern -> largest bf16 <= it (bit pattern): truncation, one step
// further down for a negative value with bits cut off.
__device__ __forceinline__ uint32_t bf16_down_bits(uint32_t u) {
  return (u >> 16) + (((u & 0xFFFFu) != 0u) & (u >> 31));
}
// Largest bf16 <= x and smallest bf16 >= x, as bit patterns.
__device__ __forceinline__ uint32_t bf16_down(double x) {
  return bf16_down_bits(__float_as_uint(__double2float_rd(x)));   // largest fp32 <= x first
}
__device__ __forceinline__ uint32_t bf16_up(double x) { return bf16_down(-x) ^ 0x8000u; }

// Values of the two codes in bits 0-7 / 8-15 of c2 by the hardware
// conversion (exact: every E4M3 value is an fp32 value; equal to e4m3_value
// for every code but the NaN ones, checked over all of them).
typedef float e4m3_pair_values __attribute__((ext_vector_type(2)));
__device__ __forceinline__ e4m3_pair_values e4m3_value2(uint32_t c2) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)c2, false);
}

// Two codes (bytes 0-1 of w, or 2-3 with HIGH) as a bf16 pair, by gfx950's
// scaled conversion with scale 1. Exact: an E4M3 value has at most four
// significant bits and an exponent inside bf16's range (equal to e4m3_value
// for every pair of codes but the NaN ones, checked over all of them).
template <bool HIGH>
__device__ __forceinline__ uint32_t codes_bf16x2(uint32_t w) {
  const auto p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH);
  uint32_t u;
  __builtin_memcpy(&u, &p, 4);
  return u;
}

// Four codes (tokens or channels in byte order) as two bf16 words.
__device__ __forceinline__ uint2 codes_bf16x4(uint32_t w) {
  return uint2{codes_bf16x2<false>(w), codes_bf16x2<true>(w)};
}

// Key of an fp32 bit pattern that orders like IEEE totalOrder, with
// consecutive fp32 values on consecutive keys (-0 just below +0), and back.
__device__ __forceinline__ uint32_t f32_key(uint32_t u) { return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u); }
__device__ __forceinline__ uint32_t f32_unkey(uint32_t k) { return k ^ ((k >> 31) ? 0x80000000u : 0xFFFFFFFFu); }

// Keys of the largest fp32 <= v * scale (kd) and the smallest fp32 >= it (ku),
// v the value of a code. The product has at most 4 + 24 significant bits:
// p = RN(v s) and its residual e = fma(v, s, -p), exact while p is a normal
// number (scales from 2^-100 up: |v| >= 2^-9 unless v = 0), put the product
// one key below p when e < 0 and one above when e > 0. Smaller scales take
// the fp64 product, which is exact, rounded each way.
__device__ __forceinline__ void product_keys(float v, float scale, uint32_t& kd, uint32_t& ku) {
  if (!(scale >= 0x1p-100f)) {
    const double x = (double)v * (double)scale;
    kd = f32_key(__float_as_uint(__double2float_rd(x)));
    ku = f32_key(__float_as_uint(__double2float_ru(x)));
    return;
  }
  const float p = v * scale;
  const float e = __builtin_fmaf(v, scale, -p);
  const uint32_t k = f32_key(__float_as_uint(p));
  kd = k - (e < 0.f ? 1u : 0u);
  ku = k + (e > 0.f ? 1u : 0u);
}

// bf16 bit patterns from such keys: the largest bf16 <= the fp32 of kd, the
// smallest bf16 >= the fp32 of ku (up(x) = -down(-x)). For the product of a
// code's value and a scale these equal bf16_down / bf16_up of the exact fp64
// product, for every code and every scale a bf16 row can have (checked).
__device__ __forceinline__ uint32_t bf16_below_key(uint32_t kd) { return bf16_down_bits(f32_unkey(kd)); }
__device__ __forceinline__ uint32_t bf16_above_key(uint32_t ku) {
  return bf16_down_bits(f32_unkey(ku) ^ 0x80000000u) ^ 0x8000u;
}

// Wave-wide maximum of unsigned values (every lane of the wave active): DPP
// within each 16-lane row (neighbours, pairs, mirrored halves, mirrored rows),
// then the cross-row lane swaps; every lane ends with the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));   // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(b[0], b[1]);
}

// Whether the fp32 value q lies within 4 ulp of a rounding boundary of E4M3
// (a midpoint between two codes): there a quotient rounded another way
// could take the other code. (Both ranges tested, then one picked: no
// branch.)
__device__ __forceinline__ bool near_e4m3_boundary(float q) {
  const uint32_t a = __float_as_uint(q) & 0x7FFFFFFFu;
  const bool normal = ((a & 0xFFFFFu) - 0x7FFFCu) <= 8u;          // the 20 bits below the 3 kept
  const float y = __uint_as_float(a) * 512.f;                     // below 2^-6: multiples of 2^-9
  const bool sub = fabsf((y - truncf(y)) - 0.5f) <= 0x1p-19f;
  return a >= 0x3C800000u ? normal : sub;
}

// The row scale RN(amax / 448) of a bf16 row maximum: amax times the fp32
// nearest 1/448, corrected once by the exact residual (an FMA); equal to the
// IEEE division for every bf16 value (checked over all of them).
__device__ __forceinline__ float row_scale(float amax) {
  constexpr float kInv448 = 1.f / 448.f;
  const float q = amax * kInv448;
  return __builtin_fmaf(__builtin_fmaf(-q, 448.f, amax), kInv448, q);
}

// Quantizes one D = 128 row held by a wave as bf16 pairs (lane l: channels 2l
// and 2l + 1, in w). Returns the lane's two codes (bits 0-7 and 8-15) and sets
// the row's scale. Every lane of the wave must take part (cross-lane max).
// Each code is that of the correctly rounded quotient x / scale: x times the
// reciprocal of the scale is within 3 ulp of it, and within 4 ulp of a
// rounding boundary the division decides; for every bf16 row maximum and
// every bf16 x up to it this gives the division's code (checked over all
// pairs). Scales below 2^-100 divide; a row of zeros has scale 0 and codes 0.
__device__ __forceinline__ uint32_t quantize_pair(uint32_t w, float& scale) {
  const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xFFFF0000u);
  const uint32_t amax = wave_max_u32(max(__float_as_uint(x0) & 0x7FFFFFFFu, __float_as_uint(x1) & 0x7FFFFFFFu));
  scale = row_scale(__uint_as_float(amax));
  const bool tiny = !(scale >= 0x1p-100f);
  const float r = __builtin_amdgcn_rcpf(scale);
  float q0 = x0 * r, q1 = x1 * r;
  const bool n0 = tiny | near_e4m3_boundary(q0), n1 = tiny | near_e4m3_boundary(q1);
  if (n0 | n1) {                                   // rare (and rows of zeros: 0 / 0, masked below)
    if (n0) q0 = x0 / scale;
    if (n1) q1 = x1 / scale;
  }
  const uint32_t c = e4m3_code2(q0, q1);
  return scale == 0.f ? 0u : c;
}

// Unsigned 16-bit maximum of the two halves of two words (one packed
// instruction).
typedef unsigned short u16_pair __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16_pair, a),
                                                                __builtin_bit_cast(u16_pair, b)));
}
// The magnitudes (bf16 bits less the sign) of two rows' bf16 pairs w0, w1
// folded into one word: low half the larger of w0's two, high half w1's.
__device__ __forceinline__ uint32_t pair_max_u16(uint32_t w0, uint32_t w1) {
  const uint32_t a = w0 & 0x7FFF7FFFu, b = w1 & 0x7FFF7FFFu;
  return pk_max_u16(__builtin_amdgcn_perm(b, a, 0x05040100u), __builtin_amdgcn_perm(b, a, 0x07060302u));
}

// Steps of a reduce-scatter over the wave: two words in, one out, each lane
// keeping the maximum of a pair of lanes for one of the two words.
// Lane-half swap: lanes 0-31 end with x over {l, l + 32}, lanes 32-63 with y.
__device__ __forceinline__ uint32_t fold32(uint32_t x, uint32_t y) {
  const auto s = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  return pk_max_u16(s[0], s[1]);
}
// 16-lane row swap: rows 0 and 2 end with x over {l, l + 16}, rows 1 and 3
// with y.
__device__ __forceinline__ uint32_t fold16(uint32_t x, uint32_t y) {
  const auto s = __builtin_amdgcn_permlane16_swap(x, y, false, false);
  return pk_max_u16(s[0], s[1]);
}
// Within each 16-lane row, by a DPP lane pattern CTRL (a mirror): the 4-lane
// banks in XB keep x folded with its mirror lanes, the other banks y.
template <int CTRL, int XB>
__device__ __forceinline__ uint32_t fold_banks(uint32_t x, uint32_t y) {
  const uint32_t a = (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)y, CTRL, 0xF, 0xF ^ XB, false);
  const uint32_t b = (uint32_t)__builtin_amdgcn_update_dpp((int)y, (int)x, CTRL, 0xF, XB, false);
  return pk_max_u16(a, b);
}

// Row maxima of a chunk of 16 key rows and 16 value rows, from their pair
// words (kp[i], vp[i]: pair_max_u16 of rows 2i and 2i + 1, every lane of the
// wave active), by a reduce-scatter instead of one all-reduce per word: two
// lane-half swaps, one row swap, two bank folds and a 4-lane all-reduce for
// the 16 words, after which lane 16 rho + 4 beta + q (q = 0..3) holds the
// wave maxima of pair i = 4 (beta >> 1) + fold_row(rho) of the keys (beta
// even) or values (beta odd): low half row 2i, high half row 2i + 1.
// fold_row: 0, 2, 1, 3 (the row swap's order; its own inverse).
__device__ __forceinline__ int fold_row(int rho) { return ((rho & 1) << 1) | (rho >> 1); }
__device__ __forceinline__ int fold_lane(bool value, int i) { return 16 * fold_row(i & 3) + 8 * (i >> 2) + 4 * value; }
__device__ __forceinline__ uint32_t chunk_row_maxima(const uint32_t (&kp)[8], const uint32_t (&vp)[8]) {
  uint32_t bk[2], bv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    bk[j] = fold16(fold32(kp[4 * j], kp[4 * j + 1]), fold32(kp[4 * j + 2], kp[4 * j + 3]));
    bv[j] = fold16(fold32(vp[4 * j], vp[4 * j + 1]), fold32(vp[4 * j + 2], vp[4 * j + 3]));
  }
  // rows of bk[j] / bv[j]: pairs 4j + (0, 2, 1, 3), each still over 16 lanes
  const uint32_t ck = fold_banks<0x140, 0x3>(bk[0], bk[1]);    // row_mirror: lanes 0-7 bk[0], 8-15 bk[1]
  const uint32_t cv = fold_banks<0x140, 0x3>(bv[0], bv[1]);
  uint32_t d = fold_banks<0x141, 0x5>(ck, cv);                 // row_half_mirror: banks 0, 2 keys, 1, 3 values
  d = pk_max_u16(d, (uint32_t)__builtin_amdgcn_mov_dpp((int)d, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  return pk_max_u16(d, (uint32_t)__builtin_amdgcn_mov_dpp((int)d, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
}

// A row's scale RN(amax / 448) and the reciprocal bracket used to code its
// elements: x lo and x hi lie below and above the correctly rounded quotient
// x / s (the reciprocal is within 1 ulp; the bracket is 2^-20 either side of
// it, the products' rounding adds 2^-24 each), scales from 2^-100 up. Rows
// with smaller scales (and rows of zeros, scale 0) get lo = -1: every element
// of theirs is coded by the division.
__device__ __forceinline__ void row_bracket(uint32_t amax_bf16, float& s, float& lo, float& hi) {
  s = row_scale(__uint_as_float(amax_bf16 << 16));
  const float r = __builtin_amdgcn_rcpf(s);
  lo = s >= 0x1p-100f ? r * (1.f - 0x1p-20f) : -1.f;
  hi = r * (1.f + 0x1p-20f);
}
// Codes of the bf16 pair w (bits 0-7: the low channel) in a row with bracket
// lo / hi (row_bracket; wave-uniform values) whose scale is s_lanes in lane
// `src`: rounding to E4M3 is monotone, so when x lo and x hi take the same
// code the correctly rounded quotient between them takes it too; otherwise
// (within 2^-20 of a rounding boundary: rare), and in rows with lo < 0, the
// division decides. A row of zeros codes to 0. Equal to e4m3_code(x / s)
// for every bf16 row maximum and every bf16 x up to it (checked over all
// pairs).
__device__ __forceinline__ uint32_t codes_bracketed(uint32_t w, float lo, float hi, float s_lanes, int src) {
  const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xFFFF0000u);
  const uint32_t a = e4m3_code2(x0 * lo, x1 * lo), b = e4m3_code2(x0 * hi, x1 * hi);
  uint32_t c = a;
  if ((a != b) | (__float_as_int(lo) < 0)) {
    const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_lanes), src));
    c = s == 0.f ? 0u : e4m3_code2(x0 / s, x1 / s);
  }
  return c;
}
// A wave-uniform copy of lane `src`'s value.
__device__ __forceinline__ float lane_value(float x, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
}

// Running channel-wise min / max of the dequantized keys of the lane's two
// channels (codes in bits 0-7 / 8-15 of c2), in IEEE totalOrder (-0 below
// +0, the order of the bf16 summaries): the fp32 neighbours of each exact
// product as keys (product_keys), rounded outward to bf16 once, when stored.
// Both roundings are monotone in that order, so this is the exact min / max
// rounded outward.
struct MinMax2 {
  uint32_t lo0 = 0xFFFFFFFFu, hi0 = 0u, lo1 = 0xFFFFFFFFu, hi1 = 0u;
  __device__ __forceinline__ void add(uint32_t c2, float scale) {
    const e4m3_pair_values v = e4m3_value2(c2);
    uint32_t kd, ku;
    product_keys(v[0], scale, kd, ku);
    lo0 = min(lo0, kd);
    hi0 = max(hi0, ku);
    product_keys(v[1], scale, kd, ku);
    lo1 = min(lo1, kd);
    hi1 = max(hi1, ku);
  }
  // the summary rows of the page
  __device__ __forceinline__ void store(uint16_t* summ_page_base, int lane) const {
    uint32_t* sp = reinterpret_cast<uint32_t*>(summ_page_base);
    sp[lane] = bf16_below_key(lo0) | (bf16_below_key(lo1) << 16);
    sp[kHeadDim / 2 + lane] = bf16_above_key(hi0) | (bf16_above_key(hi1) << 16);
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
  const e4m3_pair_values v = e4m3_value2(c2);
  uint32_t kd0, ku0, kd1, ku1;
  product_keys(v[0], scale, kd0, ku0);
  product_keys(v[1], scale, kd1, ku1);
  const uint32_t dn0 = bf16_below_key(kd0), up0 = bf16_above_key(ku0);
  const uint32_t dn1 = bf16_below_key(kd1), up1 = bf16_above_key(ku1);
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
