// Exhaustive check of the fp8 quantizer's fast steps in
// sparse_paged_attention_amd/csrc/pool_rows.h against their plain forms, on the
// GPU they run on (test program; the product library does not contain it):
//   1. e4m3_code2 (the hardware conversion) vs e4m3_code (from the fp32 bit
//      pattern), every fp32 value of magnitude <= 464, both signs, both bytes;
//   2. for every bf16 row maximum a and every bf16 x with |x| <= a, both signs:
//      row_bracket(a)'s scale vs the IEEE division a / 448, codes_bracketed
//      (reciprocal bracket) and quantize_pair (whole-wave row) vs
//      e4m3_code(x / s);
//   3. product_keys + bf16_below_key / bf16_above_key vs bf16_down / bf16_up of
//      the fp64 product, every code and every such scale; e4m3_value2 vs
//      e4m3_value, every code;
//   4. wave_max_u32, and pair_max_u16 + chunk_row_maxima (the reduce-scatter of
//      16 key and 16 value rows, with its lane map fold_lane) vs serial maxima
//      on seeded rows;
//   5. codes_bf16x2 (the scaled conversion the attention kernels decode codes
//      with) vs the bf16 bits of e4m3_value, every pair of codes, both halves
//      of the word;
//   6. split_pair (psplit.h: p - hi by one dot instruction) vs the plain
//      subtraction, every normal fp32 p below 2^9 in both slots.
// Prints one line per check with its mismatch count; exit status 0 when all are 0.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
#include "pool_rows.h"
#include "psplit.h"
using namespace spa;

constexpr int kChecks = 11;

__device__ void report(unsigned long long* cnt, uint32_t* first, int which, uint32_t a, uint32_t b, uint32_t c) {
  const unsigned long long k = atomicAdd(&cnt[which], 1ull);
  if (k < 4) {
    uint32_t* f = first + (which * 4 + k) * 3;
    f[0] = a; f[1] = b; f[2] = c;
  }
}

__global__ void check_conversion(uint32_t n, unsigned long long* cnt, uint32_t* first) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const float y = __uint_as_float(i), z = -y;
    const uint32_t hw = e4m3_code2(y, z), sw = e4m3_code(y) | (e4m3_code(z) << 8);
    if (hw != sw) report(cnt, first, 0, i, hw, sw);
  }
}

// one block per row maximum a (bf16 bits 0 .. 0x7F7F; 0: a row of zeros)
__global__ void __launch_bounds__(256) check_rows(unsigned long long* cnt, uint32_t* first) {
  const uint32_t abits = blockIdx.x;
  const float a = __uint_as_float(abits << 16);
  const float s = a / 448.f;
  float rs, lo, hi;                                 // the same in every lane (one maximum per block)
  row_bracket(abits, rs, lo, hi);
  if (threadIdx.x == 0 && __float_as_uint(rs) != __float_as_uint(s)) report(cnt, first, 1, abits, __float_as_uint(rs), __float_as_uint(s));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t n = abits + 1;                     // x patterns 0 .. abits
  // codes_bracketed: any thread, any x (the scale read from lane 0)
  for (uint32_t xb0 = wave * 64; xb0 < n; xb0 += blockDim.x) {
    const uint32_t xb = min(xb0 + (uint32_t)lane, abits);
    const uint32_t w = (xb << 16) | (xb | 0x8000u);  // channel 0: -x, channel 1: +x
    const float x = __uint_as_float(xb << 16);
    const uint32_t want = s == 0.f ? 0u : (e4m3_code(-x / s) | (e4m3_code(x / s) << 8));
    const uint32_t got = codes_bracketed(w, lane_value(lo, 0), lane_value(hi, 0), rs, 0);
    if (got != want) report(cnt, first, 2, abits, xb, got);
  }
  // quantize_pair: whole waves; lane 0 carries the maximum, lanes 1-63 the x values
  for (uint32_t base = wave * 63; base < n; base += 4 * 63) {
    const uint32_t xb = lane == 0 ? abits : min(base + (uint32_t)lane - 1u, abits);
    const uint32_t w = (xb << 16) | (xb | 0x8000u);
    float sq;
    const uint32_t got = quantize_pair(w, sq);
    const float x = __uint_as_float(xb << 16);
    const uint32_t want = s == 0.f ? 0u : (e4m3_code(-x / s) | (e4m3_code(x / s) << 8));
    if (got != want || __float_as_uint(sq) != __float_as_uint(s)) report(cnt, first, 3, abits, xb, got);
  }
}

__global__ void check_products(unsigned long long* cnt, uint32_t* first) {
  const uint32_t abits = blockIdx.x;
  const float s = __uint_as_float(abits << 16) / 448.f;
  for (uint32_t c = threadIdx.x; c < 256; c += blockDim.x) {
    if ((c & 0x7Fu) == 0x7Fu) continue;             // the NaN codes
    const float v = e4m3_value(c);
    const float v2 = e4m3_value2(c | (c << 8))[1];
    if (__float_as_uint(v2) != __float_as_uint(v)) report(cnt, first, 4, abits, c, __float_as_uint(v2));
    const double x = (double)v * (double)s;
    uint32_t kd, ku;
    product_keys(v, s, kd, ku);
    if (bf16_below_key(kd) != bf16_down(x)) report(cnt, first, 5, abits, c, bf16_below_key(kd));
    if (bf16_above_key(ku) != bf16_up(x)) report(cnt, first, 6, abits, c, bf16_above_key(ku));
  }
}

__global__ void __launch_bounds__(64) check_maxima(unsigned long long* cnt, uint32_t* first) {
  uint32_t st = blockIdx.x * 2654435761u + threadIdx.x * 40503u + 12345u;
  st ^= st << 13; st ^= st >> 17; st ^= st << 5;
  const uint32_t w0 = st >> (blockIdx.x & 7);
  const uint32_t m32 = wave_max_u32(w0);
  // 16 key rows and 16 value rows of seeded bf16 pairs, magnitudes of a
  // different range in each row
  uint32_t rows[32];
  for (int u = 0; u < 32; ++u) {
    st ^= st << 13; st ^= st >> 17; st ^= st << 5;
    rows[u] = st >> ((u * 7 + blockIdx.x) & 15);
  }
  uint32_t kp[8], vp[8];
  for (int i = 0; i < 8; ++i) {
    kp[i] = pair_max_u16(rows[2 * i], rows[2 * i + 1]);
    vp[i] = pair_max_u16(rows[16 + 2 * i], rows[16 + 2 * i + 1]);
  }
  const uint32_t m = chunk_row_maxima(kp, vp);
  __shared__ uint32_t sh[33][64];
  sh[0][threadIdx.x] = w0;
  for (int u = 0; u < 32; ++u) sh[1 + u][threadIdx.x] = rows[u];
  __syncthreads();
  uint32_t r = 0;
  for (int i = 0; i < 64; ++i) r = max(r, sh[0][i]);
  if (m32 != r) report(cnt, first, 7, blockIdx.x, threadIdx.x, m32);
  // the pair this lane holds, and the lane the kernel reads it from
  const int lane = threadIdx.x, rho = lane >> 4, beta = (lane >> 2) & 3;
  const int tau = beta & 1, i = 4 * (beta >> 1) + fold_row(rho);
  uint32_t want = 0;
  for (int hh = 0; hh < 2; ++hh) {
    uint32_t mx = 0;
    for (int l = 0; l < 64; ++l) {
      const uint32_t x = sh[1 + 16 * tau + 2 * i + hh][l];
      mx = max(mx, max(x & 0x7FFFu, (x >> 16) & 0x7FFFu));
    }
    want |= mx << (16 * hh);
  }
  if (m != want || fold_lane(tau != 0, i) != (lane & ~3)) report(cnt, first, 8, blockIdx.x, threadIdx.x, m);
}

// one thread per pair of codes (bits 0-15); NaN codes skipped
__global__ void check_decode(unsigned long long* cnt, uint32_t* first) {
  const uint32_t c2 = blockIdx.x * blockDim.x + threadIdx.x;
  if (c2 > 0xFFFFu) return;
  const uint32_t c0 = c2 & 0xFFu, c1 = c2 >> 8;
  if ((c0 & 0x7Fu) == 0x7Fu || (c1 & 0x7Fu) == 0x7Fu) return;
  const uint32_t want = (__float_as_uint(e4m3_value(c0)) >> 16) | (__float_as_uint(e4m3_value(c1)) & 0xFFFF0000u);
  const uint32_t lo = codes_bf16x2<false>(c2 | 0xA5A50000u);   // the other half holds codes that must not leak in
  const uint32_t hi = codes_bf16x2<true>((c2 << 16) | 0x5A5Au);
  if (lo != want) report(cnt, first, 9, c2, lo, want);
  if (hi != want) report(cnt, first, 9, c2 | 0x10000u, hi, want);
}

// every normal fp32 p in [2^-126, 2^9): in slot 0, and mirrored in slot 1
__global__ void check_split(unsigned long long* cnt, uint32_t* first) {
  constexpr uint32_t kLo = 0x00800000u, kHi = 0x44000000u;
  for (uint32_t u = kLo + blockIdx.x * blockDim.x + threadIdx.x; u < kHi; u += gridDim.x * blockDim.x) {
    const float p0 = __uint_as_float(u), p1 = __uint_as_float(kLo + (kHi - 1u - u));
    bf16x2_t hi, lo;
    split_pair(p0, p1, hi, lo);
    const f32x2_t v = {p0, p1};
    const bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    const f32x2_t rest = v - __builtin_convertvector(h, f32x2_t);
    const bf16x2_t l = __builtin_convertvector(rest, bf16x2_t);
    uint32_t gh, gl, wh, wl;
    __builtin_memcpy(&gh, &hi, 4); __builtin_memcpy(&gl, &lo, 4);
    __builtin_memcpy(&wh, &h, 4); __builtin_memcpy(&wl, &l, 4);
    if (gh != wh || gl != wl) report(cnt, first, 10, u, gl, wl);
  }
}

int main() {
  unsigned long long* cnt;
  uint32_t* first;
  if (hipMalloc(&cnt, kChecks * sizeof(unsigned long long)) != hipSuccess) return 2;
  if (hipMalloc(&first, kChecks * 4 * 3 * sizeof(uint32_t)) != hipSuccess) return 2;
  if (hipMemset(cnt, 0, kChecks * sizeof(unsigned long long)) != hipSuccess) return 2;
  if (hipMemset(first, 0, kChecks * 4 * 3 * sizeof(uint32_t)) != hipSuccess) return 2;
  hipLaunchKernelGGL(check_conversion, dim3(8192), dim3(256), 0, 0, 0x43E80001u, cnt, first);   // |y| <= 464
  hipLaunchKernelGGL(check_rows, dim3(0x7F80), dim3(256), 0, 0, cnt, first);
  hipLaunchKernelGGL(check_products, dim3(0x7F80), dim3(256), 0, 0, cnt, first);
  hipLaunchKernelGGL(check_maxima, dim3(65536), dim3(64), 0, 0, cnt, first);
  hipLaunchKernelGGL(check_decode, dim3(256), dim3(256), 0, 0, cnt, first);
  hipLaunchKernelGGL(check_split, dim3(8192), dim3(256), 0, 0, cnt, first);
  const hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    printf("hip error: %s\n", hipGetErrorString(e));
    return 2;
  }
  unsigned long long h[kChecks];
  uint32_t f[kChecks * 4 * 3];
  if (hipMemcpy(h, cnt, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return 2;
  if (hipMemcpy(f, first, sizeof f, hipMemcpyDeviceToHost) != hipSuccess) return 2;
  const char* names[kChecks] = {
      "hardware E4M3 conversion vs e4m3_code, all fp32 |y| <= 464",
      "row_bracket's scale vs a / 448, all bf16 a",
      "codes_bracketed vs e4m3_code(x / s), all bf16 pairs",
      "quantize_pair vs e4m3_code(x / s), all bf16 pairs",
      "e4m3_value2 vs e4m3_value, all codes",
      "bf16 below the product vs fp64, all codes x scales",
      "bf16 above the product vs fp64, all codes x scales",
      "wave_max_u32, seeded rows",
      "pair_max_u16 + chunk_row_maxima and its lane map, seeded rows",
      "codes_bf16x2 (scaled conversion) vs e4m3_value, all code pairs, both halves",
      "split_pair (dot instruction) vs the plain subtraction, all normal fp32 p < 2^9"};
  int bad = 0;
  for (int w = 0; w < kChecks; ++w) {
    printf("%s: %llu mismatches\n", names[w], h[w]);
    bad |= h[w] != 0;
    for (unsigned k = 0; k < 4 && k < h[w]; ++k)
      printf("  %08x %08x %08x\n", f[(w * 4 + k) * 3], f[(w * 4 + k) * 3 + 1], f[(w * 4 + k) * 3 + 2]);
  }
  return bad;
}
