// Probabilities split into bf16 high and low parts, the B operands of the P V
// MFMAs (P V = V hi + V lo, exact to about 2^-17 of each probability).
// Device code only (included by the kernel files).
#pragma once

#include <hip/hip_runtime.h>

namespace spa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// hi = RNE_bf16(p), lo = RNE_bf16(p - hi) for two probabilities. p - hi is
// exact in fp32 (at most 17 significant bits) and comes from one dot
// instruction per probability: (hi0, hi1) . (-1, 0) + p0 and (hi0, hi1) .
// (0, -1) + p1, whose products and sum are exact (checked against the plain
// subtraction over every normal fp32 value up to 2^9). The two constant
// pairs come from registers: written as an instruction's inline constant,
// -1.0 would fill both halves of the pair.
__device__ __forceinline__ void split_pair(float p0, float p1, bf16x2_t& hi, bf16x2_t& lo) {
  const f32x2_t v = {p0, p1};
  hi = __builtin_convertvector(v, bf16x2_t);
  uint32_t w0 = 0x0000BF80u, w1 = 0xBF800000u;     // (-1, 0) and (0, -1) as bf16 pairs
  asm("" : "+v"(w0), "+v"(w1));                   // opaque, so kept in registers (and hoisted)
  bf16x2_t m0, m1;
  __builtin_memcpy(&m0, &w0, 4);
  __builtin_memcpy(&m1, &w1, 4);
  const f32x2_t rest = {__builtin_amdgcn_fdot2_f32_bf16(hi, m0, p0, false),
                        __builtin_amdgcn_fdot2_f32_bf16(hi, m1, p1, false)};
  lo = __builtin_convertvector(rest, bf16x2_t);
}

}  // namespace spa
