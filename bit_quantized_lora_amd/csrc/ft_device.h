// Device helpers shared by several kernels of the ft library (gfx950 / CDNA4).
#pragma once

#include "ft_common.h"

namespace ft {

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// GELU between the two linears of an MLP block (FourTune section 3.3 "MLP
// Fusion" names the activation; the exact form x * Phi(x) with the error
// function is used).  Phi(x) = erfc(-x / sqrt 2) / 2 for x < 0 (no cancellation in
// the small tail) and 1 - erfc(x / sqrt 2) / 2 for x >= 0.  erfc(z), z >= 0, by
// the Chebyshev fit of Numerical Recipes (Press et al., section 6.2, "erfcc"):
// t = 1 / (1 + z/2), erfc(z) = t exp(-z^2 + P(t)) with a degree-9 polynomial P,
// fractional error below 1.2e-7 everywhere -- about one fp32 ulp, against the
// 2^-9 spacing of the bf16 result -- at a third of the cost of the library erfc.
__device__ __forceinline__ float erfc_nonneg(float z) {
  const float t = 1.0f / (1.0f + 0.5f * z);
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.26551223f);
  return t * __expf(fmaf(-z, z, p));
}
__device__ __forceinline__ float norm_cdf(float x) {
  const float e = 0.5f * erfc_nonneg(fabsf(x) * 0.70710678118654752f);
  return x < 0.0f ? e : 1.0f - e;
}
__device__ __forceinline__ float gelu_f(float x) { return x * norm_cdf(x); }
__device__ __forceinline__ float gelu_grad_f(float x) {
  const float cdf = norm_cdf(x);
  const float pdf = 0.39894228040143268f * __expf(-0.5f * x * x);
  return cdf + x * pdf;
}

// Power-of-two block scale (FourTune section 3.2, 16x16 blocks; the scale rule of
// amax / 6 rounded up to a power of two):  E = min{e : 6 * 2^e >= a} clamped to
// [-127, 127], from the bf16 magnitude bits a of the block maximum.
// a = 1.f * 2^q with 7-bit mantissa f: E = q - 2 when f <= 0.5 (1.f <= 1.5), else q - 1.
__device__ __forceinline__ int pow2_exp_bf16(uint32_t a) {
  const int e = (int)(a >> 7);
  if (e == 0) return -127;  // zero or subnormal maximum: 6 * 2^-127 covers it
  const int E = (e - 127) - 2 + ((a & 0x7f) > 0x40 ? 1 : 0);
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// 16-lane maximum inside each DPP row (quad xor 1, xor 2, half-row mirror, row mirror)
__device__ __forceinline__ uint32_t dpp_max16(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));
  return v;
}

}  // namespace ft
