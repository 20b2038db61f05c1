// Shared device/host helpers of the ft library (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ft.h"

namespace ft {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ---- host-side validation helpers -------------------------------------------------
static inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static inline bool mult16(int64_t v) { return v >= 0 && (v % 16) == 0; }

static inline ft_status launch_status() {
  return hipGetLastError() == hipSuccess ? FT_OK : FT_EHIP;
}

// ---- device helpers ------------------------------------------------------------------
__device__ __forceinline__ float bf16lo_to_f32(uint32_t packed) { return __builtin_bit_cast(float, packed << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t packed) { return __builtin_bit_cast(float, packed & 0xffff0000u); }

// round-to-nearest-even fp32 -> bf16 bits (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 values split into bf16 hi + lo: hi = rne(f), lo = rne(f - hi), each
// pair packed into a dword (element 0 in the low half).  hi + lo equals f to
// within 2^-16 relative (16 significant bits).  The conversions are the
// hardware's packed fp32 -> bf16 (round to nearest even: the same bits as
// f32_to_bf16_rne for finite values), two values per instruction.
typedef float v2f_ __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_ __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_bf16x2(float f0, float f1, uint32_t& hi, uint32_t& lo) {
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_){f0, f1}, v2bf_));
  const float h0 = __builtin_bit_cast(float, h << 16), h1 = __builtin_bit_cast(float, h & 0xffff0000u);
  hi = h;
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_){f0 - h0, f1 - h1}, v2bf_));
}
// one value: hi, lo in the low 16 bits
__device__ __forceinline__ void split_bf16(float f, uint32_t& hi, uint32_t& lo) {
  split_bf16x2(f, 0.0f, hi, lo);
  hi &= 0xffffu;
  lo &= 0xffffu;
}

// Zero n floats on the stream with a kernel (graph-capture friendly, no memset node).
ft_status fill_zero_f32(float* p, int64_t n, hipStream_t s);

}  // namespace ft
