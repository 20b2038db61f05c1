// ft_quant_block16: 16x16 block quantizer to E2M1 codes + one scale per block.
//
// FourTune, section 3.1 (the quantizer Q(.) after Eq. 2, offline for R and
// dynamic for X and G) and section 3.2 (16x16 blocks, so one scale grid serves
// the matrix and its transpose).  Scale = block amax / 6 (power-of-two rounded
// up, or fp32), element code = round-to-nearest-even E2M1 of x / scale.
//
// One workgroup quantizes a 128x128 tile: the bf16 tile is read once from HBM
// with fully coalesced 16-byte loads into LDS; each lane then owns one 16-element
// row segment of one 16x16 block (16 lanes per block), reduces the block maximum
// across its 16 lanes, converts with the hardware scaled E2M1 convert (which
// rounds to nearest-even and saturates, matching the oracle bit for bit), and
// transposes the 16x16 nibble block across the 16 lanes for the column-major
// codes.  Both code layouts are staged in LDS and written with coalesced stores.
#include "ft_common.h"

namespace ft {
namespace {

constexpr int QT = 128;                 // tile edge (elements)
constexpr int QTHREADS = 256;
constexpr int IN_PITCH = QT * 2 + 16;   // bytes per LDS input row (padded)
constexpr int RM_PITCH = QT / 2 + 8;    // bytes per LDS row-major code row (padded)
constexpr int CM_PITCH = QT / 2 + 8;    // bytes per LDS column-major code row (padded)

// Exchange with the lane whose index differs in bit MASK (MASK < 16).
template <int MASK>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  return (uint32_t)__shfl_xor((int)v, MASK, 64);
}

// E = min{e : 6 * 2^e >= a} clamped to [-127, 127], from the bf16 magnitude bits a.
// a = 1.f * 2^q with 7-bit mantissa f: E = q - 2 when f <= 0.5 (1.f <= 1.5), else q - 1.
__device__ __forceinline__ int pow2_exponent(uint32_t a) {
  int e = (int)(a >> 7);
  if (e == 0) return -127;  // zero or subnormal maximum: 6 * 2^-127 covers it
  int E = (e - 127) - 2 + ((a & 0x7f) > 0x40 ? 1 : 0);
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// Transpose a 16x16 block of nibbles held one row per lane (64 bits: positions
// = columns) so that lane i ends up with column i (positions = rows).  Step b
// swaps bit b of the lane index with bit b of the nibble position.
__device__ __forceinline__ void transpose_nibbles16(uint32_t& w0, uint32_t& w1, int i) {
  {  // bit 3: dword halves
    uint32_t send = (i & 8) ? w0 : w1;
    uint32_t recv = xor_lane<8>(send);
    if (i & 8) w0 = recv; else w1 = recv;
  }
#define FT_NIB_STEP(BIT, SHIFT, M0)                                           \
  {                                                                           \
    uint32_t r0 = xor_lane<BIT>(w0), r1 = xor_lane<BIT>(w1);                  \
    if (i & BIT) {                                                            \
      w0 = (w0 & ~(M0)) | ((r0 & ~(M0)) >> SHIFT);                            \
      w1 = (w1 & ~(M0)) | ((r1 & ~(M0)) >> SHIFT);                            \
    } else {                                                                  \
      w0 = (w0 & (M0)) | ((r0 & (M0)) << SHIFT);                              \
      w1 = (w1 & (M0)) | ((r1 & (M0)) << SHIFT);                              \
    }                                                                         \
  }
  FT_NIB_STEP(4, 16, 0x0000FFFFu)
  FT_NIB_STEP(2, 8, 0x00FF00FFu)
  FT_NIB_STEP(1, 4, 0x0F0F0F0Fu)
#undef FT_NIB_STEP
}

template <bool POW2, bool WRITE_RM, bool WRITE_CM>
__global__ void __launch_bounds__(QTHREADS)
quant_block16_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                     uint8_t* __restrict__ codes_rm, uint8_t* __restrict__ codes_cm,
                     void* __restrict__ scales, void* __restrict__ scales_cm) {
  __shared__ __attribute__((aligned(16))) uint8_t s_in[QT * IN_PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t s_rm[WRITE_RM ? QT * RM_PITCH : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_cm[WRITE_CM ? QT * CM_PITCH : 16];

  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.y * QT;
  const int64_t col0 = (int64_t)blockIdx.x * QT;
  const int trows = (int)min<int64_t>(QT, rows - row0);   // multiple of 16
  const int tcols = (int)min<int64_t>(QT, cols - col0);   // multiple of 16

  // 1. HBM -> LDS, 16-byte chunks; 16 lanes cover one 256-byte tile row.
#pragma unroll
  for (int it = 0; it < (QT * QT * 2 / 16) / QTHREADS; ++it) {
    int c = it * QTHREADS + tid;
    int r = c >> 4, q = c & 15;
    v4i v = {0, 0, 0, 0};
    if (r < trows && q * 8 < tcols)
      v = *reinterpret_cast<const v4i*>(x + (row0 + r) * ldx + col0 + q * 8);
    *reinterpret_cast<v4i*>(s_in + r * IN_PITCH + q * 16) = v;
  }
  __syncthreads();

  // 2. one 16-element row segment of one block per lane, 4 segments per lane.
  const int i = tid & 15;              // row inside the block
#pragma unroll
  for (int it = 0; it < (QT / 16) * (QT / 16) * 16 / QTHREADS; ++it) {
    const int b = it * (QTHREADS / 16) + (tid >> 4);   // block index in the tile
    const int br = b >> 3, bc = b & 7;                 // 8x8 blocks per tile
    const bool live = (br * 16 < trows) && (bc * 16 < tcols);  // uniform over the 16 lanes
    const uint8_t* src = s_in + (br * 16 + i) * IN_PITCH + bc * 32;
    v4i p0 = *reinterpret_cast<const v4i*>(src);
    v4i p1 = *reinterpret_cast<const v4i*>(src + 16);
    uint32_t d[8] = {(uint32_t)p0.x, (uint32_t)p0.y, (uint32_t)p0.z, (uint32_t)p0.w,
                     (uint32_t)p1.x, (uint32_t)p1.y, (uint32_t)p1.z, (uint32_t)p1.w};
    // block maximum of |x| on the bf16 bit patterns (magnitude order = integer order)
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t lo = d[k] & 0x7fffu, hi = (d[k] >> 16) & 0x7fffu;
      m = max(m, max(lo, hi));
    }
    m = max(m, xor_lane<8>(m));
    m = max(m, xor_lane<4>(m));
    m = max(m, xor_lane<2>(m));
    m = max(m, xor_lane<1>(m));

    uint32_t w0 = 0, w1 = 0;
    if constexpr (POW2) {
      const int E = pow2_exponent(m);
      const float sc = __builtin_bit_cast(float, (uint32_t)(E + 127) << 23);  // 2^E as the E8M0 operand
#define FT_CVT(W, K, SEL) W = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(W, bf16lo_to_f32(d[K]), bf16hi_to_f32(d[K]), sc, SEL)
      FT_CVT(w0, 0, 0); FT_CVT(w0, 1, 1); FT_CVT(w0, 2, 2); FT_CVT(w0, 3, 3);
      FT_CVT(w1, 4, 0); FT_CVT(w1, 5, 1); FT_CVT(w1, 6, 2); FT_CVT(w1, 7, 3);
#undef FT_CVT
      if (live && i == 0) {
        static_cast<uint8_t*>(scales)[(row0 / 16 + br) * (cols / 16) + col0 / 16 + bc] = (uint8_t)(E + 127);
        if (scales_cm)
          static_cast<uint8_t*>(scales_cm)[(col0 / 16 + bc) * (rows / 16) + row0 / 16 + br] = (uint8_t)(E + 127);
      }
    } else {
      const float amax = __builtin_bit_cast(float, m << 16);
      const float s = amax / 6.0f;                       // IEEE binary32 division
      const bool zero = (s == 0.0f);
      float v[16];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float a = bf16lo_to_f32(d[k]), c = bf16hi_to_f32(d[k]);
        v[2 * k] = zero ? a * 0.0f : a / s;               // ratio fl32(x / s); +-0 for a zero block
        v[2 * k + 1] = zero ? c * 0.0f : c / s;
      }
#define FT_CVT(W, K, SEL) W = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(W, v[2 * (K)], v[2 * (K) + 1], 1.0f, SEL)
      FT_CVT(w0, 0, 0); FT_CVT(w0, 1, 1); FT_CVT(w0, 2, 2); FT_CVT(w0, 3, 3);
      FT_CVT(w1, 4, 0); FT_CVT(w1, 5, 1); FT_CVT(w1, 6, 2); FT_CVT(w1, 7, 3);
#undef FT_CVT
      if (live && i == 0) {
        static_cast<float*>(scales)[(row0 / 16 + br) * (cols / 16) + col0 / 16 + bc] = s;
        if (scales_cm) static_cast<float*>(scales_cm)[(col0 / 16 + bc) * (rows / 16) + row0 / 16 + br] = s;
      }
    }
    if constexpr (WRITE_RM) {
      *reinterpret_cast<v2i*>(s_rm + (br * 16 + i) * RM_PITCH + bc * 8) = v2i{(int)w0, (int)w1};
    }
    if constexpr (WRITE_CM) {
      transpose_nibbles16(w0, w1, i);
      *reinterpret_cast<v2i*>(s_cm + (bc * 16 + i) * CM_PITCH + br * 8) = v2i{(int)w0, (int)w1};
    }
  }
  __syncthreads();

  // 3. LDS -> HBM, 8-byte stores; 8 lanes cover one 64-byte code row.
  if constexpr (WRITE_RM) {
#pragma unroll
    for (int it = 0; it < (QT * QT / 2 / 8) / QTHREADS; ++it) {
      int c = it * QTHREADS + tid;
      int r = c >> 3, q = c & 7;
      if (r < trows && q * 16 < tcols)
        *reinterpret_cast<v2i*>(codes_rm + (row0 + r) * (cols / 2) + col0 / 2 + q * 8) =
            *reinterpret_cast<const v2i*>(s_rm + r * RM_PITCH + q * 8);
    }
  }
  if constexpr (WRITE_CM) {
#pragma unroll
    for (int it = 0; it < (QT * QT / 2 / 8) / QTHREADS; ++it) {
      int c = it * QTHREADS + tid;
      int cl = c >> 3, q = c & 7;
      if (cl < tcols && q * 16 < trows)
        *reinterpret_cast<v2i*>(codes_cm + (col0 + cl) * (rows / 2) + row0 / 2 + q * 8) =
            *reinterpret_cast<const v2i*>(s_cm + cl * CM_PITCH + q * 8);
    }
  }
}

template <bool POW2>
ft_status launch_quant(const void* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* rm,
                       uint8_t* cm, void* scales, void* scales_cm, hipStream_t s) {
  dim3 grid((unsigned)((cols + QT - 1) / QT), (unsigned)((rows + QT - 1) / QT));
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (rm && cm)
    hipLaunchKernelGGL((quant_block16_kernel<POW2, true, true>), grid, dim3(QTHREADS), 0, s, xp, rows, cols, ldx, rm, cm, scales, scales_cm);
  else if (rm)
    hipLaunchKernelGGL((quant_block16_kernel<POW2, true, false>), grid, dim3(QTHREADS), 0, s, xp, rows, cols, ldx, rm, cm, scales, scales_cm);
  else
    hipLaunchKernelGGL((quant_block16_kernel<POW2, false, true>), grid, dim3(QTHREADS), 0, s, xp, rows, cols, ldx, rm, cm, scales, scales_cm);
  return launch_status();
}

}  // namespace
}  // namespace ft

extern "C" ft_status ft_quant_block16(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                                      ft_scale_mode mode, uint8_t* codes_rm, uint8_t* codes_cm,
                                      void* scales, void* scales_cm, hipStream_t stream) {
  using namespace ft;
  if (mode != FT_SCALE_POW2 && mode != FT_SCALE_F32) return FT_EINVAL;
  if (!mult16(rows) || !mult16(cols) || ldx < cols) return FT_ESHAPE;
  if (rows == 0 || cols == 0) return FT_OK;
  if (!x || !scales || (!codes_rm && !codes_cm)) return FT_EINVAL;
  if (!aligned16(x) || (ldx % 8) != 0) return FT_EALIGN;
  if ((codes_rm && !aligned16(codes_rm)) || (codes_cm && !aligned16(codes_cm)) || !aligned16(scales) ||
      (scales_cm && !aligned16(scales_cm)))
    return FT_EALIGN;
  if (rows / QT >= 65535) return FT_ESHAPE;
  return mode == FT_SCALE_POW2 ? launch_quant<true>(x, rows, cols, ldx, codes_rm, codes_cm, scales, scales_cm, stream)
                               : launch_quant<false>(x, rows, cols, ldx, codes_rm, codes_cm, scales, scales_cm, stream);
}

extern "C" const char* ft_status_str(ft_status s) {
  switch (s) {
    case FT_OK: return "ok";
    case FT_EINVAL: return "invalid argument (null pointer or unknown enum)";
    case FT_ESHAPE: return "bad shape (dimension not a multiple of 16, or ranks out of range)";
    case FT_EALIGN: return "misaligned pointer or leading dimension (16-byte alignment required)";
    case FT_EHIP: return "HIP launch failed";
    case FT_ENOTSUP: return "not supported by this build";
    case FT_ESPACE: return "workspace too small";
  }
  return "unknown status";
}
