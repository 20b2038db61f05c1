// ft_quant_block16: 16x16 block quantizer to E2M1 codes + one scale per block.
//
// FourTune, section 3.1 (the quantizer Q(.) after Eq. 2, offline for R and
// dynamic for X and G) and section 3.2 (16x16 blocks, so one scale grid serves
// the matrix and its transpose).  Scale = block amax / 6 (power-of-two rounded
// up, or fp32), element code = round-to-nearest-even E2M1 of x / scale.
//
// One workgroup quantizes a 128x128 tile: the bf16 tile is read once from HBM
// straight into registers (each lane owns one 16-element row segment of one
// 16x16 block per pass, 16 lanes per block; a wave's 4 blocks are adjacent, so
// its loads cover 16 rows x 128 contiguous bytes), reduces the block maximum
// across its 16 lanes, converts with the hardware scaled E2M1 convert from bf16
// (which rounds to nearest-even and saturates, matching the oracle bit for bit), and
// transposes the 16x16 nibble block across the 16 lanes for the column-major
// codes.  Both code layouts are staged in LDS and written with coalesced stores.
//
// Optionally the same tile also writes the pair-merged GEMM operand of Q(x)
// (along columns) and of Q(x)^T (along rows): a value-preserving re-encoding in
// which the two 16-wide blocks of a 32-wide pair share one power-of-two scale,
// so one 32-value fragment of the block-scaled MFMA carries both blocks.  The
// elements become FP6 E3M2: a block with scale byte e_b is re-expressed at the
// shared byte H as e2m1(code) * 2^(e_b - H) (shift in [-3, 2], always exact),
// when the bytes are close enough (gap d with d - min(d, 2, hi) <= 3); otherwise
// each block keeps its byte and its plain values.  An all-zero block takes its
// partner's byte.  Codes are decoded with the hardware FP4 -> f32 convert at
// scale 2^shift and re-encoded with the f32 -> FP6 (E3M2) convert, both exact
// for these values.  The tile's 128 columns (rows) are exactly one 128-wide
// operand group, so every byte of the operand, padding included, is written.
// Within a group the last 8 bytes of pairs 0..3 are stored in the order 0, 2,
// 1, 3, so that one 16-byte read gives a GEMM lane both of its pairs' tails.
#include "ft_device.h"

namespace ft {
namespace {

constexpr int QT = 128;                 // tile edge (elements)
constexpr int QTHREADS = 256;
constexpr int RM_PITCH = QT / 2 + 8;    // bytes per LDS row-major code row (padded)
constexpr int CM_PITCH = QT / 2 + 8;    // bytes per LDS column-major code row (padded)
constexpr int OP_GROUP_BYTES = 96;      // operand bytes per row per 128 reduction elements

typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
typedef unsigned v6u __attribute__((ext_vector_type(6)));

struct QuantOut {
  uint8_t* codes_rm; uint8_t* codes_cm; void* scales; void* scales_cm;
  uint8_t* op_rm; uint8_t* op_rm_scales; uint8_t* op_cm; uint8_t* op_cm_scales;
};

// Exchange with the lane whose index differs in bit MASK (MASK < 16).
template <int MASK>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  return (uint32_t)__shfl_xor((int)v, MASK, 64);
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

// One 32-element pair of a row: 16 bytes of E2M1 codes (elements 0..15 in bytes
// 0..7 from block 1, 16..31 in bytes 8..15 from block 2), block scale bytes e1,
// e2 and all-zero flags -> 6 dwords of E3M2 (element n in bits 6n..6n+5) and
// the pair's scale bytes s1, s2 (equal when merged).
__device__ __forceinline__ v6u merge_pair(const uint32_t (&w)[4], int e1, int e2, bool z1, bool z2, int& s1,
                                          int& s2) {
  int f1 = e1, f2 = e2;
  if (z1 && z2) { f1 = f2 = max(e1, e2); }
  else if (z1) { f1 = e2; }
  else if (z2) { f2 = e1; }
  const int d = abs(f1 - f2), hi = max(f1, f2);
  const int u = min(min(d, 2), hi);
  const bool merged = d - u <= 3;
  const int H = hi - u;
  s1 = merged ? H : e1;
  s2 = merged ? H : e2;
  const int t1 = merged ? f1 - H : 0, t2 = merged ? f2 - H : 0;     // in [-3, 2]
  const float m1 = __builtin_bit_cast(float, (uint32_t)(t1 + 127) << 23);
  const float m2 = __builtin_bit_cast(float, (uint32_t)(t2 + 127) << 23);
  v16f ev, od;   // even / odd elements: the convert interleaves its two inputs
#define FT_DEC(J, W, SEL, M)                                                   \
  {                                                                            \
    const v2f_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(W, M, SEL);        \
    ev[J] = v.x;                                                               \
    od[J] = v.y;                                                               \
  }
  FT_DEC(0, w[0], 0, m1) FT_DEC(1, w[0], 1, m1) FT_DEC(2, w[0], 2, m1) FT_DEC(3, w[0], 3, m1)
  FT_DEC(4, w[1], 0, m1) FT_DEC(5, w[1], 1, m1) FT_DEC(6, w[1], 2, m1) FT_DEC(7, w[1], 3, m1)
  FT_DEC(8, w[2], 0, m2) FT_DEC(9, w[2], 1, m2) FT_DEC(10, w[2], 2, m2) FT_DEC(11, w[2], 3, m2)
  FT_DEC(12, w[3], 0, m2) FT_DEC(13, w[3], 1, m2) FT_DEC(14, w[3], 2, m2) FT_DEC(15, w[3], 3, m2)
#undef FT_DEC
  return __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(ev, od, 1.0f);
}

template <bool POW2, bool WRITE_RM, bool WRITE_CM, bool OP_RM, bool OP_CM>
__global__ void __launch_bounds__(QTHREADS)
quant_block16_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, QuantOut o) {
  constexpr bool STAGE_RM = WRITE_RM || OP_RM, STAGE_CM = WRITE_CM || OP_CM, OPS = OP_RM || OP_CM;
  __shared__ __attribute__((aligned(16))) uint8_t s_rm[STAGE_RM ? QT * RM_PITCH : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_cm[STAGE_CM ? QT * CM_PITCH : 16];
  __shared__ uint8_t s_e[OPS ? 64 : 1];   // scale byte of each of the tile's 8 x 8 blocks
  __shared__ uint8_t s_z[OPS ? 64 : 1];   // 1 when every code of the block is +-0
  uint8_t* __restrict__ codes_rm = o.codes_rm;
  uint8_t* __restrict__ codes_cm = o.codes_cm;
  void* __restrict__ scales = o.scales;
  void* __restrict__ scales_cm = o.scales_cm;

  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.y * QT;
  const int64_t col0 = (int64_t)blockIdx.x * QT;
  const int trows = (int)min<int64_t>(QT, rows - row0);   // multiple of 16
  const int tcols = (int)min<int64_t>(QT, cols - col0);   // multiple of 16

  // 1. each lane owns one 16-element row segment of one block per pass, read
  //    straight from HBM (two 16-byte loads; the 4 blocks of a wave are
  //    horizontally adjacent, so a wave reads 16 rows x 128 contiguous bytes).
  //    All 4 passes' loads are issued before any is used.
  const int i = tid & 15;              // row inside the block
  constexpr int NPASS = (QT / 16) * (QT / 16) * 16 / QTHREADS;
  v4i seg[NPASS][2];
#pragma unroll
  for (int it = 0; it < NPASS; ++it) {
    const int b = it * (QTHREADS / 16) + (tid >> 4);   // block index in the tile
    const int br = b >> 3, bc = b & 7;                 // 8x8 blocks per tile
    seg[it][0] = seg[it][1] = v4i{0, 0, 0, 0};
    if (br * 16 < trows && bc * 16 < tcols) {
      const uint16_t* src = x + (row0 + br * 16 + i) * ldx + col0 + bc * 16;
      seg[it][0] = *reinterpret_cast<const v4i*>(src);
      seg[it][1] = *reinterpret_cast<const v4i*>(src + 8);
    }
  }

  // 2. per block: amax across its 16 lanes, scale, codes, layouts.
#pragma unroll
  for (int it = 0; it < NPASS; ++it) {
    const int b = it * (QTHREADS / 16) + (tid >> 4);   // block index in the tile
    const int br = b >> 3, bc = b & 7;                 // 8x8 blocks per tile
    const bool live = (br * 16 < trows) && (bc * 16 < tcols);  // uniform over the 16 lanes
    const v4i p0 = seg[it][0], p1 = seg[it][1];
    uint32_t d[8] = {(uint32_t)p0.x, (uint32_t)p0.y, (uint32_t)p0.z, (uint32_t)p0.w,
                     (uint32_t)p1.x, (uint32_t)p1.y, (uint32_t)p1.z, (uint32_t)p1.w};
    // block maximum of |x| on the bf16 bit patterns (magnitude order = integer
    // order): sign bits cleared, packed 16-bit maxima, then the two halves
    v2u16 pm = __builtin_bit_cast(v2u16, d[0] & 0x7fff7fffu);
#pragma unroll
    for (int k = 1; k < 8; ++k) pm = __builtin_elementwise_max(pm, __builtin_bit_cast(v2u16, d[k] & 0x7fff7fffu));
    uint32_t m = max((uint32_t)pm.x, (uint32_t)pm.y);
    m = max(m, xor_lane<8>(m));
    m = max(m, xor_lane<4>(m));
    m = max(m, xor_lane<2>(m));
    m = max(m, xor_lane<1>(m));

    uint32_t w0 = 0, w1 = 0;
    if constexpr (POW2) {
      const int E = pow2_exp_bf16(m);
      const float sc = __builtin_bit_cast(float, (uint32_t)(E + 127) << 23);  // 2^E as the E8M0 operand
#define FT_CVT(W, K, SEL) W = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(W, __builtin_bit_cast(v2bf, d[K]), sc, SEL)
      FT_CVT(w0, 0, 0); FT_CVT(w0, 1, 1); FT_CVT(w0, 2, 2); FT_CVT(w0, 3, 3);
      FT_CVT(w1, 4, 0); FT_CVT(w1, 5, 1); FT_CVT(w1, 6, 2); FT_CVT(w1, 7, 3);
#undef FT_CVT
      if (live && i == 0) {
        if (scales) static_cast<uint8_t*>(scales)[(row0 / 16 + br) * (cols / 16) + col0 / 16 + bc] = (uint8_t)(E + 127);
        if (scales_cm)
          static_cast<uint8_t*>(scales_cm)[(col0 / 16 + bc) * (rows / 16) + row0 / 16 + br] = (uint8_t)(E + 127);
      }
      if constexpr (OPS) {
        uint32_t nz = (w0 | w1) & 0x77777777u;   // any non-zero magnitude in this row
        nz |= xor_lane<8>(nz);
        nz |= xor_lane<4>(nz);
        nz |= xor_lane<2>(nz);
        nz |= xor_lane<1>(nz);
        if (i == 0) {
          s_e[b] = (uint8_t)(E + 127);
          s_z[b] = nz == 0 ? 1 : 0;
        }
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
    if constexpr (STAGE_RM) {
      *reinterpret_cast<v2i*>(s_rm + (br * 16 + i) * RM_PITCH + bc * 8) = v2i{(int)w0, (int)w1};
    }
    if constexpr (STAGE_CM) {
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
  // 4. pair-merged operands: item = (tile row or column, pair); 4 consecutive
  //    lanes write one operand row's 96-byte group.
  if constexpr (OP_RM) {
    const int64_t pitch = (cols + QT - 1) / QT * OP_GROUP_BYTES;
    const int64_t spitch = (cols + QT - 1) / QT * 8;
#pragma unroll
    for (int it = 0; it < (QT * 4) / QTHREADS; ++it) {
      const int item = it * QTHREADS + tid, r = item >> 2, p = item & 3;
      if (r < trows) {
        const v2i c0 = *reinterpret_cast<const v2i*>(s_rm + r * RM_PITCH + 16 * p);
        const v2i c1 = *reinterpret_cast<const v2i*>(s_rm + r * RM_PITCH + 16 * p + 8);
        const uint32_t w[4] = {(uint32_t)c0.x, (uint32_t)c0.y, (uint32_t)c1.x, (uint32_t)c1.y};
        const int b1 = (r >> 4) * 8 + 2 * p;
        int s1, s2;
        const v6u f = merge_pair(w, s_e[b1], s_e[b1 + 1], s_z[b1] != 0, s_z[b1 + 1] != 0, s1, s2);
        uint8_t* dst = o.op_rm + (row0 + r) * pitch + blockIdx.x * OP_GROUP_BYTES;
        *reinterpret_cast<v4i*>(dst + 16 * p) = v4i{(int)f[0], (int)f[1], (int)f[2], (int)f[3]};
        *reinterpret_cast<v2i*>(dst + 64 + 8 * (2 * (p & 1) + (p >> 1))) = v2i{(int)f[4], (int)f[5]};
        if ((r & 15) == 0)
          *reinterpret_cast<uint16_t*>(o.op_rm_scales + (row0 / 16 + (r >> 4)) * spitch + blockIdx.x * 8 + 2 * p) =
              (uint16_t)(s1 | (s2 << 8));
      }
    }
  }
  if constexpr (OP_CM) {
    const int64_t pitch = (rows + QT - 1) / QT * OP_GROUP_BYTES;
    const int64_t spitch = (rows + QT - 1) / QT * 8;
#pragma unroll
    for (int it = 0; it < (QT * 4) / QTHREADS; ++it) {
      const int item = it * QTHREADS + tid, cl = item >> 2, p = item & 3;
      if (cl < tcols) {
        const v2i c0 = *reinterpret_cast<const v2i*>(s_cm + cl * CM_PITCH + 16 * p);
        const v2i c1 = *reinterpret_cast<const v2i*>(s_cm + cl * CM_PITCH + 16 * p + 8);
        const uint32_t w[4] = {(uint32_t)c0.x, (uint32_t)c0.y, (uint32_t)c1.x, (uint32_t)c1.y};
        const int b1 = (2 * p) * 8 + (cl >> 4), b2 = b1 + 8;
        int s1, s2;
        const v6u f = merge_pair(w, s_e[b1], s_e[b2], s_z[b1] != 0, s_z[b2] != 0, s1, s2);
        uint8_t* dst = o.op_cm + (col0 + cl) * pitch + blockIdx.y * OP_GROUP_BYTES;
        *reinterpret_cast<v4i*>(dst + 16 * p) = v4i{(int)f[0], (int)f[1], (int)f[2], (int)f[3]};
        *reinterpret_cast<v2i*>(dst + 64 + 8 * (2 * (p & 1) + (p >> 1))) = v2i{(int)f[4], (int)f[5]};
        if ((cl & 15) == 0)
          *reinterpret_cast<uint16_t*>(o.op_cm_scales + (col0 / 16 + (cl >> 4)) * spitch + blockIdx.y * 8 + 2 * p) =
              (uint16_t)(s1 | (s2 << 8));
      }
    }
  }
}

template <bool POW2, bool RM, bool CM, bool ORM, bool OCM>
ft_status launch4(const void* x, int64_t rows, int64_t cols, int64_t ldx, const QuantOut& o, hipStream_t s) {
  dim3 grid((unsigned)((cols + QT - 1) / QT), (unsigned)((rows + QT - 1) / QT));
  hipLaunchKernelGGL((quant_block16_kernel<POW2, RM, CM, ORM, OCM>), grid, dim3(QTHREADS), 0, s,
                     static_cast<const uint16_t*>(x), rows, cols, ldx, o);
  return launch_status();
}

template <bool POW2, bool RM, bool CM>
ft_status launch_ops(const void* x, int64_t rows, int64_t cols, int64_t ldx, const QuantOut& o, hipStream_t s) {
  if constexpr (POW2) {
    if (o.op_rm && o.op_cm) return launch4<POW2, RM, CM, true, true>(x, rows, cols, ldx, o, s);
    if (o.op_rm) return launch4<POW2, RM, CM, true, false>(x, rows, cols, ldx, o, s);
    if (o.op_cm) return launch4<POW2, RM, CM, false, true>(x, rows, cols, ldx, o, s);
  }
  if constexpr (RM || CM) return launch4<POW2, RM, CM, false, false>(x, rows, cols, ldx, o, s);
  return FT_EINVAL;
}

template <bool POW2>
ft_status launch_quant(const void* x, int64_t rows, int64_t cols, int64_t ldx, const QuantOut& o, hipStream_t s) {
  if (o.codes_rm && o.codes_cm) return launch_ops<POW2, true, true>(x, rows, cols, ldx, o, s);
  if (o.codes_rm) return launch_ops<POW2, true, false>(x, rows, cols, ldx, o, s);
  if (o.codes_cm) return launch_ops<POW2, false, true>(x, rows, cols, ldx, o, s);
  return launch_ops<POW2, false, false>(x, rows, cols, ldx, o, s);
}

ft_status validate(const void* x, int64_t rows, int64_t cols, int64_t ldx) {
  if (!mult16(rows) || !mult16(cols) || ldx < cols) return FT_ESHAPE;
  if (rows == 0 || cols == 0) return FT_OK;
  if (!x) return FT_EINVAL;
  if (!aligned16(x) || (ldx % 8) != 0) return FT_EALIGN;
  if ((rows + QT - 1) / QT >= 65535) return FT_ESHAPE;
  return FT_OK;
}

}  // namespace
}  // namespace ft

extern "C" ft_status ft_quant_block16(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                                      ft_scale_mode mode, uint8_t* codes_rm, uint8_t* codes_cm,
                                      void* scales, void* scales_cm, hipStream_t stream) {
  using namespace ft;
  if (mode != FT_SCALE_POW2 && mode != FT_SCALE_F32) return FT_EINVAL;
  ft_status st = validate(x, rows, cols, ldx);
  if (st != FT_OK || rows == 0 || cols == 0) return st;
  if (!scales || (!codes_rm && !codes_cm)) return FT_EINVAL;
  if ((codes_rm && !aligned16(codes_rm)) || (codes_cm && !aligned16(codes_cm)) || !aligned16(scales) ||
      (scales_cm && !aligned16(scales_cm)))
    return FT_EALIGN;
  const QuantOut o = {codes_rm, codes_cm, scales, scales_cm, nullptr, nullptr, nullptr, nullptr};
  return mode == FT_SCALE_POW2 ? launch_quant<true>(x, rows, cols, ldx, o, stream)
                               : launch_quant<false>(x, rows, cols, ldx, o, stream);
}

extern "C" size_t ft_operand_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  return (size_t)rows * (size_t)((cols + 127) / 128) * 96;
}

extern "C" size_t ft_operand_scale_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  return (size_t)(rows / 16) * (size_t)((cols + 127) / 128) * 8;
}

extern "C" ft_status ft_quant_block16_op(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                                         uint8_t* codes_rm, uint8_t* codes_cm, uint8_t* scales,
                                         uint8_t* scales_cm, uint8_t* op_rm, uint8_t* op_rm_scales,
                                         uint8_t* op_cm, uint8_t* op_cm_scales, hipStream_t stream) {
  using namespace ft;
  ft_status st = validate(x, rows, cols, ldx);
  if (st != FT_OK || rows == 0 || cols == 0) return st;
  if (!codes_rm && !codes_cm && !op_rm && !op_cm) return FT_EINVAL;
  if ((op_rm && !op_rm_scales) || (op_cm && !op_cm_scales)) return FT_EINVAL;
  if ((codes_rm || codes_cm) && !scales) return FT_EINVAL;
  const void* ptrs[] = {codes_rm, codes_cm, scales, scales_cm, op_rm, op_rm_scales, op_cm, op_cm_scales};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FT_EALIGN;
  const QuantOut o = {codes_rm, codes_cm, scales, scales_cm, op_rm, op_rm_scales, op_cm, op_cm_scales};
  return launch_quant<true>(x, rows, cols, ldx, o, stream);
}

extern "C" const char* ft_status_str(ft_status s) {
  switch (s) {
    case FT_OK: return "ok";
    case FT_EINVAL: return "invalid argument (null pointer or unknown enum)";
    case FT_ESHAPE: return "bad shape (dimension not a multiple of 16, or ranks out of range)";
    case FT_EALIGN: return "misaligned pointer or leading dimension (16-byte alignment required)";
    case FT_EHIP: return "HIP launch failed";
    case FT_ENOTSUP: return "not supported by this library";
    case FT_ESPACE: return "workspace too small";
  }
  return "unknown status";
}
