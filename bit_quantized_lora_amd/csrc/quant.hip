// ft_quant_block16: 16x16 block quantizer to E2M1 codes + one scale per block.
//
// FourTune, section 3.1 (the quantizer Q(.) after Eq. 2, offline for R and
// dynamic for X and G) and section 3.2 (16x16 blocks, so one scale grid serves
// the matrix and its transpose).  Scale = block amax / 6 (power-of-two rounded
// up, or fp32), element code = round-to-nearest-even E2M1 of x / scale.
//
// Two kernels.  The power-of-two instances that write codes only (the GEMM
// operand Q(R), and X or G when quantized on their own) run quant_pow2_kernel:
// 256x256 tiles whose loads cover whole 128-byte lines per instruction, a lane
// holding half of one block (described at the kernel).  The fp32-scale
// instances and the instances that also write the pair-merged operands run
// quant_block16_kernel: the bf16 tile is read once from HBM straight into
// registers (each lane owns one 16-element row segment of one 16x16 block per
// pass, 16 lanes per block), the block maximum is reduced across its 16 lanes
// with DPP exchanges, and the 16x16 nibble block is transposed across the 16
// lanes for the column-major codes.  Both convert with the hardware scaled E2M1
// convert from bf16 (which rounds to nearest-even and saturates, matching the
// oracle bit for bit), stage both code layouts in LDS and write them with
// coalesced 16-byte stores; power-of-two scale bytes are staged in LDS too and
// written as one 16-byte run per block row (and block column of the
// transposed grid) where the run is whole and aligned.
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

// Tile edge: 128 (4 waves) when the pair-merged operands are written (one
// 128-wide operand group per tile), else 256 (8 waves): a 256-wide tile row of
// codes is one whole 128-byte line in both code layouts, so no line is written
// in halves by two workgroups.
constexpr int QT = 128;                 // tile edge of the operand-writing instances (elements)
constexpr int OP_GROUP_BYTES = 96;      // operand bytes per row per 128 reduction elements

typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
typedef unsigned v6u __attribute__((ext_vector_type(6)));

struct QuantOut {
  uint8_t* codes_rm; uint8_t* codes_cm; void* scales; void* scales_cm;
  uint8_t* op_rm; uint8_t* op_rm_scales; uint8_t* op_cm; uint8_t* op_cm_scales;
};

// Exchange with the lane whose index differs in bit MASK (MASK < 16), inside
// each 16-lane DPP row: quad permutes for bits 0 and 1, a rotate by 8 for bit 3,
// and for bit 2 a shift by 4 either way with the direction picked per lane.
// Every source lane lies inside the row, so no lane reads a bound value.
template <int MASK>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const int x = (int)v;
  if constexpr (MASK == 1) return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false);
  if constexpr (MASK == 2) return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false);
  if constexpr (MASK == 8) return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false);
  if constexpr (MASK == 4) {
    const int up = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xF, 0xF, false);   // row_shl:4, from lane + 4
    const int dn = __builtin_amdgcn_update_dpp(x, x, 0x114, 0xF, 0xF, false);   // row_shr:4, from lane - 4
    return (uint32_t)((__lane_id() & 4) ? dn : up);
  }
  static_assert(MASK == 1 || MASK == 2 || MASK == 4 || MASK == 8, "lane masks inside a 16-lane row");
  return v;
}

// Transpose a 16x16 block of nibbles held one row per lane (64 bits: positions
// = columns) so that lane i ends up with column i (positions = rows).  Step b
// swaps bit b of the lane index with bit b of the nibble position.
__device__ __forceinline__ void transpose_nibbles16(uint32_t& w0, uint32_t& w1, int i) {
  {  // bit 3: dword halves
    const bool hi = (i & 8) != 0;
    const uint32_t recv = xor_lane<8>(hi ? w0 : w1);
    w0 = hi ? recv : w0;
    w1 = hi ? w1 : recv;
  }
#define FT_NIB_STEP(BIT, SHIFT, M0)                                           \
  {                                                                           \
    const uint32_t r0 = xor_lane<BIT>(w0), r1 = xor_lane<BIT>(w1);            \
    const bool hi = (i & BIT) != 0;                                           \
    w0 = hi ? ((w0 & ~(M0)) | ((r0 & ~(M0)) >> SHIFT)) : ((w0 & (M0)) | ((r0 & (M0)) << SHIFT)); \
    w1 = hi ? ((w1 & ~(M0)) | ((r1 & ~(M0)) >> SHIFT)) : ((w1 & (M0)) | ((r1 & (M0)) << SHIFT)); \
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
struct QCfg {
  static constexpr bool OPS = OP_RM || OP_CM;
  static constexpr int T = OPS ? 128 : 256;                // tile edge
  static constexpr int THREADS = OPS ? 256 : 512;        // as QThreads
  static constexpr int PITCH = T / 2 + 16;                 // bytes per LDS code row (16-byte aligned, padded)
  static constexpr int BPR = T / 16;                       // blocks per tile row
};

template <bool OPS>
struct QThreads { static constexpr int value = OPS ? 256 : 512; };

template <bool POW2, bool WRITE_RM, bool WRITE_CM, bool OP_RM, bool OP_CM>
__global__ void __launch_bounds__(QThreads<OP_RM || OP_CM>::value)
quant_block16_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, QuantOut o) {
  using Q = QCfg<POW2, WRITE_RM, WRITE_CM, OP_RM, OP_CM>;
  constexpr int QT = Q::T, QTHREADS = Q::THREADS, RM_PITCH = Q::PITCH, CM_PITCH = Q::PITCH, BPR = Q::BPR;
  constexpr bool STAGE_RM = WRITE_RM || OP_RM, STAGE_CM = WRITE_CM || OP_CM, OPS = OP_RM || OP_CM;
  __shared__ __attribute__((aligned(16))) uint8_t s_rm[STAGE_RM ? QT * RM_PITCH : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_cm[STAGE_CM ? QT * CM_PITCH : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_e[POW2 ? BPR * BPR : 1];   // scale byte of each block
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
    const int br = b / BPR, bc = b % BPR;              // BPR x BPR blocks per tile
    seg[it][0] = seg[it][1] = v4i{0, 0, 0, 0};
    if (br * 16 < trows && bc * 16 < tcols) {          // read once: streaming loads
      const uint16_t* src = x + (row0 + br * 16 + i) * ldx + col0 + bc * 16;
      seg[it][0] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src));
      seg[it][1] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src + 8));
    }
  }

  // 2. per block: amax across its 16 lanes, scale, codes, layouts.
#pragma unroll
  for (int it = 0; it < NPASS; ++it) {
    const int b = it * (QTHREADS / 16) + (tid >> 4);   // block index in the tile
    const int br = b / BPR, bc = b % BPR;
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
      if (i == 0) s_e[b] = (uint8_t)(E + 127);   // both scale grids are written from LDS below
      if constexpr (OPS) {
        uint32_t nz = (w0 | w1) & 0x77777777u;   // any non-zero magnitude in this row
        nz |= xor_lane<8>(nz);
        nz |= xor_lane<4>(nz);
        nz |= xor_lane<2>(nz);
        nz |= xor_lane<1>(nz);
        if (i == 0) s_z[b] = nz == 0 ? 1 : 0;
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

  // 3a. power-of-two scale bytes: lane r < BPR writes block row r of the grid,
  //     lane 64 + c block column c of the transposed grid, each as one BPR-byte
  //     store where the run is whole and aligned, else byte by byte.
  if constexpr (POW2) {
    const int nbr = trows / 16, nbc = tcols / 16;
    const bool row_lane = scales && tid < nbr, col_lane = scales_cm && tid >= 64 && tid - 64 < nbc;
    if (row_lane || col_lane) {
      uint8_t* dst;
      int n;
      uint32_t wd[BPR / 4];
      if (row_lane) {
        const int r = tid;
        dst = static_cast<uint8_t*>(scales) + (row0 / 16 + r) * (cols / 16) + col0 / 16;
        n = nbc;
#pragma unroll
        for (int k = 0; k < BPR / 4; ++k) wd[k] = *reinterpret_cast<const uint32_t*>(s_e + r * BPR + 4 * k);
      } else {
        const int c = tid - 64;
        dst = static_cast<uint8_t*>(scales_cm) + (col0 / 16 + c) * (rows / 16) + row0 / 16;
        n = nbr;
#pragma unroll
        for (int k = 0; k < BPR / 4; ++k)
          wd[k] = (uint32_t)s_e[(4 * k) * BPR + c] | ((uint32_t)s_e[(4 * k + 1) * BPR + c] << 8) |
                  ((uint32_t)s_e[(4 * k + 2) * BPR + c] << 16) | ((uint32_t)s_e[(4 * k + 3) * BPR + c] << 24);
      }
      if (n == BPR && (reinterpret_cast<uintptr_t>(dst) & (BPR - 1)) == 0) {
        if constexpr (BPR == 16) *reinterpret_cast<v4i*>(dst) = v4i{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
        else *reinterpret_cast<v2i*>(dst) = v2i{(int)wd[0], (int)wd[1]};
      } else {
        for (int k = 0; k < n; ++k) dst[k] = (uint8_t)(wd[k >> 2] >> (8 * (k & 3)));
      }
    }
  }

  // 3. LDS -> HBM, 16-byte stores; QT / 32 lanes cover one code row of the tile
  //    (a whole 128-byte line for the 256-wide tile).  A chunk of 32 codes whose
  //    second half lies past the tile's ragged edge (an extent of 16 mod 32) is
  //    stored as its first 8 bytes only.
  constexpr int CPR = QT / 32;                          // 16-byte chunks per code row
  if constexpr (WRITE_RM) {
#pragma unroll
    for (int it = 0; it < (QT * CPR) / QTHREADS; ++it) {
      const int c = it * QTHREADS + tid, r = c / CPR, q = c % CPR;
      if (r < trows && q * 32 < tcols) {
        const v4i v = *reinterpret_cast<const v4i*>(s_rm + r * RM_PITCH + q * 16);
        uint8_t* dst = codes_rm + (row0 + r) * (cols / 2) + col0 / 2 + q * 16;
        if (q * 32 + 32 <= tcols) __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(dst));
        else *reinterpret_cast<v2i*>(dst) = v2i{v.x, v.y};
      }
    }
  }
  if constexpr (WRITE_CM) {
#pragma unroll
    for (int it = 0; it < (QT * CPR) / QTHREADS; ++it) {
      const int c = it * QTHREADS + tid, cl = c / CPR, q = c % CPR;
      if (cl < tcols && q * 32 < trows) {
        const v4i v = *reinterpret_cast<const v4i*>(s_cm + cl * CM_PITCH + q * 16);
        uint8_t* dst = codes_cm + (col0 + cl) * (rows / 2) + row0 / 2 + q * 16;
        if (q * 32 + 32 <= trows) __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(dst));
        else *reinterpret_cast<v2i*>(dst) = v2i{v.x, v.y};
      }
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

// 8x8 nibble transpose in registers: on entry a[r] nibble j is element (r, j),
// on exit a[j] nibble r is.  Three exchange stages: the off-diagonal 4x4
// quadrants (16-bit halves), then 2x2 sub-blocks (bytes), then single nibbles.
__device__ __forceinline__ void transpose_nibbles8x8(uint32_t (&a)[8]) {
#define FT_SWP(R, S, SH, M)                                \
  {                                                        \
    const uint32_t t = ((a[R] >> (SH)) ^ a[S]) & (M);      \
    a[S] ^= t;                                             \
    a[R] ^= t << (SH);                                     \
  }
  FT_SWP(0, 4, 16, 0x0000FFFFu) FT_SWP(1, 5, 16, 0x0000FFFFu) FT_SWP(2, 6, 16, 0x0000FFFFu) FT_SWP(3, 7, 16, 0x0000FFFFu)
  FT_SWP(0, 2, 8, 0x00FF00FFu) FT_SWP(1, 3, 8, 0x00FF00FFu) FT_SWP(4, 6, 8, 0x00FF00FFu) FT_SWP(5, 7, 8, 0x00FF00FFu)
  FT_SWP(0, 1, 4, 0x0F0F0F0Fu) FT_SWP(2, 3, 4, 0x0F0F0F0Fu) FT_SWP(4, 5, 4, 0x0F0F0F0Fu) FT_SWP(6, 7, 4, 0x0F0F0F0Fu)
#undef FT_SWP
}

// The power-of-two, codes-only instances: a 256x256 tile per workgroup of 8
// waves.  Wave w owns block rows 2w and 2w + 1; in pass p its lanes 0-31 read
// row 16(2w) + p and lanes 32-63 row 16(2w + 1) + p, 16 bytes each, so every
// load instruction covers two whole 512-byte row runs (whole 128-byte lines;
// a layout in which each instruction touched half of each of its lines read
// about a quarter slower).  A lane thus holds 16 rows x 8 columns, half of one
// 16x16 block; the other half sits in the neighbouring lane, so the block
// maximum is the lane's own maximum and one DPP exchange.  Codes of a row are
// one dword (the hardware scaled convert from bf16); the column-major codes
// come from two 8x8 nibble transposes in registers.  Both layouts are staged
// in LDS at 128 bytes per code line (the column-major lines with their 16-byte
// chunks XOR-swizzled by line, so a wave's staging writes spread over the
// banks) and stored as whole 128-byte lines.
constexpr int QP = 256;
constexpr int QP_THREADS = 512;
constexpr int QP_LINE = QP / 2;   // bytes per staged code line

__device__ __forceinline__ int qp_cm_chunk(int line, int k) { return k ^ ((line >> 3) & 7); }

template <bool WRITE_RM, bool WRITE_CM>
__global__ void __launch_bounds__(QP_THREADS)
quant_pow2_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, QuantOut o) {
  __shared__ __attribute__((aligned(16))) uint8_t s_rm[WRITE_RM ? QP * QP_LINE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_cm[WRITE_CM ? QP * QP_LINE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_e[16 * 16];   // scale byte of each block
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = lane & 31;                     // 16-byte piece of the tile row
  const int br = 2 * w + (lane >> 5);          // block row
  const int bc = q >> 1, hc = q & 1;           // block column, its left or right 8 columns
  const int64_t row0 = (int64_t)blockIdx.y * QP;
  const int64_t col0 = (int64_t)blockIdx.x * QP;
  const int trows = (int)min<int64_t>(QP, rows - row0);   // multiple of 16
  const int tcols = (int)min<int64_t>(QP, cols - col0);   // multiple of 16
  const bool live = br * 16 < trows && bc * 16 < tcols;

  // 1. all 16 passes' loads issued before any is used (streaming hints)
  v4i seg[16];
  const uint16_t* src = x + (row0 + br * 16) * ldx + col0 + q * 8;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    seg[p] = v4i{0, 0, 0, 0};
    if (live) seg[p] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src + p * ldx));
  }

  // 2. block maximum of |x| on the bf16 bit patterns, scale, codes
  v2u16 pm = __builtin_bit_cast(v2u16, (uint32_t)seg[0].x & 0x7fff7fffu);
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    pm = __builtin_elementwise_max(pm, __builtin_bit_cast(v2u16, (uint32_t)seg[p].x & 0x7fff7fffu));
    pm = __builtin_elementwise_max(pm, __builtin_bit_cast(v2u16, (uint32_t)seg[p].y & 0x7fff7fffu));
    pm = __builtin_elementwise_max(pm, __builtin_bit_cast(v2u16, (uint32_t)seg[p].z & 0x7fff7fffu));
    pm = __builtin_elementwise_max(pm, __builtin_bit_cast(v2u16, (uint32_t)seg[p].w & 0x7fff7fffu));
  }
  uint32_t m = max((uint32_t)pm.x, (uint32_t)pm.y);
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0xB1, 0xF, 0xF, false));   // lane ^ 1
  const int E = pow2_exp_bf16(m);
  const float sc = __builtin_bit_cast(float, (uint32_t)(E + 127) << 23);   // 2^E as the E8M0 operand
  if (hc == 0) s_e[br * 16 + bc] = (uint8_t)(E + 127);

  uint32_t rw[16];   // codes of this lane's 8 columns, one dword per row
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    uint32_t c = 0;
#define FT_CVT(V, SEL) c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(v2bf, (uint32_t)(V)), sc, SEL)
    FT_CVT(seg[p].x, 0); FT_CVT(seg[p].y, 1); FT_CVT(seg[p].z, 2); FT_CVT(seg[p].w, 3);
#undef FT_CVT
    rw[p] = c;
  }
  if constexpr (WRITE_RM) {
#pragma unroll
    for (int p = 0; p < 16; ++p)
      *reinterpret_cast<uint32_t*>(s_rm + (br * 16 + p) * QP_LINE + bc * 8 + hc * 4) = rw[p];
  }
  if constexpr (WRITE_CM) {
    uint32_t lo[8], hi[8];   // rows 0-7 and 8-15 of the block
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo[j] = rw[j];
      hi[j] = rw[8 + j];
    }
    transpose_nibbles8x8(lo);
    transpose_nibbles8x8(hi);
    // column j of the lane is code line 8q + j of the tile; the block row's 16
    // codes are bytes 8 br .. 8 br + 7 of that line (chunk br / 2, half br % 2)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int line = 8 * q + j;
      *reinterpret_cast<v2i*>(s_cm + line * QP_LINE + qp_cm_chunk(line, br >> 1) * 16 + (br & 1) * 8) =
          v2i{(int)lo[j], (int)hi[j]};
    }
  }
  __syncthreads();

  // 3a. scale bytes: lane r < 16 writes block row r of the grid, lane 64 + c
  //     block column c of the transposed grid, as one 16-byte store where the
  //     run is whole and aligned, else byte by byte.
  {
    const int nbr = trows / 16, nbc = tcols / 16;
    const bool row_lane = tid < nbr, col_lane = o.scales_cm && tid >= 64 && tid - 64 < nbc;
    if (row_lane || col_lane) {
      uint8_t* dst;
      int n;
      uint32_t wd[4];
      if (row_lane) {
        const int r = tid;
        dst = static_cast<uint8_t*>(o.scales) + (row0 / 16 + r) * (cols / 16) + col0 / 16;
        n = nbc;
#pragma unroll
        for (int k = 0; k < 4; ++k) wd[k] = *reinterpret_cast<const uint32_t*>(s_e + r * 16 + 4 * k);
      } else {
        const int c = tid - 64;
        dst = static_cast<uint8_t*>(o.scales_cm) + (col0 / 16 + c) * (rows / 16) + row0 / 16;
        n = nbr;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          wd[k] = (uint32_t)s_e[(4 * k) * 16 + c] | ((uint32_t)s_e[(4 * k + 1) * 16 + c] << 8) |
                  ((uint32_t)s_e[(4 * k + 2) * 16 + c] << 16) | ((uint32_t)s_e[(4 * k + 3) * 16 + c] << 24);
      }
      if (n == 16 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0)
        *reinterpret_cast<v4i*>(dst) = v4i{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
      else
        for (int k = 0; k < n; ++k) dst[k] = (uint8_t)(wd[k >> 2] >> (8 * (k & 3)));
    }
  }

  // 3b. code lines LDS -> HBM, 16-byte stores, 8 lanes per 128-byte line.  A
  //     chunk of 32 codes whose second half lies past a ragged tile edge is
  //     stored as its first 8 bytes only.
  if constexpr (WRITE_RM) {
#pragma unroll
    for (int it = 0; it < QP * 8 / QP_THREADS; ++it) {
      const int c = it * QP_THREADS + tid, r = c >> 3, k = c & 7;
      if (r < trows && k * 32 < tcols) {
        const v4i v = *reinterpret_cast<const v4i*>(s_rm + r * QP_LINE + k * 16);
        uint8_t* dst = o.codes_rm + (row0 + r) * (cols / 2) + col0 / 2 + k * 16;
        if (k * 32 + 32 <= tcols) __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(dst));
        else *reinterpret_cast<v2i*>(dst) = v2i{v.x, v.y};
      }
    }
  }
  if constexpr (WRITE_CM) {
#pragma unroll
    for (int it = 0; it < QP * 8 / QP_THREADS; ++it) {
      const int c = it * QP_THREADS + tid, line = c >> 3, k = c & 7;
      if (line < tcols && k * 32 < trows) {
        const v4i v = *reinterpret_cast<const v4i*>(s_cm + line * QP_LINE + qp_cm_chunk(line, k) * 16);
        uint8_t* dst = o.codes_cm + (col0 + line) * (rows / 2) + row0 / 2 + k * 16;
        if (k * 32 + 32 <= trows) __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(dst));
        else *reinterpret_cast<v2i*>(dst) = v2i{v.x, v.y};
      }
    }
  }
}

template <bool RM, bool CM>
ft_status launch_qp(const void* x, int64_t rows, int64_t cols, int64_t ldx, const QuantOut& o, hipStream_t s) {
  dim3 grid((unsigned)((cols + QP - 1) / QP), (unsigned)((rows + QP - 1) / QP));
  hipLaunchKernelGGL((quant_pow2_kernel<RM, CM>), grid, dim3(QP_THREADS), 0, s, static_cast<const uint16_t*>(x),
                     rows, cols, ldx, o);
  return launch_status();
}

template <bool POW2, bool RM, bool CM, bool ORM, bool OCM>
ft_status launch4(const void* x, int64_t rows, int64_t cols, int64_t ldx, const QuantOut& o, hipStream_t s) {
  using Q = QCfg<POW2, RM, CM, ORM, OCM>;
  dim3 grid((unsigned)((cols + Q::T - 1) / Q::T), (unsigned)((rows + Q::T - 1) / Q::T));
  hipLaunchKernelGGL((quant_block16_kernel<POW2, RM, CM, ORM, OCM>), grid, dim3(Q::THREADS), 0, s,
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
  if constexpr (POW2 && (RM || CM)) return launch_qp<RM, CM>(x, rows, cols, ldx, o, s);
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
