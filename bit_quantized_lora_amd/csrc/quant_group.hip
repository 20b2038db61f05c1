// Group-wise quantizers: the other granularities of FourTune section 4.3
// ("Impact of Quantization Granularity", Table 5).
//
// ft_quant_group: Q(.) in 1 x g groups along each row (g = 16, the paper's
// group-wise setting; g = 32, the group one scale covers in gfx950's
// block-scaled matrix instruction), with the same rules as the 16x16 blocks:
// scale 2^E, E = min{e : 6 * 2^e >= group max} clamped to [-127, 127], element
// code = round-to-nearest-even E2M1 of x / 2^E with the input's sign.  One lane
// per group: the group's bf16 values are one or two contiguous 32-byte pieces,
// so a wave reads and writes contiguous rows.
//
// ft_requant_group_t: the backward's right operand under group scales (section
// 3.2: after transposition a row's group scales lie along the reduction axis,
// so the codes cannot be reused): Q_g(deq(Q_g(R))^T), the dequantized values
// of Q_g(R) transposed and quantized again in 1 x g groups.  Exact integer /
// power-of-two arithmetic: a value is s * m * 2^(E - 1) with m in {0, 1, 2, 3,
// 4, 6, 8, 12} (twice the E2M1 magnitude), so the new group exponent is the
// largest of E_i - 2 + t(m_i) (t = ceil(log2(m / 3)): the smallest e with
// 6 * 2^e >= m * 2^(E-1)), and the new element ratio m * 2^(E_i - 1 - E') is
// exact in fp32 (or below the smallest E2M1 step when it underflows), rounded
// by the hardware E2M1 convert.  A workgroup transposes a 64 x 64 tile through
// LDS so that both the reads and the writes run along rows.
#include "ft_device.h"

namespace ft {
namespace {

constexpr int QG_THREADS = 256;
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));

template <int G>
__global__ void __launch_bounds__(QG_THREADS)
quant_group_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t gpr = cols / G;
  const int64_t idx = (int64_t)blockIdx.x * QG_THREADS + threadIdx.x;
  if (idx >= rows * gpr) return;
  const int64_t r = idx / gpr, q = idx - (idx / gpr) * gpr;
  const v4i* src = reinterpret_cast<const v4i*>(x + r * ldx + q * G);
  uint32_t w[G / 2];
#pragma unroll
  for (int k = 0; k < G / 8; ++k) {
    const v4i v = src[k];
    w[4 * k] = (uint32_t)v.x; w[4 * k + 1] = (uint32_t)v.y; w[4 * k + 2] = (uint32_t)v.z; w[4 * k + 3] = (uint32_t)v.w;
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < G / 2; ++k) m = max(m, max(w[k] & 0x7fffu, (w[k] >> 16) & 0x7fffu));
  const int E = pow2_exp_bf16(m);
  const float sc = __builtin_bit_cast(float, (uint32_t)(E + 127) << 23);
  uint32_t c[G / 8];   // 8 codes per dword, low nibble first
#pragma unroll
  for (int d = 0; d < G / 8; ++d) {
    uint32_t o = 0;
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(v2bf_t, w[4 * d]), sc, 0);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(v2bf_t, w[4 * d + 1]), sc, 1);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(v2bf_t, w[4 * d + 2]), sc, 2);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(v2bf_t, w[4 * d + 3]), sc, 3);
    c[d] = o;
  }
  uint8_t* dst = codes + r * (cols / 2) + q * (G / 2);
  if constexpr (G == 16) *reinterpret_cast<v2i*>(dst) = v2i{(int)c[0], (int)c[1]};
  else *reinterpret_cast<v4i*>(dst) = v4i{(int)c[0], (int)c[1], (int)c[2], (int)c[3]};
  scales[r * gpr + q] = (uint8_t)(E + 127);
}

// twice the E2M1 magnitude of a 3-bit magnitude code: 0, 1, 2, 3, 4, 6, 8, 12
__device__ __forceinline__ int mag2(int mc) { return mc < 4 ? mc : (mc < 6 ? 2 * mc - 4 : 4 * mc - 16); }
// ceil(log2(m / 3)) for m in {1, 2, 3, 4, 6, 8, 12}
__device__ __forceinline__ int tlog(int m) { return m == 1 ? -1 : (m <= 3 ? 0 : (m <= 6 ? 1 : 2)); }

constexpr int RT = 64;   // tile edge (elements)

template <int G>
__global__ void __launch_bounds__(QG_THREADS)
requant_t_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t rows, int64_t cols,
                 uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t) {
  __shared__ uint8_t lc[RT][RT / 2 + 4];     // codes of 64 rows x 64 columns
  __shared__ uint8_t ls[RT][RT / G];         // their group scale bytes
  const int tid = threadIdx.x;
  const int64_t tiles_c = (cols + RT - 1) / RT;
  const int64_t r0 = (blockIdx.x / tiles_c) * RT, c0 = (blockIdx.x % tiles_c) * RT;
  {  // 64 rows x 32 code bytes: 8 bytes per thread
    const int r = tid >> 2, ch = tid & 3;
    v2i v = {0, 0};
    if (r0 + r < rows && c0 + 16 * ch < cols)
      v = *reinterpret_cast<const v2i*>(codes + (r0 + r) * (cols / 2) + c0 / 2 + 8 * ch);
    *reinterpret_cast<int*>(&lc[r][8 * ch]) = v.x;
    *reinterpret_cast<int*>(&lc[r][8 * ch + 4]) = v.y;
    if (tid < RT * (RT / G)) {
      const int sr = tid / (RT / G), sq = tid % (RT / G);
      ls[sr][sq] = (r0 + sr < rows && c0 + G * sq < cols) ? scales[(r0 + sr) * (cols / G) + c0 / G + sq] : 0;
    }
  }
  __syncthreads();
  constexpr int QPC = RT / G;                // output groups per column in the tile
  if (tid >= RT * QPC) return;
  const int c = tid / QPC, q = tid % QPC;    // output row c0 + c, groups over input rows r0 + qG ..
  const int64_t oc = c0 + c, orow0 = r0 + G * q;
  if (oc >= cols || orow0 >= rows) return;
  int m[G], e[G], sgn[G];
  int Ep = -1000;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int byte = lc[G * q + i][c >> 1];
    const int code = (c & 1) ? byte >> 4 : byte & 15;
    m[i] = mag2(code & 7);
    sgn[i] = code & 8;
    e[i] = (int)ls[G * q + i][c / G] - 127;
    if (m[i]) Ep = max(Ep, e[i] - 2 + tlog(m[i]));
  }
  Ep = Ep == -1000 ? -127 : min(127, max(-127, Ep));
  uint32_t out[G / 8];
#pragma unroll
  for (int d = 0; d < G / 8; ++d) {
    uint32_t o = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = 8 * d + 2 * k + h;
        const float a = ldexpf((float)m[i], e[i] - 1 - Ep);     // exact, or below 0.25 when it underflows
        v[h] = sgn[i] ? -a : a;
      }
      if (k == 0) o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, v[0], v[1], 1.0f, 0);
      else if (k == 1) o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, v[0], v[1], 1.0f, 1);
      else if (k == 2) o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, v[0], v[1], 1.0f, 2);
      else o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, v[0], v[1], 1.0f, 3);
    }
    out[d] = o;
  }
  uint8_t* dst = codes_t + oc * (rows / 2) + orow0 / 2;
  if constexpr (G == 16) *reinterpret_cast<v2i*>(dst) = v2i{(int)out[0], (int)out[1]};
  else *reinterpret_cast<v4i*>(dst) = v4i{(int)out[0], (int)out[1], (int)out[2], (int)out[3]};
  scales_t[oc * (rows / G) + orow0 / G] = (uint8_t)(Ep + 127);
}

}  // namespace
}  // namespace ft

extern "C" ft_status ft_quant_group(const void* x, int64_t rows, int64_t cols, int64_t ldx, int32_t group,
                                    uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  using namespace ft;
  if (group != 16 && group != 32) return FT_EINVAL;
  if (!mult16(rows) || !mult16(cols) || cols % group != 0 || ldx < cols) return FT_ESHAPE;
  if (rows == 0 || cols == 0) return FT_OK;
  if (!x || !codes || !scales) return FT_EINVAL;
  if (!aligned16(x) || !aligned16(codes) || (ldx * 2) % 16 != 0) return FT_EALIGN;
  const int64_t n = rows * (cols / group);
  const dim3 grid((unsigned)((n + QG_THREADS - 1) / QG_THREADS)), block(QG_THREADS);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (group == 16) hipLaunchKernelGGL((quant_group_kernel<16>), grid, block, 0, stream, xp, rows, cols, ldx, codes, scales);
  else hipLaunchKernelGGL((quant_group_kernel<32>), grid, block, 0, stream, xp, rows, cols, ldx, codes, scales);
  return launch_status();
}

extern "C" ft_status ft_requant_group_t(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                                        int32_t group, uint8_t* codes_t, uint8_t* scales_t, hipStream_t stream) {
  using namespace ft;
  if (group != 16 && group != 32) return FT_EINVAL;
  if (!mult16(rows) || !mult16(cols) || cols % group != 0 || rows % group != 0) return FT_ESHAPE;
  if (rows == 0 || cols == 0) return FT_OK;
  if (!codes || !scales || !codes_t || !scales_t) return FT_EINVAL;
  if (!aligned16(codes) || !aligned16(codes_t)) return FT_EALIGN;
  const int64_t tiles = ((rows + RT - 1) / RT) * ((cols + RT - 1) / RT);
  const dim3 grid((unsigned)tiles), block(QG_THREADS);
  if (group == 16)
    hipLaunchKernelGGL((requant_t_kernel<16>), grid, block, 0, stream, codes, scales, rows, cols, codes_t, scales_t);
  else
    hipLaunchKernelGGL((requant_t_kernel<32>), grid, block, 0, stream, codes, scales, rows, cols, codes_t, scales_t);
  return launch_status();
}
