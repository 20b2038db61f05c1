// Block-scaled 4-bit GEMM with the low-rank up-projection fused in its epilogue.
//
//   C[m][n] = sum_k deq(A)[m][k] deq(B)[n][k]  +  sum_j P[m][j] W[j][n]
//
// forward  (FourTune Eq. 2):  A = Q(X) [M x K], B = Q(R) [N x K], P = T, W = [L2; B]
// backward (FourTune Eq. 3):  A = Q(G) [M x N], B = Q(R)^T via the column-major
//                             codes [K x N], P = V, W = [L1^T; A^T]
// Section 3.2 of the paper: the 16x16 blocks let the transposed product read the
// same codes and scales "regardless of whether the access pattern is transposed";
// here the backward pass reads R's column-major codes and the same scale grid
// through a transposed index.  Section 3.3 "LoRA Fusion": the up-projections
// are accumulated into the backbone GEMM's accumulators before the single store.
//
// How 16x16 scales reach the MFMA (scale path "S2"): gfx950's
// v_mfma_scale_f32_32x32x64_f8f6f4 gives each lane 32 consecutive K values of
// one row (or column) and ONE power-of-two (E8M0) scale for them.  A 16x16
// block changes scale every 16 K, so each lane carries exactly one 16-K block
// in the low half of its 32-slot fragment and zeros in the high half; the two
// lane halves of the wave carry two different blocks.  The scale is applied by
// the hardware exactly (power-of-two), so the result is the exact dequantized
// product accumulated in fp32.  This uses half of each MFMA's K slots.
//
// Tiling: 256 x 256 output tile per workgroup, 4 waves in 2 x 2, each wave
// 128 x 128 = 4 x 4 MFMA tiles of 32 x 32 (256 fp32 accumulators per lane).
// K advances 128 elements (64 bytes of codes per row, 8 blocks) per stage; the
// codes are double-buffered in LDS with a 16-byte-chunk XOR swizzle so that
// the fragment reads are conflict-free, and the per-stage 16 x 8 scale tiles
// of both operands are staged alongside (transposed when B's grid is read
// transposed).  Epilogue: W's 256-column slice is staged transposed in LDS;
// P is split into bf16 hi + lo (hi + lo = P to 2^-16) and multiplied on bf16
// MFMA 32x32x16, so the fp32 low-rank intermediate keeps ~16 significant bits.
#include "ft_common.h"
#include "ft_internal.h"

namespace ft {
namespace {

constexpr int BM = 256, BN = 256;
constexpr int BKB = 64;                         // code bytes per row per stage (128 K)
constexpr int GT = 256;                         // threads
constexpr int A_ST = BM * BKB, B_ST = BN * BKB;
constexpr int SA_ST = (BM / 16) * 8, SB_ST = (BN / 16) * 8;
constexpr int STAGE = A_ST + B_ST + SA_ST + SB_ST;
constexpr int MAIN_LDS = 2 * STAGE;
constexpr int EPI_LDS = BN * (2 * 128 + 16);
constexpr int GEMM_LDS = MAIN_LDS > EPI_LDS ? MAIN_LDS : EPI_LDS;

__device__ __forceinline__ int swz(int row, int q) { return row * BKB + ((q ^ ((row >> 2) & 3)) << 4); }

template <bool OUT_BF16>
__global__ void __launch_bounds__(GT, 1) gemm_w4a4_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[GEMM_LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;

  const int64_t tiles_m = (g.M + BM - 1) / BM;
  const int64_t tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t nkt = (g.K + 127) / 128;
  const int64_t Mb = g.M / 16, Nb = g.N / 16, Kb = g.K / 16;

  // ---- global -> register prefetch of one stage ----
  v4i pa[4], pb[4];
  uint8_t ps = 127;
  auto gload = [&](int64_t kt) {
    const int64_t k0 = kt * 128;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = it * GT + tid, row = c >> 2, q = c & 3;
      const int64_t kel = k0 + 32 * q;
      const int64_t am = m0 + row, bn = n0 + row;
      v4i va = {0, 0, 0, 0}, vb = {0, 0, 0, 0};
      if (kel < g.K) {
        const bool full = kel + 32 <= g.K;   // else exactly 16 K remain (K % 32 == 16)
        if (am < g.M) {
          const uint8_t* p = g.A + am * g.lda + kel / 2;
          if (full) va = *reinterpret_cast<const v4i*>(p);
          else { v2i h = *reinterpret_cast<const v2i*>(p); va = v4i{h.x, h.y, 0, 0}; }
        }
        if (bn < g.N) {
          const uint8_t* p = g.B + bn * g.ldb + kel / 2;
          if (full) vb = *reinterpret_cast<const v4i*>(p);
          else { v2i h = *reinterpret_cast<const v2i*>(p); vb = v4i{h.x, h.y, 0, 0}; }
        }
      }
      pa[it] = va; pb[it] = vb;
    }
    const int t = tid & 127, rb = t >> 3, kb = t & 7;
    const int64_t gkb = kt * 8 + kb;
    if (tid < 128) {
      const int64_t grb = m0 / 16 + rb;
      ps = (grb < Mb && gkb < Kb) ? g.sA[grb * g.sA_rs + gkb] : (uint8_t)127;
    } else {
      const int64_t gnb = n0 / 16 + rb;
      ps = (gnb < Nb && gkb < Kb) ? g.sB[gnb * g.sB_ns + gkb * g.sB_ks] : (uint8_t)127;
    }
  };
  auto lstore = [&](int stage) {
    uint8_t* As = smem + stage * STAGE;
    uint8_t* Bs = As + A_ST;
    uint8_t* Ss = Bs + B_ST;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = it * GT + tid, row = c >> 2, q = c & 3;
      *reinterpret_cast<v4i*>(As + swz(row, q)) = pa[it];
      *reinterpret_cast<v4i*>(Bs + swz(row, q)) = pb[it];
    }
    Ss[tid] = ps;   // [0,128): A scales [16 rb][8 kb]; [128,256): B scales
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  if (nkt > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int64_t kt = 0; kt < nkt; ++kt) {
    const int cur = (int)(kt & 1);
    if (kt + 1 < nkt) gload(kt + 1);
    const uint8_t* As = smem + cur * STAGE;
    const uint8_t* Bs = As + A_ST;
    const uint8_t* SAs = Bs + B_ST;
    const uint8_t* SBs = SAs + SA_ST;
    v4i af[4][2], bf[4][2];
    int sa[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 128 + 32 * i + l32;
      af[i][0] = *reinterpret_cast<const v4i*>(As + swz(ra, 2 * lh));
      af[i][1] = *reinterpret_cast<const v4i*>(As + swz(ra, 2 * lh + 1));
      sa[i] = *reinterpret_cast<const int*>(SAs + (ra >> 4) * 8 + 4 * lh);
      const int rbn = wn * 128 + 32 * i + l32;
      bf[i][0] = *reinterpret_cast<const v4i*>(Bs + swz(rbn, 2 * lh));
      bf[i][1] = *reinterpret_cast<const v4i*>(Bs + swz(rbn, 2 * lh + 1));
      sb[i] = *reinterpret_cast<const int*>(SBs + (rbn >> 4) * 8 + 4 * lh);
    }
#define FT_KSTEP(KK)                                                                              \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                               \
      const v8i aop = {af[i][(KK) >> 1][((KK) & 1) * 2], af[i][(KK) >> 1][((KK) & 1) * 2 + 1], 0, 0, 0, 0, 0, 0}; \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                             \
        const v8i bop = {bf[j][(KK) >> 1][((KK) & 1) * 2], bf[j][(KK) >> 1][((KK) & 1) * 2 + 1], 0, 0, 0, 0, 0, 0}; \
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop, acc[i][j], 4, 4, KK, sa[i], KK, sb[j]); \
      }                                                                                           \
    }
    FT_KSTEP(0)
    FT_KSTEP(1)
    FT_KSTEP(2)
    FT_KSTEP(3)
#undef FT_KSTEP
    if (kt + 1 < nkt) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: + P W (bf16 hi/lo split of P on bf16 MFMA) ----
  const int rho = g.ra + g.rb;
  if (rho > 0) {
    const int pitch = 2 * rho + 16;   // bytes per LDS row of W^T
    for (int c = tid; c < rho * (BN / 8); c += GT) {
      const int j = c / (BN / 8), q = c % (BN / 8);
      const int64_t n = n0 + 8 * q;
      v4i v = {0, 0, 0, 0};
      if (n < g.N) {
        const uint16_t* wrow = j < g.ra ? g.Wa + (int64_t)j * g.N : g.Wb + (int64_t)(j - g.ra) * g.N;
        v = *reinterpret_cast<const v4i*>(wrow + n);
      }
      const uint32_t w[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint16_t*>(smem + (8 * q + e) * pitch + 2 * j) = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
    __syncthreads();
    for (int ks = 0; ks < rho / 16; ++ks) {
      v8bf phi[4], plo[4], wf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + wm * 128 + 32 * i + l32;
        const int col = 16 * ks + 8 * lh;
        v4f p0 = {0, 0, 0, 0}, p1 = {0, 0, 0, 0};
        if (row < g.M) {
          p0 = *reinterpret_cast<const v4f*>(g.P + row * rho + col);
          p1 = *reinterpret_cast<const v4f*>(g.P + row * rho + col + 4);
        }
        const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        uint32_t h[8], l[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) split_bf16(pv[e], h[e], l[e]);
        v4i hv = {(int)(h[0] | h[1] << 16), (int)(h[2] | h[3] << 16), (int)(h[4] | h[5] << 16), (int)(h[6] | h[7] << 16)};
        v4i lv = {(int)(l[0] | l[1] << 16), (int)(l[2] | l[3] << 16), (int)(l[4] | l[5] << 16), (int)(l[6] | l[7] << 16)};
        phi[i] = __builtin_bit_cast(v8bf, hv);
        plo[i] = __builtin_bit_cast(v8bf, lv);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int nl = wn * 128 + 32 * j + l32;
        wf[j] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(smem + nl * pitch + 2 * (16 * ks + 8 * lh)));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(phi[i], wf[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(plo[i], wf[j], acc[i][j], 0, 0, 0);
        }
    }
  }

  // ---- store C ----
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + 32 * j + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (row < g.M && col < g.N) {
          if constexpr (OUT_BF16)
            static_cast<uint16_t*>(g.C)[row * g.ldc + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
          else
            static_cast<float*>(g.C)[row * g.ldc + col] = acc[i][j][r];
        }
      }
    }
}

}  // namespace

ft_status launch_gemm_w4a4(const GemmArgs& g, bool out_bf16, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return FT_OK;
  const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  if (tiles >= (int64_t)1 << 31) return FT_ESHAPE;
  if (out_bf16)
    hipLaunchKernelGGL(gemm_w4a4_kernel<true>, dim3((unsigned)tiles), dim3(GT), 0, s, g);
  else
    hipLaunchKernelGGL(gemm_w4a4_kernel<false>, dim3((unsigned)tiles), dim3(GT), 0, s, g);
  return launch_status();
}

}  // namespace ft
