// ft_lowrank_fused: shared down-projection of the stabilizer and LoRA branches.
//
// FourTune section 3.3 ("LoRA Fusion"): the branches share their input, so one
// pass over it computes both down-projections:  out = [in wa^T | in wb^T]
// (forward: in = X, wa = L1^T, wb = A^T; backward: in = G, wa = L2, wb = B).
//
// HBM-bound (arithmetic intensity = rank FLOP/byte): the input is read exactly
// once.  One workgroup owns 32 rows and all rank columns; its 8 waves split the
// reduction dimension into interleaved 128-column chunks, each wave keeping a
// 32 x rank fp32 accumulator on bf16 MFMA 32x32x16; the 8 partial tiles are
// summed through LDS in a fixed order, so the result is deterministic.
#include "ft_common.h"

namespace ft {
namespace {

constexpr int LR_WAVES = 8;
constexpr int LR_THREADS = LR_WAVES * 64;
constexpr int LR_ROWS = 32;
constexpr int LR_CHUNK = 128;          // reduction columns per wave step (8 MFMA k-steps)
constexpr int LR_PITCH = 33;           // floats per LDS partial row (padded)

template <int NCT>  // number of 32-wide rank column tiles (1..4)
__global__ void __launch_bounds__(LR_THREADS)
lowrank_kernel(const uint16_t* __restrict__ in, int64_t M, int64_t Kin, int64_t ld_in,
               const uint16_t* __restrict__ wa, int ra, const uint16_t* __restrict__ wb, int rb,
               float* __restrict__ out) {
  __shared__ float s_part[LR_WAVES * LR_ROWS * LR_PITCH];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rho = ra + rb;
  const int64_t row0 = (int64_t)blockIdx.x * LR_ROWS;
  const int lr = lane & 31;             // row (A) / rank column (B) inside a 32-tile
  const int kh = (lane >> 5) * 8;       // this lane's 8-element half of a 16-wide k-step

  const int64_t arow = row0 + lr;
  const bool arow_ok = arow < M;
  const uint16_t* aptr = in + (arow_ok ? arow : 0) * ld_in + kh;

  const uint16_t* wptr[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    int j = ct * 32 + lr;
    wptr[ct] = j < ra ? wa + (int64_t)j * Kin + kh : (j < rho ? wb + (int64_t)(j - ra) * Kin + kh : nullptr);
  }

  v16f acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct] = v16f{};

  const int64_t nchunks = (Kin + LR_CHUNK - 1) / LR_CHUNK;
  for (int64_t c = wave; c < nchunks; c += LR_WAVES) {
    const int64_t k0 = c * LR_CHUNK;
    v4i a[8];
    v4i b[NCT][8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int64_t k = k0 + s * 16;
      const bool kok = k < Kin;                        // Kin is a multiple of 16
      a[s] = (kok && arow_ok) ? *reinterpret_cast<const v4i*>(aptr + k) : v4i{0, 0, 0, 0};
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        b[ct][s] = (kok && wptr[ct]) ? *reinterpret_cast<const v4i*>(wptr[ct] + k) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[s]),
                                                          __builtin_bit_cast(v8bf, b[ct][s]), acc[ct], 0, 0, 0);
    }
  }

  // fixed-order reduction of the 8 wave partials, one 32x32 column tile at a time
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    float* mine = s_part + wave * LR_ROWS * LR_PITCH;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      mine[row * LR_PITCH + lr] = acc[ct][r];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < (LR_ROWS * 32) / LR_THREADS; ++e) {
      int idx = e * LR_THREADS + threadIdx.x;
      int row = idx >> 5, col = idx & 31;
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < LR_WAVES; ++w) v += s_part[(w * LR_ROWS + row) * LR_PITCH + col];
      int j = ct * 32 + col;
      if (row0 + row < M && j < rho) out[(row0 + row) * rho + j] = v;
    }
    __syncthreads();
  }
}

}  // namespace
}  // namespace ft

extern "C" ft_status ft_lowrank_fused(const void* in, int64_t M, int64_t Kin, int64_t ld_in,
                                      const void* wa, int32_t ra, const void* wb, int32_t rb,
                                      float* out, hipStream_t stream) {
  using namespace ft;
  if (!mult16(M) || !mult16(Kin) || ld_in < Kin) return FT_ESHAPE;
  if (ra < 0 || rb < 0 || (ra % 16) || (rb % 16) || ra + rb > 128) return FT_ESHAPE;
  const int rho = ra + rb;
  if (M == 0 || rho == 0) return FT_OK;
  if (!out || (ra && !wa) || (rb && !wb) || (Kin && !in)) return FT_EINVAL;
  if ((Kin && !aligned16(in)) || (ld_in % 8) || (ra && !aligned16(wa)) || (rb && !aligned16(wb)) ||
      !aligned16(out))
    return FT_EALIGN;
  if (Kin == 0) return fill_zero_f32(out, M * rho, stream);  // empty reduction
  dim3 grid((unsigned)((M + LR_ROWS - 1) / LR_ROWS));
  const uint16_t* ip = static_cast<const uint16_t*>(in);
  const uint16_t* a = static_cast<const uint16_t*>(wa);
  const uint16_t* b = static_cast<const uint16_t*>(wb);
  const int nct = (rho + 31) / 32;
  switch (nct) {
    case 1: hipLaunchKernelGGL(lowrank_kernel<1>, grid, dim3(LR_THREADS), 0, stream, ip, M, Kin, ld_in, a, ra, b, rb, out); break;
    case 2: hipLaunchKernelGGL(lowrank_kernel<2>, grid, dim3(LR_THREADS), 0, stream, ip, M, Kin, ld_in, a, ra, b, rb, out); break;
    case 3: hipLaunchKernelGGL(lowrank_kernel<3>, grid, dim3(LR_THREADS), 0, stream, ip, M, Kin, ld_in, a, ra, b, rb, out); break;
    default: hipLaunchKernelGGL(lowrank_kernel<4>, grid, dim3(LR_THREADS), 0, stream, ip, M, Kin, ld_in, a, ra, b, rb, out); break;
  }
  return launch_status();
}
