// ft_lowrank_fused: shared down-projection of the stabilizer and LoRA branches.
//
// FourTune section 3.3 ("LoRA Fusion"): the branches share their input, so one
// pass over it computes both down-projections:  out = [in wa^T | in wb^T]
// (forward: in = X, wa = L1^T, wb = A^T; backward: in = G, wa = L2, wb = B).
//
// HBM-bound (arithmetic intensity = rank FLOP/byte): the input is read exactly
// once.  A workgroup owns 128 rows (4 waves x 32) and a contiguous range of
// 128-column chunks of the reduction; the split over the reduction gives the
// launch enough workgroups to keep every CU streaming.  Per chunk, the weight
// slice [rank x 128] is copied to LDS once (buffer_load ... lds, 16-byte-chunk
// XOR swizzle against bank conflicts) and shared by the 4 waves, while each wave
// prefetches its own 32 input rows of the next chunk into registers.  Products
// run on bf16 MFMA 32x32x16 with fp32 accumulation.  Each split writes its
// partial sums to the workspace and a second pass adds the splits in a fixed
// order, so the result is deterministic.
#include "ft_common.h"

namespace ft {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int LR_THREADS = 256;
constexpr int LR_ROWS = 128;            // rows per workgroup (4 waves x 32)
constexpr int LR_CHUNK = 128;           // reduction columns per chunk (8 MFMA k-steps)
constexpr int LR_WROW = LR_CHUNK * 2;   // bytes per LDS weight row (256, swizzled, unpadded)
constexpr int LR_WBUF = 128 * LR_WROW;  // one weight chunk (up to 128 ranks)
constexpr uint32_t RSRC_FLAGS = 0x00020000u;

#define FT_WAIT_VMCNT0() __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8))
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ int wswz(int row, int q) { return row * LR_WROW + ((q ^ (row & 15)) << 4); }

int64_t chunks_per_split(int64_t M, int64_t Kin) {
  const int64_t nchunks = (Kin + LR_CHUNK - 1) / LR_CHUNK;
  const int64_t rblocks = (M + LR_ROWS - 1) / LR_ROWS;
  int64_t s = (512 + rblocks - 1) / rblocks;        // aim for ~2 workgroups per CU
  if (s > nchunks) s = nchunks;
  if (s < 1) s = 1;
  int64_t cps = (nchunks + s - 1) / s;
  return cps < 4 ? (nchunks < 4 ? nchunks : 4) : cps;   // at least 4 chunks of work per split
}

int64_t num_splits(int64_t M, int64_t Kin) {
  const int64_t nchunks = (Kin + LR_CHUNK - 1) / LR_CHUNK;
  const int64_t cps = chunks_per_split(M, Kin);
  return (nchunks + cps - 1) / cps;
}

template <int NCT>  // number of 32-wide rank column tiles (1..4)
__global__ void __launch_bounds__(LR_THREADS)
lowrank_kernel(const uint16_t* __restrict__ in, int64_t M, int64_t Kin, int64_t ld_in,
               const uint16_t* __restrict__ wa, int ra, const uint16_t* __restrict__ wb, int rb,
               int64_t cps, float* __restrict__ out, int64_t out_split_stride) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_w[2 * LR_WBUF];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rho = ra + rb;
  const int l32 = lane & 31, lh = lane >> 5;
  const int64_t row0 = (int64_t)blockIdx.x * LR_ROWS;
  const int64_t nchunks = (Kin + LR_CHUNK - 1) / LR_CHUNK;
  const int64_t c_begin = (int64_t)blockIdx.y * cps;
  const int64_t c_end = min(nchunks, c_begin + cps);

  const int64_t arow = row0 + 32 * wave + l32;
  const bool arow_ok = arow < M;
  const uint16_t* aptr = in + (arow_ok ? arow : 0) * ld_in + 8 * lh;

  const __amdgpu_buffer_rsrc_t rWa =
      __builtin_amdgcn_make_buffer_rsrc((void*)wa, 0, (int)((int64_t)ra * Kin * 2), RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rWb =
      __builtin_amdgcn_make_buffer_rsrc((void*)wb, 0, (int)((int64_t)rb * Kin * 2), RSRC_FLAGS);

  // weight chunk c -> LDS buffer: DMA instruction i covers rank rows 4i .. 4i+3;
  // lane l fills physical 16-byte chunk l & 15 of row 4i + l/16
  auto issue_w = [&](int buf, int64_t c) {
    for (int i = wave; i < rho / 4; i += LR_THREADS / 64) {
      const int row = 4 * i + (lane >> 4);
      const int q = (lane & 15) ^ (row & 15);
      const int64_t col = c * LR_CHUNK + 8 * q;
      const bool in_a = 4 * i < ra;                   // ra is a multiple of 16: rows 4i..4i+3 share a matrix
      const int jj = in_a ? row : row - ra;
      const uint32_t off = col < Kin ? (uint32_t)(((int64_t)jj * Kin + col) * 2) : 0x80000000u;
      uint8_t* dst = s_w + buf * LR_WBUF + 4 * i * LR_WROW;
      if (in_a) __builtin_amdgcn_raw_ptr_buffer_load_lds(rWa, (lds_void*)dst, 16, off, 0, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(rWb, (lds_void*)dst, 16, off, 0, 0, 0);
    }
  };
  auto load_x = [&](v4i (&a)[8], int64_t c) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int64_t k = c * LR_CHUNK + 16 * s;
      a[s] = (arow_ok && k < Kin) ? *reinterpret_cast<const v4i*>(aptr + k) : v4i{0, 0, 0, 0};
    }
  };

  v16f acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct] = v16f{};

  v4i xa[8], xb[8];
  if (c_begin < c_end) {
    issue_w(0, c_begin);
    load_x(xa, c_begin);
  }
  for (int64_t c = c_begin; c < c_end; ++c) {
    const int buf = (int)((c - c_begin) & 1);
    compiler_fence();
    FT_WAIT_VMCNT0();                    // this wave's DMA and loads of chunk c are done
    __builtin_amdgcn_s_barrier();        // every wave's DMA landed; buffer buf^1 is free
    compiler_fence();
    if (c + 1 < c_end) {
      issue_w(buf ^ 1, c + 1);
      load_x(xb, c + 1);
    }
    const uint8_t* wbuf = s_w + buf * LR_WBUF;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int j = 32 * ct + l32;
        const v4i b = j < rho ? *reinterpret_cast<const v4i*>(wbuf + wswz(j, 2 * s + lh)) : v4i{0, 0, 0, 0};
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, xa[s]),
                                                          __builtin_bit_cast(v8bf, b), acc[ct], 0, 0, 0);
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) xa[s] = xb[s];
  }

  float* o = out + (int64_t)blockIdx.y * out_split_stride;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int j = 32 * ct + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = row0 + 32 * wave + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (row < M && j < rho) o[row * rho + j] = acc[ct][r];
    }
  }
}

__global__ void sum_splits_kernel(const float* __restrict__ part, int64_t splits, int64_t n, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v = 0.0f;
  for (int64_t s = 0; s < splits; ++s) v += part[s * n + i];
  out[i] = v;
}

}  // namespace
}  // namespace ft

extern "C" size_t ft_lowrank_workspace(int64_t M, int64_t Kin, int32_t rho) {
  using namespace ft;
  if (M <= 0 || Kin <= 0 || rho <= 0) return 0;
  const int64_t S = num_splits(M, Kin);
  return S > 1 ? (size_t)(S * M * rho * sizeof(float)) : 0;
}

extern "C" ft_status ft_lowrank_fused(const void* in, int64_t M, int64_t Kin, int64_t ld_in,
                                      const void* wa, int32_t ra, const void* wb, int32_t rb,
                                      float* out, void* workspace, size_t ws_bytes, hipStream_t stream) {
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
  if ((int64_t)rho * Kin * 2 >= ((int64_t)1 << 31)) return FT_ESHAPE;
  const size_t need = ft_lowrank_workspace(M, Kin, rho);
  if (need && (!workspace || ws_bytes < need)) return workspace ? FT_ESPACE : FT_EINVAL;
  if (need && !aligned16(workspace)) return FT_EALIGN;
  const int64_t cps = chunks_per_split(M, Kin);
  const int64_t S = num_splits(M, Kin);
  float* dst = S > 1 ? static_cast<float*>(workspace) : out;
  dim3 grid((unsigned)((M + LR_ROWS - 1) / LR_ROWS), (unsigned)S);
  const uint16_t* ip = static_cast<const uint16_t*>(in);
  const uint16_t* a = static_cast<const uint16_t*>(wa);
  const uint16_t* b = static_cast<const uint16_t*>(wb);
  const int64_t stride = M * rho;
  const int nct = (rho + 31) / 32;
  switch (nct) {
    case 1: hipLaunchKernelGGL(lowrank_kernel<1>, grid, dim3(LR_THREADS), 0, stream, ip, M, Kin, ld_in, a, ra, b, rb, cps, dst, stride); break;
    case 2: hipLaunchKernelGGL(lowrank_kernel<2>, grid, dim3(LR_THREADS), 0, stream, ip, M, Kin, ld_in, a, ra, b, rb, cps, dst, stride); break;
    case 3: hipLaunchKernelGGL(lowrank_kernel<3>, grid, dim3(LR_THREADS), 0, stream, ip, M, Kin, ld_in, a, ra, b, rb, cps, dst, stride); break;
    default: hipLaunchKernelGGL(lowrank_kernel<4>, grid, dim3(LR_THREADS), 0, stream, ip, M, Kin, ld_in, a, ra, b, rb, cps, dst, stride); break;
  }
  if (launch_status() != FT_OK) return FT_EHIP;
  if (S > 1) {
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((stride + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(workspace), S, stride, out);
    return launch_status();
  }
  return FT_OK;
}
