// Adapter weight gradients of FourTune section 3.2 (reductions over tokens):
//
//   dA^T = V[:, rs:]^T X      (V[:, rs:] = G B^T from the backward down-projection)
//   dB   = T[:, rs:]^T G      (T[:, rs:] = X A from the forward down-projection)
//
// Both are dW[j][c] = sum_m P[m][poff + j] Q[m][c] with a small fp32 P and a
// large bf16 Q read once from HBM.  The MFMA needs runs of consecutive m in
// both operands, so (1) a tiny pre-pass writes P's slice transposed and split
// into bf16 hi + lo planes [r x M]; (2) each wave stages 64 x 64 tiles of Q
// row-major in its own LDS region (16-byte writes) and takes the MFMA's
// token-major B fragments with transposing LDS reads (ds_read_b64_tr_b16: four
// tokens of one column per read) and accumulates on bf16 MFMA 32x32x16; (3) the
// 4 waves of a workgroup, each owning
// every 4th 64-row chunk of the workgroup's token range, are summed through LDS
// in a fixed order, and token-range splits (for parallelism when the output is
// narrow) are summed by a final pass in a fixed order: results are deterministic.
#include "ft_internal.h"

namespace ft {
namespace {

constexpr int LG_COLS = 64;                  // output columns per workgroup (128-byte rows of Q)
constexpr int LG_CHUNK = 64;
constexpr int LG_WAVES = 4;
constexpr int LG_THREADS = LG_WAVES * 64;
constexpr int Q_PITCH = 2 * LG_COLS + 16;     // bytes per LDS row of a staged Q tile (conflict-free tr reads)
constexpr int RED_PITCH = 33;                // floats per LDS row of a 32 x 32 partial

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

int choose_splits(int64_t M, int64_t ncols) {
  const int64_t strips = (ncols + LG_COLS - 1) / LG_COLS;
  int64_t s = (512 + strips - 1) / strips;
  const int64_t smax = M / 256 > 0 ? M / 256 : 1;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

// P[m][poff + j] -> hi/lo bf16 planes Pt[j][m]
__global__ void split_transpose_kernel(const float* __restrict__ P, int64_t ldp, int poff, int r,
                                       int64_t M, uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= M * r) return;
  const int64_t m = idx / r;
  const int j = (int)(idx % r);
  uint32_t h, l;
  split_bf16(P[m * ldp + poff + j], h, l);
  hi[(int64_t)j * M + m] = (uint16_t)h;
  lo[(int64_t)j * M + m] = (uint16_t)l;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

template <int NRT>  // 32-row tiles over the adapter rank r (1..4)
__global__ void __launch_bounds__(LG_THREADS)
lora_grad_kernel(const uint16_t* __restrict__ Phi, const uint16_t* __restrict__ Plo, int r,
                 const uint16_t* __restrict__ Q, int64_t M, int64_t ncols, int64_t rows_per_split,
                 float* __restrict__ out, int64_t out_split_stride) {
  __shared__ __attribute__((aligned(16))) uint8_t s_q[LG_WAVES][LG_CHUNK * Q_PITCH];
  __shared__ float s_red[LG_WAVES * 32 * RED_PITCH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  const int64_t c0 = (int64_t)blockIdx.x * LG_COLS;
  const int64_t ms = (int64_t)blockIdx.y * rows_per_split;
  const int64_t me = min(M, ms + rows_per_split);
  uint8_t* qs = s_q[wave];
  // transposing read: within each 16-lane group, source lane 4r + q points at
  // row (token) 8 * (group >> 1) + r and columns 16 * (group & 1) + 4q .. +3
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_row = 8 * (g16 >> 1) + (s16 >> 2);
  const int tr_col = 16 * (g16 & 1) + 4 * (s16 & 3);

  v16f acc[NRT][2];
#pragma unroll
  for (int t = 0; t < NRT; ++t) acc[t][0] = acc[t][1] = v16f{};

  // Q[mb : mb+64, c0 : c0+64] in registers (lane: rows t >> 3 of 8 chunks of 16
  // bytes); the next tile's loads are in flight while this one is consumed
  auto load_q = [&](v4i (&v)[8], int64_t mb) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = lane + 64 * u, m = t >> 3, q = t & 7;
      v[u] = (mb + m < me && c0 + 8 * q < ncols) ? *reinterpret_cast<const v4i*>(Q + (mb + m) * ncols + c0 + 8 * q)
                                               : v4i{0, 0, 0, 0};
    }
  };
  v4i qa[8], qb[8];
  const int64_t mstep = LG_WAVES * LG_CHUNK;
  int64_t mb = ms + (int64_t)wave * LG_CHUNK;
  if (mb < me) load_q(qa, mb);
  for (; mb < me; mb += mstep) {
    // tile -> LDS, row-major, 16-byte chunks
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = lane + 64 * u, m = t >> 3, q = t & 7;
      *reinterpret_cast<v4i*>(qs + m * Q_PITCH + 16 * q) = qa[u];
    }
    if (mb + mstep < me) load_q(qb, mb + mstep);
    wave_sync();
#pragma unroll
    for (int ks = 0; ks < LG_CHUNK / 16; ++ks) {
      const int64_t m = mb + 16 * ks + 8 * lh;   // 8 consecutive tokens of this lane
      v8bf bq[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const uint8_t* b0 = qs + (16 * ks + tr_row) * Q_PITCH + 2 * (32 * ct + tr_col);
        const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(b0));
        const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(b0 + 4 * Q_PITCH));
        const v2i l2 = __builtin_bit_cast(v2i, lo4), h2 = __builtin_bit_cast(v2i, hi4);
        bq[ct] = __builtin_bit_cast(v8bf, v4i{l2.x, l2.y, h2.x, h2.y});
      }
#pragma unroll
      for (int t = 0; t < NRT; ++t) {
        const int j = 32 * t + l32;
        v4i h = {0, 0, 0, 0}, l = {0, 0, 0, 0};
        if (j < r && m < me) {   // M and the split bounds are multiples of 16
          h = *reinterpret_cast<const v4i*>(Phi + (int64_t)j * M + m);
          l = *reinterpret_cast<const v4i*>(Plo + (int64_t)j * M + m);
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          acc[t][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, h), bq[ct], acc[t][ct], 0, 0, 0);
          acc[t][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, l), bq[ct], acc[t][ct], 0, 0, 0);
        }
      }
    }
    wave_sync();
#pragma unroll
    for (int u = 0; u < 8; ++u) qa[u] = qb[u];
  }

  // sum the 4 wave partials in a fixed order and store this split's result
  float* outs = out + (int64_t)blockIdx.y * out_split_stride;
#pragma unroll
  for (int t = 0; t < NRT; ++t)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float* mine = s_red + wave * 32 * RED_PITCH;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mine[(8 * (rr >> 2) + 4 * lh + (rr & 3)) * RED_PITCH + l32] = acc[t][ct][rr];
      __syncthreads();
#pragma unroll
      for (int e = 0; e < (32 * 32) / LG_THREADS; ++e) {
        const int idx = e * LG_THREADS + threadIdx.x, row = idx >> 5, col = idx & 31;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < LG_WAVES; ++w) v += s_red[(w * 32 + row) * RED_PITCH + col];
        const int j = 32 * t + row;
        const int64_t cc = c0 + 32 * ct + col;
        if (j < r && cc < ncols) outs[(int64_t)j * ncols + cc] = v;
      }
      __syncthreads();
    }
}

// out = sum over the splits of part[s], added in split order from 0.0f
// (deterministic).  Each thread adds 4 consecutive values (n is a multiple of 4:
// the rank and the column count are multiples of 16) with 16-byte loads, the
// split loop unrolled so that its loads are in flight together.
__global__ void sum_splits_kernel(const float* __restrict__ part, int splits, int64_t n, float* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  v4f v = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
  for (int s = 0; s < splits; ++s) v += *reinterpret_cast<const v4f*>(part + (int64_t)s * n + i);
  *reinterpret_cast<v4f*>(out + i) = v;
}

}  // namespace

size_t lora_grad_workspace(int64_t M, int64_t ncols, int r) {
  if (r == 0 || M == 0 || ncols == 0) return 0;
  const int S = choose_splits(M, ncols);
  size_t b = 2 * align256((size_t)r * M * 2);
  if (S > 1) b += align256((size_t)S * r * ncols * 4);
  return b;
}

ft_status launch_lora_grad(const float* P, int64_t ldp, int poff, int r, const uint16_t* Q,
                           int64_t M, int64_t ncols, float* dW, void* ws, hipStream_t s) {
  if (r == 0 || ncols == 0) return FT_OK;
  if (r % 16 || ncols % 16 || !aligned16(dW)) return FT_ESHAPE;   // the split sum's 16-byte accesses
  if (M == 0) return fill_zero_f32(dW, (int64_t)r * ncols, s);
  const int S = choose_splits(M, ncols);
  uint8_t* w = static_cast<uint8_t*>(ws);
  uint16_t* hi = reinterpret_cast<uint16_t*>(w);
  uint16_t* lo = reinterpret_cast<uint16_t*>(w + align256((size_t)r * M * 2));
  float* part = S > 1 ? reinterpret_cast<float*>(w + 2 * align256((size_t)r * M * 2)) : dW;
  const int64_t n = M * r;
  hipLaunchKernelGGL(split_transpose_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, P, ldp, poff, r, M, hi, lo);
  if (launch_status() != FT_OK) return FT_EHIP;
  // token range per split: a multiple of 64 rows
  int64_t per = (M + S - 1) / S;
  per = (per + LG_CHUNK - 1) / LG_CHUNK * LG_CHUNK;
  const int S_used = (int)((M + per - 1) / per);
  dim3 grid((unsigned)((ncols + LG_COLS - 1) / LG_COLS), (unsigned)S_used);
  const int64_t stride = (int64_t)r * ncols;
  const int nrt = (r + 31) / 32;
  switch (nrt) {
    case 1: hipLaunchKernelGGL(lora_grad_kernel<1>, grid, dim3(LG_THREADS), 0, s, hi, lo, r, Q, M, ncols, per, part, stride); break;
    case 2: hipLaunchKernelGGL(lora_grad_kernel<2>, grid, dim3(LG_THREADS), 0, s, hi, lo, r, Q, M, ncols, per, part, stride); break;
    case 3: hipLaunchKernelGGL(lora_grad_kernel<3>, grid, dim3(LG_THREADS), 0, s, hi, lo, r, Q, M, ncols, per, part, stride); break;
    default: hipLaunchKernelGGL(lora_grad_kernel<4>, grid, dim3(LG_THREADS), 0, s, hi, lo, r, Q, M, ncols, per, part, stride); break;
  }
  if (launch_status() != FT_OK) return FT_EHIP;
  if (S > 1) {
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((stride / 4 + 255) / 256)), dim3(256), 0, s, part, S_used, stride, dW);
    return launch_status();
  }
  return FT_OK;
}

}  // namespace ft
