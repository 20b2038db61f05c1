// Adapter weight gradients of FourTune section 3.2 taken by extra workgroups of
// the backward's dX GEMM launch, so that the backward is one kernel launch on
// the caller's stream (no second stream, no cross-stream events):
//
//   problem 0:  dA^T[j][c] = sum_m V[m][poff + j] X[m][c]     (c < K)
//   problem 1:  dB[j][c]   = sum_m T[m][poff + j] G[m][c]     (c < N)
//
// The GEMM's own workgroups come first in the grid; the adapter workgroups
// follow, so the hardware places them on the CUs the GEMM's last round leaves
// free (or after the GEMM when it fills every CU).  A unit of work is one
// problem's 64-column strip over one token range (split); workgroup w takes
// units w, w + nwg, ...  Within a unit each of the 8 waves stages every 8th
// chunk of CH tokens of the strip in its own LDS region (16-byte writes) and
// accumulates on bf16 MFMA 32x32x16: the A operand is P's rank slice (8
// consecutive tokens of one rank per lane, read from the fp32 P and split into
// bf16 hi + lo in registers), the B operand is the Q chunk read token-major with
// transposing LDS reads (ds_read_b64_tr_b16).  The 8 wave partials are added
// through LDS in wave order.  With one token range the unit stores dA^T / dB
// directly; with several, each range stores an fp32 partial and
// adapter_sum_kernel adds them in range order.  The result depends on the shape
// and the range count only, never on which workgroup took a unit.
#pragma once

#include "ft_common.h"

namespace ft {

struct AdaptArgs {
  const float* P[2] = {nullptr, nullptr};       // V, T: fp32 [M][ldp]
  const uint16_t* Q[2] = {nullptr, nullptr};    // X [M][K], G [M][N]: bf16
  float* out[2] = {nullptr, nullptr};           // dA^T [r][K], dB [r][N]
  int64_t ncols[2] = {0, 0};                    // K, N
  int strips[2] = {0, 0};                       // 64-column strips (0: the problem is not computed)
  float* part = nullptr;                        // splits > 1: [splits][r * ncols[0] + r * ncols[1]] (the
                                                // second term only when problem 1 is computed)
  int64_t M = 0, ldp = 0, rows_per_split = 0;
  int poff = 0, r = 0, splits = 1, units = 0, nwg = 0;
};

constexpr int AD_COLS = 64;                     // output columns per unit (128-byte rows of Q)
constexpr int AD_PITCH = 2 * AD_COLS + 16;      // bytes per LDS row of a staged Q chunk
constexpr int AD_RED_PITCH = 33;                // floats per LDS row of a 32 x 32 wave partial
constexpr int AD_WAVES = 8;
constexpr int AD_MAX_R = 64;                    // ranks per unit: two 32-rank MFMA tiles
// tokens per wave chunk: 32 keeps the chunk's P values, two chunks of Q and the
// accumulators within the GEMM kernel's register budget (64 spills)
constexpr int AD_CH = 32;
// LDS of the adapter workgroup with CH-token chunks (the reduction reuses the chunk area)
constexpr int ad_lds_bytes(int ch) {
  return AD_WAVES * ch * AD_PITCH > AD_WAVES * 32 * AD_RED_PITCH * 4 ? AD_WAVES * ch * AD_PITCH
                                                                     : AD_WAVES * 32 * AD_RED_PITCH * 4;
}

namespace adapt_detail {

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// one unit: problem p, 64-column strip `strip`, token range s.  NRT: 32-rank
// MFMA tiles (r <= 32 NRT).  Loads go through buffer resources that cover the
// unit's token range: a lane whose rows or columns fall outside points its
// offset past the range (AD_OOR) and reads zeros, so no load is branched.
constexpr uint32_t AD_RSRC_FLAGS = 0x00020000u;   // raw buffer, 32-bit dword format (gfx9 family)
constexpr uint32_t AD_OOR = 0x80000000u;          // an offset past every range

template <int CH, int NRT>
__device__ __forceinline__ void unit(const AdaptArgs& a, int p, int strip, int s, uint8_t* lds) {
  constexpr int NL = CH / 8;        // 16-byte Q pieces per lane per chunk (CH rows x 8 pieces / 64 lanes)
  constexpr int NKS = CH / 16;      // MFMA k-steps per chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  const int64_t ncols = a.ncols[p], ldp = a.ldp;
  const int r = a.r;
  const int64_t c0 = (int64_t)strip * AD_COLS;
  const int64_t ms = (int64_t)s * a.rows_per_split;
  const int64_t me = min(a.M, ms + a.rows_per_split);
  const int rows = (int)(me - ms);
  // the unit's rows of Q (from column c0) and of P (from column poff)
  const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.Q[p] + ms * ncols + c0), 0, (int)((int64_t)rows * ncols * 2 - c0 * 2), AD_RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.P[p] + ms * ldp + a.poff), 0, (int)((int64_t)rows * ldp * 4 - a.poff * 4), AD_RSRC_FLAGS);
  uint8_t* qs = lds + wave * (CH * AD_PITCH);
  // transposing read: within each 16-lane group, source lane 4r + q points at
  // token 8 * (group >> 1) + r and columns 16 * (group & 1) + 4q .. +3
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_row = 8 * (g16 >> 1) + (s16 >> 2);
  const int tr_col = 16 * (g16 & 1) + 4 * (s16 & 3);
  // Q piece of this lane: token (lane >> 3) + 8u of the chunk, columns 8 (lane & 7) ..
  const bool q_on = c0 + 8 * (lane & 7) < ncols;
  const uint32_t q_row_b = (uint32_t)(ncols * 2);

  v16f acc[NRT][2];
#pragma unroll
  for (int t = 0; t < NRT; ++t) acc[t][0] = acc[t][1] = v16f{};

  // chunk rows [rb, rb + CH) of the unit (rb relative to ms)
  auto load_q = [&](v4i (&v)[NL], int rb) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const uint32_t off = q_on ? (uint32_t)(rb + (lane >> 3) + 8 * u) * q_row_b + 16u * (uint32_t)(lane & 7) : AD_OOR;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rQ, off, 0, 0);
    }
  };
  // P[m .. m + 7][poff + j] for the lane's rank j = 32 t + l32 and tokens
  // m = rb + 16 ks + 8 lh (rows past the range read 0: the bounds are multiples of 16)
  float pv[NKS][NRT][8];
  auto load_p = [&](int rb) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int t = 0; t < NRT; ++t) {
        const int j = 32 * t + l32;
        const uint32_t o0 = j < r ? ((uint32_t)(rb + 16 * ks + 8 * lh) * (uint32_t)ldp + (uint32_t)j) * 4u : AD_OOR;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          pv[ks][t][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rP, o0 + (uint32_t)(i * ldp * 4), 0, 0));
      }
    }
  };

  v4i qa[NL], qb[NL];
  const int step = AD_WAVES * CH;
  int rb = wave * CH;
  if (rb < rows) load_q(qa, rb);
  for (; rb < rows; rb += step) {
    load_p(rb);   // issued before the next chunk's Q loads, so waiting for it leaves those in flight
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int t = lane + 64 * u, m = t >> 3, q = t & 7;
      *reinterpret_cast<v4i*>(qs + m * AD_PITCH + 16 * q) = qa[u];
    }
    if (rb + step < rows) load_q(qb, rb + step);
    wave_sync();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      v8bf bq[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const uint8_t* b0 = qs + (16 * ks + tr_row) * AD_PITCH + 2 * (32 * ct + tr_col);
        const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(b0));
        const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(b0 + 4 * AD_PITCH));
        const v2i l2 = __builtin_bit_cast(v2i, lo4), h2 = __builtin_bit_cast(v2i, hi4);
        bq[ct] = __builtin_bit_cast(v8bf, v4i{l2.x, l2.y, h2.x, h2.y});
      }
#pragma unroll
      for (int t = 0; t < NRT; ++t) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split_bf16x2(pv[ks][t][2 * i], pv[ks][t][2 * i + 1], h[i], l[i]);
        const v8bf hv = __builtin_bit_cast(v8bf, v4i{(int)h[0], (int)h[1], (int)h[2], (int)h[3]});
        const v8bf lv = __builtin_bit_cast(v8bf, v4i{(int)l[0], (int)l[1], (int)l[2], (int)l[3]});
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          acc[t][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hv, bq[ct], acc[t][ct], 0, 0, 0);
          acc[t][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lv, bq[ct], acc[t][ct], 0, 0, 0);
        }
      }
    }
    wave_sync();
#pragma unroll
    for (int u = 0; u < NL; ++u) qa[u] = qb[u];
  }

  // the 8 wave partials added in wave order through LDS (over the chunk area)
  const int64_t plane = (int64_t)r * (a.ncols[0] + (a.strips[1] ? a.ncols[1] : 0));   // one range's partials
  float* dst = a.splits == 1 ? a.out[p] : a.part + (int64_t)s * plane + (p ? (int64_t)r * a.ncols[0] : 0);
  float* s_red = reinterpret_cast<float*>(lds);
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float* mine = s_red + wave * 32 * AD_RED_PITCH;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mine[(8 * (rr >> 2) + 4 * lh + (rr & 3)) * AD_RED_PITCH + l32] = acc[t][ct][rr];
      __syncthreads();
#pragma unroll
      for (int e = 0; e < (32 * 32) / (AD_WAVES * 64); ++e) {
        const int idx = e * AD_WAVES * 64 + tid, row = idx >> 5, col = idx & 31;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < AD_WAVES; ++w) v += s_red[(w * 32 + row) * AD_RED_PITCH + col];
        const int j = 32 * t + row;
        const int64_t cc = c0 + 32 * ct + col;
        if (j < r && cc < ncols) dst[(int64_t)j * ncols + cc] = v;
      }
      __syncthreads();
    }
  }
}

}  // namespace adapt_detail

// every unit of workgroup wg (of a.nwg adapter workgroups); 512 threads;
// a.r <= 32 NRT
template <int CH, int NRT>
__device__ __forceinline__ void adapter_run(const AdaptArgs& a, int wg, uint8_t* lds) {
  for (int u = wg; u < a.units; u += a.nwg) {
    const int s = u % a.splits;
    int st = u / a.splits;
    const int p = st < a.strips[0] ? 0 : 1;
    if (p) st -= a.strips[0];
    adapt_detail::unit<CH, NRT>(a, p, st, s, lds);
  }
}

}  // namespace ft
