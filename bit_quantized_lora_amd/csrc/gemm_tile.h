// Device pieces shared by the GEMM kernels of the quantized linear: LDS DMA
// helpers, accumulator types, the low-rank up-projection passes (FourTune
// section 3.3 "LoRA Fusion": P W accumulated into the backbone GEMM's
// accumulators) and the output stores.  Included by the .hip files of the
// kernels only; everything has internal linkage.
#pragma once

#include "ft_common.h"
#include "ft_device.h"
#include "ft_internal.h"

namespace ft {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

constexpr int BKB = 64;                         // code bytes per row per stage (128 K)

constexpr uint32_t RSRC_FLAGS = 0x00020000u;   // raw buffer, 32-bit dword format (gfx9 family)

__device__ __forceinline__ int swz(int row, int q) { return row * BKB + ((q ^ ((row >> 2) & 3)) << 4); }

// s_waitcnt with only a vector-memory count (expcnt and lgkmcnt left at their maxima)
#define FT_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt((((N) & 15) | (((N) >> 4) << 14)) | (7 << 4) | (15 << 8))

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// DMA helpers: the buffer-load-to-LDS builtin is called from these non-template
// functions (called from a kernel templated on the tile configuration, it left
// that kernel without a host launch stub).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}
// per-lane offset voff plus a wave-uniform offset soff (scalar operand)
__device__ __forceinline__ void dma16s(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, off, 0, 0, 0);
}

template <int TMI, int TNI>
using AccT = v16f[TMI][TNI];

// An empty asm statement that reads the accumulators: the MFMAs producing them
// are issued before it, so they cannot be sunk past a following wait or barrier.
template <int TMI, int TNI>
__device__ __forceinline__ void pin_acc(AccT<TMI, TNI>& acc) {
#pragma unroll
  for (int i = 0; i < TMI; ++i)
#pragma unroll
    for (int j = 0; j < TNI; ++j) {
#if defined(__HIP_DEVICE_COMPILE__)   // (the host pass has no VGPR constraint)
      asm volatile("" ::"v"(acc[i][j]));
#endif
    }
}

// 4 x 4 transpose within each quad of lanes: on entry lane t of a quad holds
// element (k, t) in v[k]; on exit it holds element (t, k) in v[k].  Two butterfly
// stages over lane bits 0 and 1, each exchanging half of the values with DPP.
__device__ __forceinline__ float dpp_xor1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ void quad_transpose4(float (&v)[4], int t) {
  const bool b0 = t & 1, b1 = t & 2;
#pragma unroll
  for (int k = 0; k < 4; k += 2) {
    const float r = dpp_xor1(b0 ? v[k] : v[k + 1]);
    if (b0) v[k] = r; else v[k + 1] = r;
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float r = dpp_xor2(b1 ? v[k] : v[k + 2]);
    if (b1) v[k] = r; else v[k + 2] = r;
  }
}

// + P W over the tile, then store C.  smem must be free (callers synchronize first).
//
// W rows (rank-major, [rho x N]) are copied to LDS with buffer_load ... lds, one
// tile-wide row per DMA instruction at a pitch of row bytes + 32 (bank-conflict-free
// for the transposed reads below).  The bf16 MFMA's B operand needs 8 consecutive ranks of
// one output column per lane; two ds_read_b64_tr_b16 deliver them: within each
// 16-lane group, result lane i, slot r receives element i % 4 of the 8 bytes that
// source lane 4r + i/4 addressed, so source lanes point 4 columns wide into 4
// consecutive rows.  P's rows for up to 64 ranks are fetched with all loads in
// flight at once; ranks beyond one chunk are processed in further passes.
// BNc: tile width (W rows staged at a pitch of 2*BNc + 32 bytes); CHUNK: ranks
// per pass (their P values are held in registers while the pass runs).
template <int TMI, int CHUNK>
using PRegs = v4f[TMI][CHUNK / 16][2];

// Loads of chunk jc (ranks jc .. jc+nr-1, nr = min(CHUNK, jend - jc); jend < 0:
// all rho ranks): W rows to LDS (lanes 0 .. BNc/8-1: 16 bytes = 8 columns
// each), this wave's P rows to registers.
template <int TMI, int TNI, int NWAVES, int BNc, int CHUNK>
__device__ __forceinline__ void lowrank_load(PRegs<TMI, CHUNK>& p, const GemmArgs& g, uint8_t* smem, int jc,
                                             int64_t m0, int64_t n0, int wave, int lane, int wm, int l32, int lh,
                                             int jend = -1) {
  constexpr int W_PITCH = 2 * BNc + 32;
  const int rho = g.ra + g.rb;
  const int nr = min(CHUNK, (jend < 0 ? rho : jend) - jc);      // multiple of 16
  const __amdgpu_buffer_rsrc_t rWa =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.Wa, 0, (int)((int64_t)g.ra * g.N * 2), RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rWb =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.Wb, 0, (int)((int64_t)g.rb * g.N * 2), RSRC_FLAGS);
  for (int jr = wave; jr < nr; jr += NWAVES) {
    const int j = jc + jr;
    const bool in_a = j < g.ra;
    const int jj = in_a ? j : j - g.ra;
    const int64_t n = n0 + 8 * lane;
    const uint32_t off = (lane < BNc / 8 && n < g.N) ? (uint32_t)(((int64_t)jj * g.N + n) * 2) : 0x80000000u;
    if (lane < BNc / 8) {
      if (in_a) __builtin_amdgcn_raw_ptr_buffer_load_lds(rWa, (lds_void*)(smem + jr * W_PITCH), 16, off, 0, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(rWb, (lds_void*)(smem + jr * W_PITCH), 16, off, 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < TMI; ++i) {
    const int64_t row = m0 + wm * 32 * TMI + 32 * i + l32;
#pragma unroll
    for (int ks = 0; ks < CHUNK / 16; ++ks) {
      p[i][ks][0] = p[i][ks][1] = v4f{0, 0, 0, 0};
      if (16 * ks < nr && row < g.M) {
        const float* src = g.P + row * rho + jc + 16 * ks + 8 * lh;
        p[i][ks][0] = *reinterpret_cast<const v4f*>(src);
        p[i][ks][1] = *reinterpret_cast<const v4f*>(src + 4);
      }
    }
  }
}

// acc += (P_hi + P_lo) W for chunk jc on bf16 MFMA 32x32x16 (its loads complete
// and visible to the workgroup)
template <int TMI, int TNI, int BNc, int CHUNK>
__device__ __forceinline__ void lowrank_mma(AccT<TMI, TNI>& acc, const PRegs<TMI, CHUNK>& p, const GemmArgs& g,
                                            const uint8_t* smem, int jc, int lane, int wn, int jend = -1) {
  constexpr int W_PITCH = 2 * BNc + 32;
  const int nr = min(CHUNK, (jend < 0 ? g.ra + g.rb : jend) - jc);
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_row = 8 * (g16 >> 1) + (s16 >> 2);             // + 16 ks + 4 t
  const int tr_col = 16 * (g16 & 1) + 4 * (s16 & 3);           // + wn*32*TNI + 32 j
#pragma unroll
  for (int ks = 0; ks < CHUNK / 16; ++ks) {
    if (16 * ks < nr) {
      v8bf wf[TNI];
#pragma unroll
      for (int j = 0; j < TNI; ++j) {
        const uint8_t* b0 = smem + (16 * ks + tr_row) * W_PITCH + 2 * (wn * 32 * TNI + 32 * j + tr_col);
        const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(b0));
        const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(b0 + 4 * W_PITCH));
        const v2i l2 = __builtin_bit_cast(v2i, lo4), h2 = __builtin_bit_cast(v2i, hi4);
        wf[j] = __builtin_bit_cast(v8bf, v4i{l2.x, l2.y, h2.x, h2.y});
      }
#pragma unroll
      for (int i = 0; i < TMI; ++i) {
        const float pv[8] = {p[i][ks][0].x, p[i][ks][0].y, p[i][ks][0].z, p[i][ks][0].w,
                             p[i][ks][1].x, p[i][ks][1].y, p[i][ks][1].z, p[i][ks][1].w};
        uint32_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16x2(pv[2 * e], pv[2 * e + 1], h[e], l[e]);
        const v8bf phi = __builtin_bit_cast(v8bf, v4i{(int)h[0], (int)h[1], (int)h[2], (int)h[3]});
        const v8bf plo = __builtin_bit_cast(v8bf, v4i{(int)l[0], (int)l[1], (int)l[2], (int)l[3]});
#pragma unroll
        for (int j = 0; j < TNI; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(phi, wf[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(plo, wf[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }
}

// Chunks from jc0 on, each: loads, wait for all of this wave's memory operations,
// barrier, MFMAs, barrier (LDS free for the next chunk).  smem must be free.
template <int TMI, int TNI, int NWAVES, int BNc, int CHUNK>
__device__ __forceinline__ void lowrank_into_acc(AccT<TMI, TNI>& acc, const GemmArgs& g, uint8_t* smem,
                                                 int64_t m0, int64_t n0, int tid, int wave, int wm, int wn,
                                                 int l32, int lh, int jc0 = 0, int jend = -1) {
  const int lane = tid & 63;
  const int je = jend < 0 ? g.ra + g.rb : jend;
  for (int jc = jc0; jc < je; jc += CHUNK) {
    PRegs<TMI, CHUNK> p;
    lowrank_load<TMI, TNI, NWAVES, BNc, CHUNK>(p, g, smem, jc, m0, n0, wave, lane, wm, l32, lh, je);
    compiler_fence();
    FT_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    lowrank_mma<TMI, TNI, BNc, CHUNK>(acc, p, g, smem, jc, lane, wn, je);
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  }
}

// Low-rank term after the main loop for ranks j0 .. j0+nt-1 (nt <= CHUNK) whose
// tiles fit one ring buffer each: W [nt x BNc] and P [BMc x nt] are fetched by
// DMA during the last stages into ring buffers those stages no longer need, so
// their loads overlap the main loop's last MFMAs, and the products follow the
// last k-step.  LDS layouts, 16-byte chunks XOR-swizzled against bank conflicts:
// W row j (pitch 2 BNc) keeps chunk c at c ^ (2 (j & 3)), so the 4 rows of a
// transposing read fall in distinct banks; P row r (nt / 4 chunks) keeps chunk c
// at r (nt / 4) + (c ^ ((r >> 1) & 3)), so 8 consecutive rows of a 16-byte read
// do.
template <int NWAVES, int BNc>
__device__ __forceinline__ void tail_issue_w(const GemmArgs& g, uint8_t* dst, int64_t n0, int wave, int lane, int j0,
                                             int nt) {
  const __amdgpu_buffer_rsrc_t rWa =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.Wa, 0, (int)((int64_t)g.ra * g.N * 2), RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rWb =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.Wb, 0, (int)((int64_t)g.rb * g.N * 2), RSRC_FLAGS);
  for (int jr = wave; jr < nt; jr += NWAVES) {
    const int j = j0 + jr;                                       // rank; LDS row jr
    const bool in_a = j < g.ra;
    const int jj = in_a ? j : j - g.ra;
    const int c = lane ^ (2 * (j & 3));                          // the chunk this lane fetches
    const int64_t n = n0 + 8 * c;
    const uint32_t off = (lane < BNc / 8 && n < g.N) ? (uint32_t)(((int64_t)jj * g.N + n) * 2) : 0x80000000u;
    if (lane < BNc / 8) {
      if (in_a) dma16(rWa, dst + jr * 2 * BNc, off);
      else dma16(rWb, dst + jr * 2 * BNc, off);
    }
  }
}

template <int NWAVES, int BMc>
__device__ __forceinline__ void tail_issue_p(const GemmArgs& g, uint8_t* dst, int64_t m0, int wave, int lane, int j0,
                                             int nt) {
  const int rho = g.ra + g.rb, cpr = nt / 4;
  const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.P + m0 * rho), 0, (int)(min<int64_t>(BMc, g.M - m0) * rho * 4), RSRC_FLAGS);
  const int nq = BMc * cpr / 64;                                 // 1-KiB DMAs (BMc * nt % 256 == 0)
  for (int q = wave; q < nq; q += NWAVES) {
    const int pos = 64 * q + lane, r = pos / cpr, cs = pos - r * cpr;
    const int c = cs ^ ((r >> 1) & 3);
    dma16(rP, dst + 1024 * q, (uint32_t)((r * rho + j0) * 4 + c * 16));
  }
}

// acc += (P_hi + P_lo) W from the tiles tail_issue_w / tail_issue_p staged
template <int TMI, int TNI, int BNc, int CHUNK>
__device__ __forceinline__ void tail_lowrank_mma(AccT<TMI, TNI>& acc, const uint8_t* wbuf, const uint8_t* pbuf,
                                                 int nt, int lane, int wm, int wn, int l32, int lh) {
  const int cpr = nt / 4;
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_row = 8 * (g16 >> 1) + (s16 >> 2);             // + 16 ks (+ 4 for the second read)
  const int tr_col = 16 * (g16 & 1) + 4 * (s16 & 3);           // + wn 32 TNI + 32 j
#pragma unroll
  for (int ks = 0; ks < CHUNK / 16; ++ks) {
    if (16 * ks < nt) {
      v8bf wf[TNI];
#pragma unroll
      for (int j = 0; j < TNI; ++j) {
        const int row = 16 * ks + tr_row, col = wn * 32 * TNI + 32 * j + tr_col;
        const uint8_t* b0 = wbuf + row * 2 * BNc + (((col >> 3) ^ (2 * (row & 3))) << 4) + 2 * (col & 7);
        const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(b0));
        const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(b0 + 4 * 2 * BNc));
        const v2i l2 = __builtin_bit_cast(v2i, lo4), h2 = __builtin_bit_cast(v2i, hi4);
        wf[j] = __builtin_bit_cast(v8bf, v4i{l2.x, l2.y, h2.x, h2.y});
      }
#pragma unroll
      for (int i = 0; i < TMI; ++i) {
        const int r = wm * 32 * TMI + 32 * i + l32, c0 = 4 * ks + 2 * lh;
        const v4f p0 = *reinterpret_cast<const v4f*>(pbuf + 16 * (r * cpr + (c0 ^ ((r >> 1) & 3))));
        const v4f p1 = *reinterpret_cast<const v4f*>(pbuf + 16 * (r * cpr + ((c0 + 1) ^ ((r >> 1) & 3))));
        const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        uint32_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16x2(pv[2 * e], pv[2 * e + 1], h[e], l[e]);
        const v8bf phi = __builtin_bit_cast(v8bf, v4i{(int)h[0], (int)h[1], (int)h[2], (int)h[3]});
        const v8bf plo = __builtin_bit_cast(v8bf, v4i{(int)l[0], (int)l[1], (int)l[2], (int)l[3]});
#pragma unroll
        for (int j = 0; j < TNI; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(phi, wf[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(plo, wf[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }
}

template <bool OUT_BF16, int TMI, int TNI>
__device__ __forceinline__ void store_acc(AccT<TMI, TNI>& acc, const GemmArgs& g, int64_t m0, int64_t n0, int lane,
                                          int wm, int wn, int l32, int lh) {
  // Store: each lane holds 4 consecutive rows of one column per group of 4
  // accumulator values; a 4 x 4 transpose across the 4 lanes of a quad (DPP quad
  // permutes) gives each lane one row of 4 consecutive columns, so the tile goes
  // out in 8-byte (bf16) or 16-byte (fp32) stores: 4x fewer store instructions.
  const int t4 = lane & 3;
#pragma unroll
  for (int i = 0; i < TMI; ++i)
#pragma unroll
    for (int j = 0; j < TNI; ++j) {
      const int64_t col = n0 + wn * 32 * TNI + 32 * j + (l32 & ~3);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        quad_transpose4(v, t4);
        const int64_t row = m0 + wm * 32 * TMI + 32 * i + 8 * q + 4 * lh + t4;
        if (row < g.M && col < g.N) {
          if constexpr (OUT_BF16) {
            const uint32_t lo = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
            const uint32_t hi = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
            *reinterpret_cast<v2i*>(static_cast<uint16_t*>(g.C) + row * g.ldc + col) = v2i{(int)lo, (int)hi};
          } else {
            *reinterpret_cast<v4f*>(static_cast<float*>(g.C) + row * g.ldc + col) = v4f{v[0], v[1], v[2], v[3]};
          }
        }
      }
    }
}

// bf16 store through LDS: the quad-transposed rows go to a row-major tile image
// in LDS (pitch 2 BNc + 64 bytes, so the 8 rows of one write fall in different
// banks), then the workgroup writes the tile with 16-byte stores, consecutive
// lanes along a row: whole 128-byte lines instead of the 64-byte row pieces the
// accumulator layout gives.  smem must be free (callers synchronize first).
template <int TMI, int TNI, int NWAVES, int BMc, int BNc>
__device__ __forceinline__ void store_acc_bf16_lds(AccT<TMI, TNI>& acc, const GemmArgs& g, uint8_t* smem,
                                                   int64_t m0, int64_t n0, int tid, int wm, int wn, int l32,
                                                   int lh) {
  constexpr int PITCH = 2 * BNc + 64;
  const int t4 = tid & 3;
#pragma unroll
  for (int i = 0; i < TMI; ++i)
#pragma unroll
    for (int j = 0; j < TNI; ++j) {
      const int col = wn * 32 * TNI + 32 * j + (l32 & ~3);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        quad_transpose4(v, t4);
        const int row = wm * 32 * TMI + 32 * i + 8 * q + 4 * lh + t4;
        const uint32_t lo = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
        *reinterpret_cast<v2i*>(smem + row * PITCH + 2 * col) = v2i{(int)lo, (int)hi};
      }
    }
  compiler_fence();
  __syncthreads();
  compiler_fence();
  constexpr int CH = BNc / 8;                                   // 16-byte chunks per row
  constexpr int PER = BMc * CH / (64 * NWAVES);                 // chunks per thread
  static_assert(BMc * CH % (64 * NWAVES) == 0, "whole passes over the tile");
  uint16_t* C = static_cast<uint16_t*>(g.C);
  v4i val[PER];
#pragma unroll
  for (int it = 0; it < PER; ++it) {   // all LDS reads first, then all stores
    const int e = tid + 64 * NWAVES * it, r = e / CH, c = e - (e / CH) * CH;
    val[it] = *reinterpret_cast<const v4i*>(smem + r * PITCH + 16 * c);
  }
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int e = tid + 64 * NWAVES * it, r = e / CH, c = e - (e / CH) * CH;
    const int64_t row = m0 + r, col = n0 + 8 * c;
    if (row < g.M && col < g.N) __builtin_nontemporal_store(val[it], reinterpret_cast<v4i*>(C + row * g.ldc + col));
  }
}

template <bool OUT_BF16, int TMI, int TNI, int NWAVES, int BNc, int CHUNK>
__device__ __forceinline__ void epilogue_and_store(AccT<TMI, TNI>& acc, const GemmArgs& g, uint8_t* smem,
                                                   int64_t m0, int64_t n0, int tid, int wave, int wm, int wn,
                                                   int l32, int lh) {
  lowrank_into_acc<TMI, TNI, NWAVES, BNc, CHUNK>(acc, g, smem, m0, n0, tid, wave, wm, wn, l32, lh);
  store_acc<OUT_BF16, TMI, TNI>(acc, g, m0, n0, tid & 63, wm, wn, l32, lh);
}

constexpr int GROUP_M = 4;   // tile rows per raster group

int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                 hipSuccess && c > 0)
      n = c;
    else
      n = 256;
  }
  return n;
}

// fraction of workgroup slots busy over the launch (one workgroup per CU)
double fill(int64_t tiles, int cus) { return (double)tiles / (double)(((tiles + cus - 1) / cus) * cus); }

}  // namespace
}  // namespace ft
