// bf16 x 4-bit GEMM of the precision variants (FourTune section 4.3, "Impact of
// Precision Configurations", Table 4: W4A16G4 keeps the activations in 16 bits,
// W4A4G16 the output gradient; the weight residual stays quantized in both):
//
//   C[m][n] = sum_k A[m][k] deq(B)[n][k]  +  sum_j P[m][j] W[j][n]
//
// W4A16 forward (Eq. 2 with X in place of Q(X)):  A = X bf16 [M x K],
//                B = Q(R) [N x K], P = T, W = [L2; B]
// G16 backward  (Eq. 3 with G in place of Q(G)):  A = G bf16 [M x N],
//                B = Q(R)^T [K x N] (R's column-major codes, transposed scale
//                grid), P = V, W = [L1^T; A^T]
//
// A bf16 operand is not representable in 4 bits, so the product runs on the
// bf16 MFMA (v_mfma_f32_32x32x16_bf16) and B's codes are dequantized in
// registers: an E2M1 value times its block's power-of-two scale has at most two
// significant bits, so it is exact in bf16 (2^-128 .. 4 * 2^126 covers every
// block scale a bf16 input can produce).  v_cvt_scalef32_pk_bf16_fp4 turns two
// codes into two scaled bf16 values.
//
// Reduction order: within a 32-element stage, lane half h of the MFMA takes the
// 16 consecutive elements 16h .. 16h+15, split over the two k-steps (8 each);
// A and B use the same assignment, so the sum is unchanged.  The 8 B elements a
// lane converts per k-step then lie in one 16-element block (one scale), and
// its A elements are 16 consecutive bf16 (two 16-byte LDS reads).
//
// Tiling: 256 x 256 output tile per workgroup, 8 waves in 2 x 4, each 128 x 64
// = 4 x 2 MFMA tiles (B conversions shared by 4 row tiles).  K advances 32
// elements per stage: A 256 rows x 64 bytes (16-byte chunks XOR-swizzled by row
// bits 2-3, conflict-free 16-lane reads), B 256 rows x 16 bytes, and per
// 16-row block of B an 8-byte window of its scale row holding the stage's two
// scale bytes (the window starts at the dword boundary below them, so any scale
// row pitch works; DMA moves whole dwords).  A 6-stage LDS ring filled by
// buffer_load ... lds; every wave issues 3 DMA instructions per stage (waves
// 0-3: two A, one B; waves 4-7: two A, one scale), so waits are compile-time
// counts.  The low-rank term
// goes into the accumulators before the main loop (its loads overlap the
// pipeline fill); the tile is stored as in the 4-bit GEMM.
#include "ft_common.h"
#include "ft_device.h"
#include "ft_internal.h"
#include "gemm_tile.h"

namespace ft {
namespace {

constexpr int H_BM = 256, H_BN = 256;
constexpr int H_WN = 4;                              // waves 2 x 4
constexpr int H_TMI = 4, H_TNI = 2;                  // 32 x 32 tiles per wave
constexpr int H_KS = 32;                             // reduction elements per stage
constexpr int H_A_ST = H_BM * 2 * H_KS;              // bf16 A rows (64 bytes)
constexpr int H_B_ST = H_BN * H_KS / 2;              // code rows (16 bytes)
constexpr int H_S_ST = (H_BN / 16) * 8;              // scale windows
constexpr int H_STAGE = H_A_ST + H_B_ST + H_S_ST;
constexpr int H_NS = 6;                              // ring depth (stages)
constexpr int H_DPS = 3;                             // DMA instructions per wave per stage
constexpr int H_CHUNK = 48;                          // low-rank ranks per pass
constexpr int H_W_PITCH = 2 * H_BN + 32;
constexpr int hmax(int a, int b) { return a > b ? a : b; }
constexpr int H_SMEM = hmax(hmax(H_NS * H_STAGE, (H_NS - 1) * H_STAGE + H_CHUNK * H_W_PITCH),
                            H_BM * (2 * H_BN + 64));
static_assert(2 * H_KS == BKB, "A rows use the 64-byte row swizzle");
static_assert(H_SMEM <= 160 * 1024, "LDS");

// wait until at most n stages' DMAs of this wave remain in flight (n wave-uniform)
__device__ __forceinline__ void wait_stages(int n) {
  switch (n) {
    case 0: FT_WAIT_VMCNT(0); break;
    case 1: FT_WAIT_VMCNT(H_DPS); break;
    case 2: FT_WAIT_VMCNT(2 * H_DPS); break;
    case 3: FT_WAIT_VMCNT(3 * H_DPS); break;
    case 4: FT_WAIT_VMCNT(4 * H_DPS); break;
    default: FT_WAIT_VMCNT(5 * H_DPS); break;
  }
}

// E8M0 byte -> the float 2^(byte - 127) (byte 0: the subnormal 2^-127)
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  return __builtin_bit_cast(float, b ? b << 23 : 0x00400000u);
}

// 8 E2M1 codes (one dword, element e in nibble e) times scale -> 8 bf16
__device__ __forceinline__ v8bf dequant8(uint32_t w, float sc) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  typedef __bf16 v4bf_t __attribute__((ext_vector_type(4)));
  const v4bf_t lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const v4bf_t hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// this wave's fragments of one stage: A for one k-step, B codes and scales for both
struct AFrag {
  v4i a[H_TMI];
};
struct BFrag {
  v2i codes[H_TNI];   // dword s: the 8 codes of k-step s
  uint32_t sb[H_TNI];  // E8M0 scale byte (converted where used, off the read's critical path)
};

__device__ __forceinline__ void read_a(AFrag& f, const uint8_t* st, int s, int wm, int l32, int lh) {
#pragma unroll
  for (int i = 0; i < H_TMI; ++i)
    f.a[i] = *reinterpret_cast<const v4i*>(st + swz(wm * 32 * H_TMI + 32 * i + l32, 2 * lh + s));
}

// scale window of 16-row block b starts at dword floor((b * sB_rs + 2 kt) / 4);
// the stage's two bytes sit at (b * sB_rs + 2 kt) % 4 and the next
__device__ __forceinline__ void read_b(BFrag& f, const uint8_t* st, int kt, int srs4, int wn, int l32, int lh) {
#pragma unroll
  for (int j = 0; j < H_TNI; ++j) {
    const int row = wn * 32 * H_TNI + 32 * j + l32;
    f.codes[j] = *reinterpret_cast<const v2i*>(st + H_A_ST + row * 16 + 8 * lh);
    const int blk = row >> 4;
    const int pos = (blk * srs4 + 2 * kt) & 3;
    f.sb[j] = st[H_A_ST + H_B_ST + 8 * blk + pos + lh];
  }
}

template <int S>
__device__ __forceinline__ void dequant_b(v8bf (&bv)[H_TNI], const BFrag& f) {
#pragma unroll
  for (int j = 0; j < H_TNI; ++j) bv[j] = dequant8((uint32_t)f.codes[j][S], e8m0_value(f.sb[j]));
}

// keeps values computed before a following wait / barrier (asm operand)
__device__ __forceinline__ void pin_b(const v8bf (&bv)[H_TNI]) {
#pragma unroll
  for (int j = 0; j < H_TNI; ++j) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" ::"v"(bv[j]));
#endif
  }
}

template <int I0, int I1>
__device__ __forceinline__ void mma_rows(AccT<H_TMI, H_TNI>& acc, const AFrag& a, const v8bf (&bv)[H_TNI]) {
#pragma unroll
  for (int i = I0; i < I1; ++i) {
    const v8bf av = __builtin_bit_cast(v8bf, a.a[i]);
#pragma unroll
    for (int j = 0; j < H_TNI; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[j], acc[i][j], 0, 0, 0);
  }
}

// A: bf16 [M x K] with row pitch lda BYTES; B: codes [N x K/2], pitch ldb bytes;
// B's block scales sB[(n / 16) * sB_rs + k / 16]; K any multiple of 16.
// TRANS_B: backward instantiation (separate name in profiles).
template <bool OUT_BF16, bool TRANS_B>
__global__ void __launch_bounds__(512, 1)
gemm_a16_kernel(GemmArgs g, int tiles_m, int tiles_n, int per_xcd) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[H_SMEM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / H_WN, wn = wave % H_WN;
  const int l32 = lane & 31, lh = lane >> 5;

  // XCD-aware raster (hardware places workgroup b on XCD b % 8)
  const int b = blockIdx.x;
  const int v = (b & 7) * per_xcd + (b >> 3);
  if (v >= tiles_m * tiles_n) return;
  const int grp = v / (GROUP_M * tiles_n);
  const int first_m = grp * GROUP_M;
  const int gm = min(GROUP_M, tiles_m - first_m);
  const int in_grp = v - grp * GROUP_M * tiles_n;
  const int64_t m0 = (int64_t)(first_m + in_grp % gm) * H_BM;
  const int64_t n0 = (int64_t)(in_grp / gm) * H_BN;
  const int nkt = (int)((g.K + H_KS - 1) / H_KS);
  const bool k_tail = (g.K % H_KS) != 0;            // the last stage holds 16 elements

  // buffer resources for this tile: rows past M / N read as zero
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.A + m0 * g.lda), 0, (int)(min<int64_t>(H_BM, g.M - m0) * g.lda), RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.B + n0 * g.ldb), 0, (int)(min<int64_t>(H_BN, g.N - n0) * g.ldb), RSRC_FLAGS);
  // scale windows: the range runs to the end of the scale grid, so a window may
  // reach into the next tile's rows (unused bytes); only a dword cut by the
  // grid's end reads as zero, and its bytes are then copied one by one
  const uint8_t* s_tile = g.sB + (n0 / 16) * g.sB_rs;
  const int s_range = (int)((g.N / 16 - n0 / 16) * g.sB_rs);
  const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc((void*)s_tile, 0, s_range, RSRC_FLAGS);
  const int srs4 = (int)(g.sB_rs & 3);

  // DMA instructions of a stage: A rows 16q .. 16q+15 for q = wave, wave + 8 (lane
  // l -> row l >> 2, physical chunk l & 3, global chunk (l & 3) ^ row bits 2-3);
  // waves 0-3 also B rows 64 wave .. +63 (one 16-byte row per lane); waves 4-7
  // lanes 0-7 the scale dwords 8 (wave - 4) + lane: block 2 of them per window.
  const uint32_t vA = (uint32_t)((lane >> 2) * g.lda) + 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
  const uint32_t vB = (uint32_t)(lane * g.ldb);
  const bool b_wave = wave < 4;
  const int sd = 8 * (wave - 4) + lane;
  const bool s_on = !b_wave && lane < 8;
  const int s_blk = sd >> 1, s_half = sd & 1;
  const int s_row = (int)(s_blk * g.sB_rs);

  auto issue = [&](int stage, int kt) {
    uint8_t* base = smem + stage * H_STAGE;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = wave + 8 * u;
      dma16s(rA, base + q * 1024, vA, __builtin_amdgcn_readfirstlane((uint32_t)(16 * q * g.lda) + kt * 64u));
    }
    if (b_wave) {
      dma16s(rB, base + H_A_ST + wave * 1024, vB,
             __builtin_amdgcn_readfirstlane((uint32_t)(64 * wave * g.ldb) + kt * 16u));
    } else {
      if (s_on) {
        const int w0 = ((s_row + 2 * kt) & ~3) + 4 * s_half;
        dma4(rS, base + H_A_ST + H_B_ST + 32 * (wave - 4), (uint32_t)w0);
        if (w0 + 4 > s_range && w0 < s_range) {
          // the loads below complete after the DMA (in order), so their LDS
          // writes land after its zeros; lgkmcnt(0): written before any barrier
          uint8_t* dst = base + H_A_ST + H_B_ST + 4 * sd;
          for (int e = 0; e < 4; ++e)
            if (w0 + e < s_range) dst[e] = s_tile[w0 + e];
          __builtin_amdgcn_s_waitcnt(0xC07F);
        }
      }
    }
  };

  AccT<H_TMI, H_TNI> acc;
#pragma unroll
  for (int i = 0; i < H_TMI; ++i)
#pragma unroll
    for (int j = 0; j < H_TNI; ++j) acc[i][j] = v16f{};

  // low-rank term first, in the ring's last buffer (unused by the fill); its
  // loads are issued before the fill's and awaited by count
  const int rho = g.ra + g.rb;
  const int nfill = min(H_NS - 1, nkt);
  uint8_t* lr_smem = smem + (H_NS - 1) * H_STAGE;
  PRegs<H_TMI, H_CHUNK> pr;
  if (rho > 0) lowrank_load<H_TMI, H_TNI, 8, H_BN, H_CHUNK>(pr, g, lr_smem, 0, m0, n0, wave, lane, wm, l32, lh);
#pragma unroll
  for (int s = 0; s < H_NS - 1; ++s)
    if (s < nkt) issue(s, s);
  if (rho > 0) {
    compiler_fence();
    wait_stages(nfill);
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    lowrank_mma<H_TMI, H_TNI, H_BN, H_CHUNK>(acc, pr, g, lr_smem, 0, lane, wn);
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (rho > H_CHUNK)
      lowrank_into_acc<H_TMI, H_TNI, 8, H_BN, H_CHUNK>(acc, g, lr_smem, m0, n0, tid, wave, wm, wn, l32, lh,
                                                       H_CHUNK);
  }

  // Main loop.  Iteration kt: read k-step 1's A of stage kt, run k-step 0; wait
  // for this wave's DMA of stage kt+1, barrier (all of stage kt+1 landed; every
  // wave done with stage kt-1), read k-step 0's A and the B data of stage kt+1;
  // run k-step 1, issuing the DMA of stage kt+NS-1 into stage kt-1's buffer
  // halfway.  B of k-step 1 is dequantized before its codes are replaced.
  if (nkt > 0) {
    AFrag c0, p1;
    BFrag bf;
    v8bf b0[H_TNI], b1[H_TNI];
    compiler_fence();
    wait_stages(nfill - 1);
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    read_a(c0, smem, 0, wm, l32, lh);
    read_b(bf, smem, 0, srs4, wn, l32, lh);
    for (int kt = 0; kt < nkt; ++kt) {
      const uint8_t* st = smem + __builtin_amdgcn_readfirstlane((kt % H_NS) * H_STAGE);
      read_a(p1, st, 1, wm, l32, lh);
      if (k_tail && kt == nkt - 1 && lh) {   // elements 16 .. 31 of the last stage are past K:
#pragma unroll                                // zero codes and zero A (both, so no 0 * inf)
        for (int i = 0; i < H_TMI; ++i) c0.a[i] = p1.a[i] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < H_TNI; ++j) bf.codes[j] = v2i{0, 0};
      }
      dequant_b<0>(b0, bf);
      dequant_b<1>(b1, bf);
      __builtin_amdgcn_sched_barrier(0);
      mma_rows<0, H_TMI>(acc, c0, b0);
      pin_acc(acc);
      pin_b(b1);
      __builtin_amdgcn_sched_barrier(0);
      // (also in the last iteration, where the reads fetch an unused buffer: no
      // branch around them, so the LDS counter stays straight-line for the MFMAs)
      compiler_fence();
      wait_stages(max(0, min(H_NS - 3, nkt - kt - 2)));
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      const uint8_t* nx = smem + __builtin_amdgcn_readfirstlane(((kt + 1) % H_NS) * H_STAGE);
      read_a(c0, nx, 0, wm, l32, lh);
      read_b(bf, nx, kt + 1, srs4, wn, l32, lh);
      __builtin_amdgcn_sched_barrier(0);
      mma_rows<0, H_TMI / 2>(acc, p1, b1);
      pin_acc(acc);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + H_NS - 1 < nkt) issue((kt + H_NS - 1) % H_NS, kt + H_NS - 1);
      __builtin_amdgcn_sched_barrier(0);
      mma_rows<H_TMI / 2, H_TMI>(acc, p1, b1);
    }
  }
  compiler_fence();
  __builtin_amdgcn_s_barrier();   // every wave done reading the ring
  compiler_fence();
  if constexpr (OUT_BF16)
    store_acc_bf16_lds<H_TMI, H_TNI, 8, H_BM, H_BN>(acc, g, smem, m0, n0, tid, wm, wn, l32, lh);
  else
    store_acc<false, H_TMI, H_TNI>(acc, g, m0, n0, lane, wm, wn, l32, lh);
}

}  // namespace

ft_status launch_gemm_a16(const GemmArgs& g, bool out_bf16, bool trans_b, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return FT_OK;
  const int64_t tiles_m = (g.M + H_BM - 1) / H_BM, tiles_n = (g.N + H_BN - 1) / H_BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles >= ((int64_t)1 << 28)) return FT_ESHAPE;
  // 32-bit buffer offsets: a tile's rows of A and B, the scale rows
  if (H_BM * g.lda >= ((int64_t)1 << 31) || H_BN * g.ldb >= ((int64_t)1 << 31) ||
      (g.N / 16) * g.sB_rs >= ((int64_t)1 << 31))
    return FT_ESHAPE;
  const int per_xcd = (int)((tiles + 7) / 8);
  const dim3 grid((unsigned)(8 * per_xcd)), block(512);
  const int tm = (int)tiles_m, tn = (int)tiles_n;
  if (out_bf16) {
    if (trans_b) hipLaunchKernelGGL((gemm_a16_kernel<true, true>), grid, block, 0, s, g, tm, tn, per_xcd);
    else hipLaunchKernelGGL((gemm_a16_kernel<true, false>), grid, block, 0, s, g, tm, tn, per_xcd);
  } else {
    if (trans_b) hipLaunchKernelGGL((gemm_a16_kernel<false, true>), grid, block, 0, s, g, tm, tn, per_xcd);
    else hipLaunchKernelGGL((gemm_a16_kernel<false, false>), grid, block, 0, s, g, tm, tn, per_xcd);
  }
  return launch_status();
}

}  // namespace ft
