// Block-scaled 4-bit GEMM with the low-rank up-projection fused in its epilogue.
//
//   C[m][n] = sum_k deq(A)[m][k] deq(B)[n][k]  +  sum_j P[m][j] W[j][n]
//
// forward  (FourTune Eq. 2):  A = Q(X) [M x K], B = Q(R) [N x K], P = T, W = [L2; B]
// backward (FourTune Eq. 3):  A = Q(G) [M x N], B = Q(R)^T [K x N] (R's column-major
//                             codes and transposed scale grid), P = V, W = [L1^T; A^T]
// Section 3.2 of the paper: with 16x16 blocks the transposed product reads the
// same codes and the same block scales, only laid out transposed, so Q(R) is
// never dequantized or re-quantized.  Section 3.3 "LoRA Fusion": the
// up-projections are accumulated into the backbone GEMM's accumulators before
// the single store of C.
//
// How 16x16 scales reach the MFMA (scale path "S2"): gfx950's
// v_mfma_scale_f32_32x32x64_f8f6f4 gives each lane 32 consecutive K values of
// one row (or column) and ONE power-of-two (E8M0) scale for them.  A 16x16
// block changes scale every 16 K, so each lane carries exactly one 16-K block
// in the low half of its 32-slot fragment and zeros in the high half; the two
// lane halves of the wave carry two different blocks.  The hardware applies the
// power-of-two scales exactly, so the result is the exact dequantized product
// accumulated in fp32.  Half of each MFMA's K slots carry data.
//
// Kernels (all of them 8 waves, two per SIMD, so one wave's LDS or barrier wait
// overlaps the other's MFMAs; K advances 128 elements = 64 code bytes per row,
// 8 blocks, per stage):
//
// Pipelined kernel, one workgroup per output tile (reduction length a multiple
// of 128): a 4-stage LDS ring filled by buffer_load ... lds (global -> LDS
// without registers).  Each DMA instruction writes 1 KiB = 16 tile rows
// contiguously; the 16-byte-chunk XOR swizzle that keeps the fragment reads
// conflict-free is applied by choosing which global chunk each lane fetches.
// Out-of-range rows read as zero (buffer range check).  One barrier per stage;
// each wave waits only for its own DMA of the stage about to be consumed
// (explicit vmcnt), keeping 2 stages in flight.  Tiles are mapped XCD-aware:
// consecutive workgroups land on different XCDs, so the linear id is re-grouped
// such that each XCD works on a compact block of output tiles (shared A/B panels
// in that XCD's L2).  Tile shapes: 256 x 256, 192 x 384 (when it fills the CUs
// in fewer partial rounds), and 128 x 128 for products with fewer big tiles
// than CUs, with an optional split of the reduction (fp32 partial tiles summed
// in split order by a second kernel).
//
// Generic kernel (any multiple-of-16 reduction length): 4 waves of 128 x 128,
// register-staged double buffer with per-chunk bounds checks; used only when
// K % 128 != 0.
//
// Low-rank term: W's slice is staged transposed in LDS; P is split into bf16
// hi + lo (hi + lo = P to 2^-16 relative) and multiplied on bf16 MFMA 32x32x16,
// so the fp32 low-rank intermediate keeps ~16 bits.  The pipelined kernel adds
// its last ranks (up to one pass) after the 4-bit products when their tiles fit
// the ring buffers the last stages free (loaded during those stages), and the
// others before them, in passes of up to CHUNK ranks.  The split depends on the
// tile shape, the ranks and the stage count only, not on the epilogue, so the
// launches of a shape sum each output in the same order (the generic kernel
// adds the whole term after the products).
#include "ft_common.h"
#include "ft_device.h"
#include "ft_internal.h"
#include "gemm_tile.h"

namespace ft {
// (tile configurations have external linkage: kernels templated on an
//  internal-linkage type get no host launch stub)
constexpr int TC_BKB = 64;
constexpr int tc_max(int a, int b) { return a > b ? a : b; }
// Tile configurations: BM x BN per workgroup, 8 waves in WM x (8 / WM), each
// wave (32*TMI) x (32*TNI).  The square 256 x 256 tile is the default; the
// 192 x 384 tile (same operand bytes per FLOP) is taken when it fills the chip
// in fewer partial rounds, e.g. 4608 x 12288 = 768 tiles = 3 full rounds on
// 256 CUs where 256 x 256 gives 864 tiles = 3.4 rounds.
// GS: scale granularity.  0: 16x16 blocks (the method's); 16 or 32: 1 x GS
// groups along each row (section 4.3's group-wise setting, and the group the
// block-scaled MFMA takes per scale), scale bytes [rows][K / GS].
template <int BM_, int BN_, int WM_, int TMI_, int NS_, int CHUNK_, int GS_ = 0>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = 8 / WM_, TMI = TMI_;
  static constexpr int TNI = BN_ / (8 / WM_) / 32;
  static constexpr int NS = NS_, CHUNK = CHUNK_, GS = GS_;
  static constexpr int A_ST = BM * TC_BKB, B_ST = BN * TC_BKB;
  // scale dwords per stage: two per 16-row block, or 128 / GS bytes per row
  static constexpr int DPR = GS ? 128 / GS / 4 : 0;                   // ... dwords per row (group modes)
  static constexpr int SA_DW = GS ? BM * DPR : BM / 16 * 2, SB_DW = GS ? BN * DPR : BN / 16 * 2;
  static constexpr int STAGE = A_ST + B_ST + (SA_DW + SB_DW) * 4;
  static constexpr int N16 = (BM + BN) / 16;                          // 1-KiB DMAs per stage
  static constexpr int NQ = (N16 + 7) / 8;                            // ... per wave, at most
  // Scale DMAs go to the waves with one code DMA fewer (waves [FS, 8)), or to
  // every wave when the code DMAs divide evenly, so that every wave issues the
  // same number DPS of DMA instructions per stage (compile-time wait counts).
  // Of the SW scale waves, the first WA fetch A's scale dwords, the others B's.
  static constexpr int FS = N16 % 8, SW = 8 - FS;
  // group modes: the scale dwords take SQ whole 64-lane DMA instructions,
  // spread evenly over the waves (A's first, then B's)
  static constexpr int SQ = (SA_DW + SB_DW) / 64;
  static constexpr int DPS = GS ? NQ + SQ / 8 : (FS ? NQ : NQ + 1);
  static constexpr int WA_RAW = (SW * SA_DW + (SA_DW + SB_DW) / 2) / (SA_DW + SB_DW);
  static constexpr int WA = WA_RAW < 1 ? 1 : (WA_RAW > SW - 1 ? SW - 1 : WA_RAW);
  static constexpr int LA = (SA_DW + WA - 1) / WA, LB = (SB_DW + (SW - WA) - 1) / (SW - WA);
  static constexpr int W_PITCH = 2 * BN + 32;                          // low-rank W rows in LDS
  static constexpr int SMEM = tc_max(tc_max(NS * STAGE, (NS - 1) * STAGE + CHUNK * W_PITCH),
                                     BM * (2 * BN + 64));                 // bf16 output tile image
  static_assert(BM == WM * 32 * TMI && BN == WN * 32 * TNI, "tile shape");
  static_assert(GS || (SW >= 2 && LA <= 64 && LB <= 64), "scale DMA split");
  // every scale wave has at least one dword to fetch
  static_assert(GS || ((WA - 1) * LA < SA_DW && (SW - WA - 1) * LB < SB_DW), "idle scale wave");
  static_assert(!GS || (FS == 0 && SA_DW % 64 == 0 && SB_DW % 64 == 0 && SQ % 8 == 0), "group-mode DMA split");
  static_assert(SMEM <= 160 * 1024, "LDS");
};
// CHUNK: ranks per low-rank pass; its W rows (pitch 2 BN + 32 bytes) go to the
// last stage buffer (and the LDS beyond the ring where they need more)
using CfgSquare = TileCfg<256, 256, 4, 2, 4, 48>;
using CfgWide = TileCfg<192, 384, 2, 3, 4, 48>;
// 128 x 128 tile (8 waves of 64 x 32) for products too small to give every CU a
// 256 x 256 tile (few rows, e.g. the 512 text tokens of a FLUX block): four
// times the tiles, two workgroups per CU (66 KiB of LDS each)
using CfgSmall = TileCfg<128, 128, 2, 2, 4, 64>;
template <int I, int GS = 0> struct CfgOf { using type = TileCfg<256, 256, 4, 2, 4, 48, GS>; };
template <> struct CfgOf<1, 0> { using type = CfgWide; };
template <> struct CfgOf<2, 0> { using type = CfgSmall; };
constexpr int cfg_occ(int cfg) { return cfg == 2 ? 2 : 1; }   // workgroups per CU the kernel is built for
// Most low-rank ranks (a multiple of 16, at most one pass of `chunk`) whose W
// rows [nt x bn] bf16 and P rows [bm x nt] fp32 each fit one ring buffer of
// `stage` bytes, with P in whole 1-KiB DMAs: the ranks the pipelined kernel
// adds after its main loop (256 x 256: 32, 192 x 384: 48, 128 x 128: 32)
constexpr int tail_ranks_max(int bm, int bn, int stage, int chunk) {
  int nt = chunk - chunk % 16;
  while (nt > 0 && (nt * 2 * bn > stage || bm * nt * 4 > stage || (bm * nt) % 256 != 0)) nt -= 16;
  return nt;
}
static_assert(tail_ranks_max(256, 256, CfgSquare::STAGE, CfgSquare::CHUNK) == 32, "square tail ranks");
static_assert(tail_ranks_max(192, 384, CfgWide::STAGE, CfgWide::CHUNK) == 48, "wide tail ranks");
static_assert(tail_ranks_max(128, 128, CfgSmall::STAGE, CfgSmall::CHUNK) == 32, "small tail ranks");
}  // namespace ft

namespace ft {
namespace {


constexpr int BM = 256, BN = 256;
constexpr int GT = 256;                         // threads, generic kernel (4 waves, 128 x 128 each)
constexpr int PGT = 512;                        // threads, pipelined kernel (8 waves, 64 x 128 each)
constexpr int A_ST = BM * BKB, B_ST = BN * BKB;
constexpr int S_ST = (BM / 16) * 8 + (BN / 16) * 8;   // A scales [16][8] then B scales [16][8]
constexpr int STAGE = A_ST + B_ST + S_ST;
constexpr int NS = 4;                           // pipeline depth (stages)
constexpr int PIPE_LDS = NS * STAGE;
constexpr int GEN_LDS = 2 * STAGE;
constexpr int EPI_LDS = 64 * 544;               // W chunk of the epilogue (64 ranks, 256-wide tile)
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int PIPE_SMEM = cmax(PIPE_LDS, EPI_LDS);
constexpr int GEN_SMEM = cmax(GEN_LDS, EPI_LDS);


// One 128-K stage for this wave's (32*TMI) x (32*TNI) sub-tile of a BMc x BNc
// workgroup tile (TMI*TNI MFMAs per k-step).  Stage layout: A codes [BMc][64],
// B codes [BNc][64], A scales [BMc/16][8], B scales [BNc/16][8].
template <int TMI, int TNI, int BMc, int BNc>
__device__ __forceinline__ void mfma_stage(AccT<TMI, TNI>& acc, const uint8_t* st, int wm, int wn, int l32, int lh) {
  const uint8_t* As = st;
  const uint8_t* Bs = st + BMc * BKB;
  const uint8_t* SAs = Bs + BNc * BKB;
  const uint8_t* SBs = SAs + (BMc / 16) * 8;
  v4i af[TMI][2], bf[TNI][2];
  int sa[TMI], sb[TNI];
#pragma unroll
  for (int i = 0; i < TMI; ++i) {
    const int ra = wm * 32 * TMI + 32 * i + l32;
    af[i][0] = *reinterpret_cast<const v4i*>(As + swz(ra, 2 * lh));
    af[i][1] = *reinterpret_cast<const v4i*>(As + swz(ra, 2 * lh + 1));
    sa[i] = *reinterpret_cast<const int*>(SAs + (ra >> 4) * 8 + 4 * lh);
  }
#pragma unroll
  for (int i = 0; i < TNI; ++i) {
    const int rbn = wn * 32 * TNI + 32 * i + l32;
    bf[i][0] = *reinterpret_cast<const v4i*>(Bs + swz(rbn, 2 * lh));
    bf[i][1] = *reinterpret_cast<const v4i*>(Bs + swz(rbn, 2 * lh + 1));
    sb[i] = *reinterpret_cast<const int*>(SBs + (rbn >> 4) * 8 + 4 * lh);
  }
  // k-step KK: each lane's 16-K block (8 code bytes) = bytes [8KK, 8KK+8) of its 32-byte
  // half row; the E8M0 scale of that block is byte KK of the scale dword (op_sel = KK).
#define FT_KSTEP(KK)                                                                              \
  _Pragma("unroll") for (int i = 0; i < TMI; ++i) {                                                 \
    const v8i aop = {af[i][(KK) >> 1][((KK) & 1) * 2], af[i][(KK) >> 1][((KK) & 1) * 2 + 1], 0, 0, 0, 0, 0, 0}; \
    _Pragma("unroll") for (int j = 0; j < TNI; ++j) {                                             \
      const v8i bop = {bf[j][(KK) >> 1][((KK) & 1) * 2], bf[j][(KK) >> 1][((KK) & 1) * 2 + 1], 0, 0, 0, 0, 0, 0}; \
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop, acc[i][j], 4, 4, KK, sa[i], KK, sb[j]); \
    }                                                                                             \
  }
  FT_KSTEP(0)
  FT_KSTEP(1)
  FT_KSTEP(2)
  FT_KSTEP(3)
#undef FT_KSTEP
}

// The same stage split for software pipelining: part P holds k-steps 2P and 2P+1
// (one 16-byte read per row tile and operand); the scale dwords cover all four.
template <int TMI, int TNI>
struct Part {
  v4i a[TMI], b[TNI];
};

template <int TMI, int TNI, int BMc, int BNc>
__device__ __forceinline__ void read_part(Part<TMI, TNI>& f, const uint8_t* st, int p, int wm, int wn, int l32,
                                          int lh) {
#pragma unroll
  for (int i = 0; i < TMI; ++i)
    f.a[i] = *reinterpret_cast<const v4i*>(st + swz(wm * 32 * TMI + 32 * i + l32, 2 * lh + p));
#pragma unroll
  for (int j = 0; j < TNI; ++j)
    f.b[j] = *reinterpret_cast<const v4i*>(st + BMc * BKB + swz(wn * 32 * TNI + 32 * j + l32, 2 * lh + p));
}

template <int TMI, int TNI, int BMc, int BNc>
__device__ __forceinline__ void read_scales(int (&sa)[TMI], int (&sb)[TNI], const uint8_t* st, int wm, int wn,
                                            int l32, int lh) {
  const uint8_t* SAs = st + (BMc + BNc) * BKB;
  const uint8_t* SBs = SAs + (BMc / 16) * 8;
#pragma unroll
  for (int i = 0; i < TMI; ++i)
    sa[i] = *reinterpret_cast<const int*>(SAs + ((wm * 32 * TMI + 32 * i + l32) >> 4) * 8 + 4 * lh);
#pragma unroll
  for (int j = 0; j < TNI; ++j)
    sb[j] = *reinterpret_cast<const int*>(SBs + ((wn * 32 * TNI + 32 * j + l32) >> 4) * 8 + 4 * lh);
}

// k-step KK of a stage from its part (KK >> 1).  A 16-byte read holds the lane's
// blocks of k-steps 2P (dwords 0-1) and 2P+1 (dwords 2-3).  A goes in whole; B
// keeps only the k-step's block and zeros in the other half, so the products of
// A's other block vanish (E2M1 has no infinities or NaNs: zero times any code is
// zero).  Both operands take scale byte KK (op_sel): A's other block is never
// scaled into the sum.  Only B needs a padded copy, one per column tile.
template <int KK, int TMI, int TNI>
__device__ __forceinline__ void mma_kstep(AccT<TMI, TNI>& acc, const Part<TMI, TNI>& f, const int (&sa)[TMI],
                                          const int (&sb)[TNI]) {
  const v4i z = {0, 0, 0, 0};
  v8i bop[TNI];
#pragma unroll
  for (int j = 0; j < TNI; ++j) {
    const v4i bv = f.b[j];
    bop[j] = (KK & 1) ? __builtin_shufflevector(bv, z, 4, 4, 2, 3, 4, 4, 4, 4)
                      : __builtin_shufflevector(bv, z, 0, 1, 4, 4, 4, 4, 4, 4);
  }
#pragma unroll
  for (int i = 0; i < TMI; ++i) {
    const v4i av = f.a[i];
    const v8i aop = __builtin_shufflevector(av, z, 0, 1, 2, 3, 4, 4, 4, 4);
#pragma unroll
    for (int j = 0; j < TNI; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop[j], acc[i][j], 4, 4, KK, sa[i], KK, sb[j]);
  }
}

// Group modes (per-row scales, bytes [rows][K / GS]; in LDS one row after
// another, DPR dwords each, A's rows then B's).  1 x 16: the lane's dword holds
// the scales of its four 16-K blocks (k-steps 0-3), as in the 16x16 layout.
// 1 x 32: part P's 16-byte read is the lane's 32-K group 2 lh + P, so the
// lane's two bytes sit at 2 lh, 2 lh + 1 of its row's dword: shifted down, the
// part selects byte P.
template <int GS, int TMI, int TNI, int BMc, int BNc>
__device__ __forceinline__ void read_scales_g(int (&sa)[TMI], int (&sb)[TNI], const uint8_t* st, int wm, int wn,
                                              int l32, int lh) {
  constexpr int RB = 128 / GS;                                   // scale bytes per row per stage
  const uint8_t* SAs = st + (BMc + BNc) * BKB;
  const uint8_t* SBs = SAs + BMc * RB;
#pragma unroll
  for (int i = 0; i < TMI; ++i) {
    const int r = wm * 32 * TMI + 32 * i + l32;
    if constexpr (GS == 16) sa[i] = *reinterpret_cast<const int*>(SAs + r * RB + 4 * lh);
    else sa[i] = (int)(*reinterpret_cast<const uint32_t*>(SAs + r * RB) >> (16 * lh));
  }
#pragma unroll
  for (int j = 0; j < TNI; ++j) {
    const int r = wn * 32 * TNI + 32 * j + l32;
    if constexpr (GS == 16) sb[j] = *reinterpret_cast<const int*>(SBs + r * RB + 4 * lh);
    else sb[j] = (int)(*reinterpret_cast<const uint32_t*>(SBs + r * RB) >> (16 * lh));
  }
}

// 1 x 32 groups: one MFMA per tile covers part P's 64 K (every K slot carries
// data), rows I0 .. I1-1 of the wave's tiles.
template <int P, int I0, int I1, int TMI, int TNI>
__device__ __forceinline__ void mma_full(AccT<TMI, TNI>& acc, const Part<TMI, TNI>& f, const int (&sa)[TMI],
                                         const int (&sb)[TNI]) {
  const v4i z = {0, 0, 0, 0};
#pragma unroll
  for (int i = I0; i < I1; ++i) {
    const v8i aop = __builtin_shufflevector(f.a[i], z, 0, 1, 2, 3, 4, 4, 4, 4);
#pragma unroll
    for (int j = 0; j < TNI; ++j) {
      const v8i bop = __builtin_shufflevector(f.b[j], z, 0, 1, 2, 3, 4, 4, 4, 4);
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop, acc[i][j], 4, 4, P, sa[i], P, sb[j]);
    }
  }
}

template <int P, int TMI, int TNI>
__device__ __forceinline__ void mma_part(AccT<TMI, TNI>& acc, const Part<TMI, TNI>& f, const int (&sa)[TMI],
                                         const int (&sb)[TNI]) {
  mma_kstep<2 * P>(acc, f, sa, sb);
  mma_kstep<2 * P + 1>(acc, f, sa, sb);
}


// MLP fusion epilogue (FourTune section 3.3 "MLP Fusion": the first linear's
// GEMM carries the activation and the quantization of the next linear's input).
// The tile of Y (bf16) goes through the LDS image as in store_acc_bf16_lds; each
// thread stores its 16-byte pieces of Y, then h = GELU(Y) (fp32 math on the bf16
// value, rounded to bf16) to H and back into the image; then Q(h) (16 x 16
// blocks, power-of-two scales, E2M1 codes, the ft_quant_block16 rule) from the
// image: 16 lanes per block, one block row per lane, the block maximum by DPP
// within the 16 lanes.  Codes row-major [M][N/2], scales [M/16][N/16].
template <int TMI, int TNI, int NWAVES, int BMc, int BNc>
__device__ __forceinline__ void store_gelu_quant_lds(AccT<TMI, TNI>& acc, const GemmArgs& g, uint8_t* smem,
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
  constexpr int PER = BMc * CH / (64 * NWAVES);
  static_assert(BMc * CH % (64 * NWAVES) == 0, "whole passes over the tile");
  uint16_t* Y = static_cast<uint16_t*>(g.C);
  uint16_t* H = static_cast<uint16_t*>(g.H);
  v4i val[PER];
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int e = tid + 64 * NWAVES * it, r = e / CH, c = e - (e / CH) * CH;
    val[it] = *reinterpret_cast<const v4i*>(smem + r * PITCH + 16 * c);
  }
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int e = tid + 64 * NWAVES * it, r = e / CH, c = e - (e / CH) * CH;
    const int64_t row = m0 + r, col = n0 + 8 * c;
    const bool in = row < g.M && col < g.N;
    if (in) *reinterpret_cast<v4i*>(Y + row * g.ldc + col) = val[it];
    const uint32_t w[4] = {(uint32_t)val[it].x, (uint32_t)val[it].y, (uint32_t)val[it].z, (uint32_t)val[it].w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = f32_to_bf16_rne(gelu_f(bf16lo_to_f32(w[k]))) | (f32_to_bf16_rne(gelu_f(bf16hi_to_f32(w[k]))) << 16);
    const v4i hv = {(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    if (in) *reinterpret_cast<v4i*>(H + row * g.ldc + col) = hv;
    *reinterpret_cast<v4i*>(smem + r * PITCH + 16 * c) = hv;
  }
  compiler_fence();
  __syncthreads();
  compiler_fence();
  constexpr int BC = BNc / 16, NBLK = (BMc / 16) * BC;          // blocks per tile
  constexpr int GROUPS = 64 * NWAVES / 16;                      // 16-lane groups
  const int grp = tid >> 4, li = tid & 15;
#pragma unroll 1
  for (int b = grp; b < NBLK; b += GROUPS) {                    // uniform within each 16-lane group
    const int br = b / BC, bc = b - (b / BC) * BC, r = 16 * br + li;
    const v4i x0 = *reinterpret_cast<const v4i*>(smem + r * PITCH + 32 * bc);
    const v4i x1 = *reinterpret_cast<const v4i*>(smem + r * PITCH + 32 * bc + 16);
    const uint32_t d[8] = {(uint32_t)x0.x, (uint32_t)x0.y, (uint32_t)x0.z, (uint32_t)x0.w,
                           (uint32_t)x1.x, (uint32_t)x1.y, (uint32_t)x1.z, (uint32_t)x1.w};
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = max(m, max(d[k] & 0x7fffu, (d[k] >> 16) & 0x7fffu));
    const int E = pow2_exp_bf16(dpp_max16(m));
    const float sc = __builtin_bit_cast(float, (uint32_t)(E + 127) << 23);
    uint32_t c0 = 0, c1 = 0;   // byte k of c0 / c1: codes of values 2k, 2k+1 / 8+2k, 9+2k (low nibble first)
#define FT_CVT2(K)                                                                          \
    c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c0, __builtin_bit_cast(v2bf, d[K]), sc, K); \
    c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c1, __builtin_bit_cast(v2bf, d[4 + K]), sc, K);
    FT_CVT2(0)
    FT_CVT2(1)
    FT_CVT2(2)
    FT_CVT2(3)
#undef FT_CVT2
    const int64_t row = m0 + r, col = n0 + 16 * bc;
    if (row < g.M && col < g.N) {
      *reinterpret_cast<v2i*>(g.hq + row * (g.N / 2) + col / 2) = v2i{(int)c0, (int)c1};
      if (li == 0) g.hs[(row / 16) * (g.N / 16) + col / 16] = (uint8_t)(E + 127);
    }
  }
}


// ---------------------------------------------------------------------------------------
// Pipelined kernel (K % 128 == 0)
// ---------------------------------------------------------------------------------------


// TRANS_B: backward instantiation (B = Q(R)^T); same code, separate name in profiles.
// GELU_Q: MLP fusion epilogue (store_gelu_quant_lds; forward, bf16 Y)
// GS: scale granularity (TileCfg); the group modes use the square tile.
// SPLIT: split reduction (GemmArgs::splits, ::part): work item v = s * tiles + t
// takes split s of tile t and stores its fp32 partial tile; split 0 alone adds
// the low-rank term.
// ANRT > 0: workgroups past the GEMM's 8 * per_xcd compute the adapter
// gradients of g_in.ad (adapter_tile.h; r <= 32 ANRT) in chunks of AD_CH tokens
// per wave.

template <bool OUT_BF16, bool TRANS_B, int CFG, bool GELU_Q = false, int GS = 0, bool SPLIT = false,
          int ANRT = 0>
__global__ void __launch_bounds__(PGT, cfg_occ(CFG))   // CFG: 0 square, 1 wide, 2 small tile
gemm_w4a4_kernel(GemmArgs g_in, int tiles_m, int tiles_n, int per_xcd) {
  using C = typename CfgOf<CFG, GS>::type;
  static_assert(!(SPLIT && GELU_Q), "the MLP fusion epilogue needs the whole reduction");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::SMEM];
  if constexpr (ANRT > 0) {
    static_assert(ad_lds_bytes(AD_CH) <= C::SMEM && PGT == AD_WAVES * 64, "adapter workgroup");
    const int wg = (int)blockIdx.x - 8 * per_xcd;
    if (wg >= 0) {
      adapter_run<AD_CH, ANRT>(g_in.ad, wg, smem);
      return;
    }
  }
  constexpr int BMc = C::BM, BNc = C::BN, NSc = C::NS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int l32 = lane & 31, lh = lane >> 5;

  // XCD-aware raster: hardware places workgroup b on XCD b % 8
  const int b = blockIdx.x;
  int v = (b & 7) * per_xcd + (b >> 3);
  const int ntile = tiles_m * tiles_n;
  if (v >= ntile * (SPLIT ? g_in.splits : 1)) return;
  int sp = 0;                                                  // split of the reduction
  if constexpr (SPLIT) {
    sp = v / ntile;
    v -= sp * ntile;
  }
  GemmArgs g = g_in;
  if (sp) g.ra = g.rb = 0;                                     // the low-rank term: split 0 only
  const int grp = v / (GROUP_M * tiles_n);
  const int first_m = grp * GROUP_M;
  const int gm = min(GROUP_M, tiles_m - first_m);
  const int in_grp = v - grp * GROUP_M * tiles_n;
  const int64_t m0 = (int64_t)(first_m + in_grp % gm) * BMc;
  const int64_t n0 = (int64_t)(in_grp / gm) * BNc;
  // stages [k0, k0 + nkt) of the reduction
  const int nk_all = (int)(g.K / 128);
  int k0 = 0, nkt = nk_all;
  if constexpr (SPLIT) {
    k0 = (int)((int64_t)sp * nk_all / g.splits);
    nkt = (int)((int64_t)(sp + 1) * nk_all / g.splits) - k0;
  }

  // buffer resources for this tile; rows past M / N fall outside the range and read 0
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.A + m0 * g.lda), 0, (int)(min<int64_t>(BMc, g.M - m0) * g.lda), RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.B + n0 * g.ldb), 0, (int)(min<int64_t>(BNc, g.N - n0) * g.ldb), RSRC_FLAGS);
  const bool scale_w = wave >= C::FS;                          // this wave fetches scale dwords
  const bool scale_b = wave >= C::FS + C::WA;
  const __amdgpu_buffer_rsrc_t rS = scale_b
      ? __builtin_amdgcn_make_buffer_rsrc((void*)(g.sB + (n0 / 16) * g.sB_rs), 0,
                                          (int)(min<int64_t>(BNc / 16, (g.N - n0) / 16) * g.sB_rs), RSRC_FLAGS)
      : __builtin_amdgcn_make_buffer_rsrc((void*)(g.sA + (m0 / 16) * g.sA_rs), 0,
                                          (int)(min<int64_t>(BMc / 16, (g.M - m0) / 16) * g.sA_rs), RSRC_FLAGS);
  const int64_t s_rs = scale_b ? g.sB_rs : g.sA_rs;

  // DMA instruction q (0 .. N16-1) of a stage fills 16 rows: A rows 16q .. for
  // q < BM/16, else B rows; wave w issues q = w, w + 8, ...  Lane l lands at
  // physical chunk l & 3 of row l >> 2 (the swizzle picks the global chunk; its
  // row bits 2-3 are lane bits 4-5 since every DMA starts at a multiple of 16
  // rows).  The lane's part of the offset is one register per operand; the
  // row-block and stage parts are wave-uniform (scalar offset).
  const int nq = (C::N16 - wave + 7) / 8;                      // this wave's count (uniform)
  const uint32_t lane_chunk = 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
  const uint32_t vA = (uint32_t)((lane >> 2) * g.lda) + lane_chunk;
  const uint32_t vB = (uint32_t)((lane >> 2) * g.ldb) + lane_chunk;
  // scale dwords: A's are [BM/16][2], B's [BN/16][2]; wave w of its group takes a
  // contiguous run of LA (LB) of them, one per lane
  const int sw = scale_b ? wave - C::FS - C::WA : wave - C::FS;
  const int sl = scale_b ? C::LB : C::LA;
  const int sd = sw * sl + lane;
  const bool s_on = scale_w && lane < sl && sd < (scale_b ? C::SB_DW : C::SA_DW);
  const uint32_t offS = (uint32_t)((sd >> 1) * s_rs + 4 * (sd & 1));
  const int s_lds = C::A_ST + C::B_ST + 4 * ((scale_b ? C::SA_DW : 0) + sw * sl);
  // group modes: the scale rows of the tile's A and B rows ([rows][K / GS] bytes)
  const __amdgpu_buffer_rsrc_t rSA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.sA + m0 * g.sA_rs), 0, (int)(min<int64_t>(BMc, g.M - m0) * g.sA_rs), RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rSB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.sB + n0 * g.sB_rs), 0, (int)(min<int64_t>(BNc, g.N - n0) * g.sB_rs), RSRC_FLAGS);

  auto issue = [&](int stage, int kt) {
    uint8_t* base = smem + stage * C::STAGE;
#pragma unroll
    for (int u = 0; u < C::NQ; ++u) {
      const int q = wave + 8 * u;
      if (u < nq) {
        const bool isb = q >= BMc / 16;
        const int r0 = isb ? 16 * q - BMc : 16 * q;
        const uint32_t soff = (uint32_t)(r0 * (isb ? g.ldb : g.lda)) + (uint32_t)(k0 + kt) * BKB;
        dma16s(isb ? rB : rA, base + (isb ? C::A_ST : 0) + r0 * BKB, isb ? vB : vA,
               __builtin_amdgcn_readfirstlane(soff));
      }
    }
    if constexpr (C::GS == 0) {
      if (scale_w) {   // wave-uniform: the instruction counts even where no lane is active
        if (s_on) dma4(rS, base + s_lds, offS + (uint32_t)(k0 + kt) * 8);
      }
    } else {
      // scale DMA instruction t = wave + 8u covers scale dwords 64t .. 64t+63 of
      // the stage (A's rows, then B's; each instruction within one of them)
#pragma unroll
      for (int u = 0; u < C::SQ / 8; ++u) {
        const int t = wave + 8 * u;
        const bool isb = t * 64 >= C::SA_DW;
        const int d = t * 64 + lane - (isb ? C::SA_DW : 0);
        const int row = d / C::DPR, part = d - (d / C::DPR) * C::DPR;
        const uint32_t off =
            (uint32_t)(row * (isb ? g.sB_rs : g.sA_rs)) + (uint32_t)((k0 + kt) * (128 / C::GS) + 4 * part);
        dma4(isb ? rSB : rSA, base + C::A_ST + C::B_ST + 256 * t, off);
      }
    }
  };

  AccT<C::TMI, C::TNI> acc;
#pragma unroll
  for (int i = 0; i < C::TMI; ++i)
#pragma unroll
    for (int j = 0; j < C::TNI; ++j) acc[i][j] = v16f{};

  // The low-rank up-projection P W.  Its last nt ranks (all of them, or as many
  // as fit: NT_MAX, whose W and P tiles fit one ring buffer each) follow the
  // main loop when the reduction has at least NS stages:
  // the tiles are fetched during the last stages into buffers those stages have
  // freed (tail_issue_w).  The other ranks go into the accumulators first, in
  // the buffer of stage NS-1 (free until the first steady iteration): the loads
  // of their first chunk are issued ahead of the pipeline fill and awaited by
  // count (the fill's DMAs, all younger, may stay in flight), so both overlap;
  // further chunks follow one by one.  The split depends only on the tile
  // shape, the ranks and the stage count, so every kernel of a shape (plain,
  // MLP-fusion epilogue, adapter workgroups) sums each output in the same order.
  constexpr int NT_MAX = tail_ranks_max(BMc, BNc, C::STAGE, C::CHUNK);
  const int rho = g.ra + g.rb;
  const int nt = rho <= NT_MAX ? rho : NT_MAX;
  const bool tail_lr = rho > 0 && nt > 0 && nkt >= NSc && (BMc * nt) % 256 == 0;
  const int rho_head = tail_lr ? rho - nt : rho;
  uint8_t* lr_smem = smem + (NSc - 1) * C::STAGE;
  PRegs<C::TMI, C::CHUNK> pr;
  if (rho_head > 0)
    lowrank_load<C::TMI, C::TNI, 8, BNc, C::CHUNK>(pr, g, lr_smem, 0, m0, n0, wave, lane, wm, l32, lh, rho_head);
#pragma unroll
  for (int s = 0; s < NSc - 1; ++s)
    if (s < nkt) issue(s, s);
  if (rho_head > 0) {
    compiler_fence();
    if (nkt >= NSc - 1) FT_WAIT_VMCNT(C::DPS * (NSc - 1));
    else if (nkt == 2) FT_WAIT_VMCNT(C::DPS * 2);
    else if (nkt == 1) FT_WAIT_VMCNT(C::DPS);
    else FT_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    lowrank_mma<C::TMI, C::TNI, BNc, C::CHUNK>(acc, pr, g, lr_smem, 0, lane, wn, rho_head);
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (rho_head > C::CHUNK)
      lowrank_into_acc<C::TMI, C::TNI, 8, BNc, C::CHUNK>(acc, g, lr_smem, m0, n0, tid, wave, wm, wn, l32, lh,
                                                         C::CHUNK, rho_head);
  }

  // Main loop, software-pipelined across the stage barrier.  Iteration kt reads
  // part 1 of stage kt, runs part 0's MFMAs, then waits for its own DMA of stage
  // kt+1 and meets the barrier (every wave's DMA of kt+1 visible; every wave done
  // reading stage kt-1, whose buffer then takes stage kt+NS-1), reads part 0 of
  // stage kt+1 and runs part 1's MFMAs, issuing the DMA of stage kt+NS-1 between
  // its two k-steps: the LDS reads of one part are in flight while the MFMAs of
  // the other execute, also across the barrier.  A DMA issued at iteration
  // s-NS+1 is awaited at iteration s-1.  Scheduling barriers keep the compiler
  // from moving the MFMAs across the wait, the barrier and the DMA issue.
  static_assert(NSc == 4, "the wait counts below assume a 4-stage ring");
  Part<C::TMI, C::TNI> c0, p1;   // part 0 (current, then next stage's) and part 1
  int sa[C::TMI], sb[C::TNI], na[C::TMI], nb[C::TNI];
  // steady: stage kt+NS-1 exists, so after kt+1 one more stage (kt+2) is in flight
  auto step = [&](int kt, bool steady) __attribute__((always_inline)) {
    const uint8_t* st = smem + __builtin_amdgcn_readfirstlane((kt % NSc) * C::STAGE);
    read_part<C::TMI, C::TNI, BMc, BNc>(p1, st, 1, wm, wn, l32, lh);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (C::GS == 32) mma_full<0, 0, C::TMI>(acc, c0, sa, sb);
    else mma_part<0>(acc, c0, sa, sb);
    pin_acc(acc);
    __builtin_amdgcn_sched_barrier(0);
    if (steady || kt + 1 < nkt) {
      compiler_fence();
      if (steady || kt + 2 < nkt) FT_WAIT_VMCNT(C::DPS);
      else FT_WAIT_VMCNT(0);
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      if (!steady && tail_lr) {   // from here on the buffer of stage kt-1 is free
        if (kt == nkt - 3) tail_issue_w<8, BNc>(g, smem + ((nkt - 4) % NSc) * C::STAGE, n0, wave, lane, rho_head, nt);
        else if (kt == nkt - 2)
          tail_issue_p<8, BMc>(g, smem + ((nkt - 3) % NSc) * C::STAGE, m0, wave, lane, rho_head, nt);
      }
      const uint8_t* nx = smem + __builtin_amdgcn_readfirstlane(((kt + 1) % NSc) * C::STAGE);
      read_part<C::TMI, C::TNI, BMc, BNc>(c0, nx, 0, wm, wn, l32, lh);
      if constexpr (C::GS) read_scales_g<C::GS, C::TMI, C::TNI, BMc, BNc>(na, nb, nx, wm, wn, l32, lh);
      else read_scales<C::TMI, C::TNI, BMc, BNc>(na, nb, nx, wm, wn, l32, lh);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (C::GS == 32) mma_full<1, 0, C::TMI / 2>(acc, p1, sa, sb);
    else mma_kstep<2>(acc, p1, sa, sb);
    pin_acc(acc);
    __builtin_amdgcn_sched_barrier(0);
    // the next DMA between part 1's two k-steps: its LDS writes then overlap
    // MFMAs instead of the fragment reads just issued
    if (steady) issue((kt + NSc - 1) % NSc, kt + NSc - 1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (C::GS == 32) mma_full<1, C::TMI / 2, C::TMI>(acc, p1, sa, sb);
    else mma_kstep<3>(acc, p1, sa, sb);
#pragma unroll
    for (int i = 0; i < C::TMI; ++i) sa[i] = na[i];
#pragma unroll
    for (int j = 0; j < C::TNI; ++j) sb[j] = nb[j];
  };
  compiler_fence();
  if (nkt >= NSc - 1) FT_WAIT_VMCNT(C::DPS * (NSc - 2));
  else FT_WAIT_VMCNT(0);
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  read_part<C::TMI, C::TNI, BMc, BNc>(c0, smem, 0, wm, wn, l32, lh);
  if constexpr (C::GS) read_scales_g<C::GS, C::TMI, C::TNI, BMc, BNc>(sa, sb, smem, wm, wn, l32, lh);
  else read_scales<C::TMI, C::TNI, BMc, BNc>(sa, sb, smem, wm, wn, l32, lh);
  const int n_steady = max(0, nkt - (NSc - 1));
  int kt = 0;
  for (; kt < n_steady; ++kt) step(kt, true);
  for (; kt < nkt; ++kt) step(kt, false);   // the last NS-1 stages: nothing more to fetch
  if (tail_lr) {
    compiler_fence();
    FT_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    tail_lowrank_mma<C::TMI, C::TNI, BNc, C::CHUNK>(acc, smem + ((nkt - 4) % NSc) * C::STAGE,
                                                    smem + ((nkt - 3) % NSc) * C::STAGE, nt, lane, wm, wn, l32, lh);
  }
  if constexpr (SPLIT) {
    GemmArgs gp = g;                                           // fp32 partial tile of split sp
    gp.C = g.part + (int64_t)sp * g.M * g.N;
    gp.ldc = g.N;
    store_acc<false, C::TMI, C::TNI>(acc, gp, m0, n0, lane, wm, wn, l32, lh);
  } else if constexpr (GELU_Q) {
    static_assert(OUT_BF16 && !TRANS_B, "MLP fusion epilogue: forward, bf16 output");
    compiler_fence();
    __builtin_amdgcn_s_barrier();   // every wave done reading the last stage
    compiler_fence();
    store_gelu_quant_lds<C::TMI, C::TNI, 8, BMc, BNc>(acc, g, smem, m0, n0, tid, wm, wn, l32, lh);
  } else if constexpr (OUT_BF16) {
    compiler_fence();
    __builtin_amdgcn_s_barrier();   // every wave done reading the last stage
    compiler_fence();
    store_acc_bf16_lds<C::TMI, C::TNI, 8, BMc, BNc>(acc, g, smem, m0, n0, tid, wm, wn, l32, lh);
  } else {
    store_acc<OUT_BF16, C::TMI, C::TNI>(acc, g, m0, n0, lane, wm, wn, l32, lh);
  }
}

// ---------------------------------------------------------------------------------------
// Pair-merged operand kernel (scale path "S3"): full 32-K fragments
// ---------------------------------------------------------------------------------------
// Operands are the pair-merged FP6 (E3M2) re-encoding of the quantized matrices
// (ft_quant_block16_op): per row and 128-K group, 64 bytes of pair heads (the
// first 16 of each pair's 24 bytes, pairs 0..3) and 32 bytes of pair tails
// (last 8 bytes, pairs 0, 2, 1, 3); pair scale bytes [rows/16][groups * 8].  A
// lane of the 32x32x64 MFMA takes one whole pair of its row (32 K = 6 dwords) and
// one scale byte when the pair is merged (equal bytes), so every K slot carries
// data.  K-step ks of a stage covers pairs 2ks (lanes 0-31) and 2ks+1 (lanes
// 32-63).  When any lane of a k-step holds an unmerged pair (unequal bytes: an
// exponent gap too wide for E3M2), the wave takes that k-step as two MFMAs per
// tile: A restricted to the first 16 K of each lane's pair (dwords 0-2) with
// scale byte 0 of both operands, then to the last 16 K (dwords 3-5) with byte 1.
// B needs no masking: the zeros of A remove the other half of its products, and
// B's byte 0 / byte 1 are its two blocks' scales (equal when merged).
//
// Stage (128 K), per operand: three [256 rows][32 bytes] regions -- heads of
// pairs 0-1, heads of pairs 2-3, tails (unit 0: pairs 0 and 2, unit 1: pairs 1
// and 3) -- each row's two 16-byte units XOR-swizzled by row bits 2 and 3, so a
// lane's reads of all three regions share one offset.  Then the pair scales
// (A [16][8], B [16][8]).  3-stage LDS ring, 7 DMA instructions per wave per
// stage (one per region and operand, plus scales), one barrier per stage.
constexpr int M6_ROW = 32;                                // bytes per row of a region
constexpr int M6_REG = BM * M6_ROW;                       // one region (8 KiB)
constexpr int M6_OPB = 3 * M6_REG;                        // one operand's regions
constexpr int M6_STAGE = 2 * M6_OPB + 256;
constexpr int M6_NS = 3;
constexpr int M6_DMAS = 7;                                // DMA instructions per wave per stage
constexpr int M6_SMEM = cmax(M6_NS * M6_STAGE, EPI_LDS);

// unit u (0, 1) of a region row, swizzled so 16 consecutive rows hit distinct banks
__device__ __forceinline__ int tswz(int row, int u) {
  return row * M6_ROW + ((u ^ ((row >> 2) & 1) ^ ((row >> 3) & 1)) << 4);
}

__device__ __forceinline__ bool unmerged(int s) { return ((s ^ (s >> 8)) & 0xff) != 0; }

// aoff / boff: this lane's region offset for its first A / B row (rows of the
// other tiles are 32 rows = 1 KiB further; swizzle bits are unchanged).
__device__ __forceinline__ void mfma_stage_m6(AccT<2, 4>& acc, const uint8_t* st, int aoff, int boff, int asc,
                                              int bsc) {
  const uint8_t* A = st;
  const uint8_t* B = st + M6_OPB;
  const uint8_t* S = st + 2 * M6_OPB;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    // this lane's pair: 16-byte head, 8-byte tail (contiguous registers), scale bytes (s1, s2)
    v8i aop[2], bop[4];
    int sA[2], sB[4];
    bool split = false;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const v4i h = *reinterpret_cast<const v4i*>(A + ks * M6_REG + aoff + i * 32 * M6_ROW);
      const v2i t = *reinterpret_cast<const v2i*>(A + 2 * M6_REG + aoff + i * 32 * M6_ROW + 8 * ks);
      aop[i] = v8i{h.x, h.y, h.z, h.w, t.x, t.y, 0, 0};
      sA[i] = (int)(*reinterpret_cast<const uint16_t*>(S + asc + 16 * i + 4 * ks));
      split |= unmerged(sA[i]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4i h = *reinterpret_cast<const v4i*>(B + ks * M6_REG + boff + j * 32 * M6_ROW);
      const v2i t = *reinterpret_cast<const v2i*>(B + 2 * M6_REG + boff + j * 32 * M6_ROW + 8 * ks);
      bop[j] = v8i{h.x, h.y, h.z, h.w, t.x, t.y, 0, 0};
      sB[j] = (int)(*reinterpret_cast<const uint16_t*>(S + 128 + bsc + 16 * j + 4 * ks));
      split |= unmerged(sB[j]);
    }
    // merged k-step: one MFMA per tile over the whole pair.  Otherwise the same
    // MFMAs take only the first 16 K of A (scale bytes 0), and a second round the
    // last 16 K (scale bytes 1).
    const bool two = __builtin_amdgcn_ballot_w64(split) != 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v8i a = aop[i];
      if (two) a[3] = a[4] = a[5] = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop[j], acc[i][j], 3, 3, 0, sA[i], 0, sB[j]);
    }
    if (two) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const v8i a = {0, 0, 0, aop[i][3], aop[i][4], aop[i][5], 0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop[j], acc[i][j], 3, 3, 1, sA[i], 1, sB[j]);
      }
    }
  }
}

// A: operand of the left matrix [M x K]; B: operand of the right matrix [N x K];
// lda / ldb = operand row pitch (groups * 96 bytes); sA_rs / sB_rs = groups * 8.
template <bool OUT_BF16, bool TRANS_B>
__global__ void __launch_bounds__(PGT, 1)
gemm_m6_kernel(GemmArgs g, int tiles_m, int tiles_n, int per_xcd) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[M6_SMEM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;

  const int b = blockIdx.x;
  const int v = (b & 7) * per_xcd + (b >> 3);
  if (v >= tiles_m * tiles_n) return;
  const int grp = v / (GROUP_M * tiles_n);
  const int first_m = grp * GROUP_M;
  const int gm = min(GROUP_M, tiles_m - first_m);
  const int in_grp = v - grp * GROUP_M * tiles_n;
  const int64_t m0 = (int64_t)(first_m + in_grp % gm) * BM;
  const int64_t n0 = (int64_t)(in_grp / gm) * BN;
  const int nkt = (int)((g.K + 127) / 128);

  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.A + m0 * g.lda), 0, (int)(min<int64_t>(BM, g.M - m0) * g.lda), RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.B + n0 * g.ldb), 0, (int)(min<int64_t>(BN, g.N - n0) * g.ldb), RSRC_FLAGS);
  const bool scale_b = wave >= 4;
  const __amdgpu_buffer_rsrc_t rS = scale_b
      ? __builtin_amdgcn_make_buffer_rsrc((void*)(g.sB + (n0 / 16) * g.sB_rs), 0,
                                          (int)(min<int64_t>(BN / 16, (g.N - n0) / 16) * g.sB_rs), RSRC_FLAGS)
      : __builtin_amdgcn_make_buffer_rsrc((void*)(g.sA + (m0 / 16) * g.sA_rs), 0,
                                          (int)(min<int64_t>(BM / 16, (g.M - m0) / 16) * g.sA_rs), RSRC_FLAGS);
  const int64_t s_rs = scale_b ? g.sB_rs : g.sA_rs;

  // DMA r of this wave fills rows 32*wave .. +32 of region r: lane l -> physical
  // unit l & 1 of row l >> 1 (the swizzle picks which global unit it fetches)
  uint32_t offA, offB;
  {
    const int row = 32 * wave + (lane >> 1);
    const int u = (lane & 1) ^ ((row >> 2) & 1) ^ ((row >> 3) & 1);
    offA = (uint32_t)(row * g.lda + 16 * u);
    offB = (uint32_t)(row * g.ldb + 16 * u);
  }
  const uint32_t offS = (uint32_t)((4 * (wave & 3) + (lane >> 1)) * s_rs + 4 * (lane & 1));
  const int s_lds = 2 * M6_OPB + 32 * wave;
  // global byte of region r within a 96-byte group: heads 0-1 at 0, heads 2-3 at 32, tails at 64
  auto issue = [&](int stage, int kt) {
    uint8_t* base = smem + __builtin_amdgcn_readfirstlane(stage * M6_STAGE);
    const uint32_t kofs = (uint32_t)kt * 96;
#pragma unroll
    for (int r = 0; r < 3; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void*)(base + r * M6_REG + 32 * wave * M6_ROW), 16,
                                               offA + kofs + 32 * r, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 3; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void*)(base + M6_OPB + r * M6_REG + 32 * wave * M6_ROW), 16,
                                               offB + kofs + 32 * r, 0, 0, 0);
    if (lane < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void*)(base + s_lds), 4, offS + (uint32_t)kt * 8, 0, 0, 0);
  };
  // fragment read offsets: A rows wm*64 + 32i + l32, B rows wn*128 + 32j + l32
  const int aoff = tswz(wm * 64 + l32, lh), boff = tswz(wn * 128 + l32, lh);
  const int asc = ((wm * 64 + l32) >> 4) * 8 + 2 * lh, bsc = ((wn * 128 + l32) >> 4) * 8 + 2 * lh;

  AccT<2, 4> acc;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

#pragma unroll
  for (int s = 0; s < M6_NS - 1; ++s)
    if (s < nkt) issue(s, s);

  int kt = 0;
  for (; kt + M6_NS - 1 < nkt; ++kt) {
    compiler_fence();
    FT_WAIT_VMCNT(M6_DMAS * (M6_NS - 2));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    issue((kt + M6_NS - 1) % M6_NS, kt + M6_NS - 1);
    // stage base as an opaque uniform value: keeps loop strength reduction from
    // turning every fragment address into its own induction variable
    const int cur = __builtin_amdgcn_readfirstlane((kt % M6_NS) * M6_STAGE);
    mfma_stage_m6(acc, smem + cur, aoff, boff, asc, bsc);
  }
  for (; kt < nkt; ++kt) {
    compiler_fence();
    FT_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    const int cur = __builtin_amdgcn_readfirstlane((kt % M6_NS) * M6_STAGE);
    mfma_stage_m6(acc, smem + cur, aoff, boff, asc, bsc);
  }
  compiler_fence();
  FT_WAIT_VMCNT(0);
  __syncthreads();
  epilogue_and_store<OUT_BF16, 2, 4, 8, 256, 64>(acc, g, smem, m0, n0, tid, wave, wm, wn, l32, lh);
}

// ---------------------------------------------------------------------------------------
// Generic kernel (any K multiple of 16)
// ---------------------------------------------------------------------------------------
template <bool OUT_BF16>
__global__ void __launch_bounds__(GT, 1) gemm_w4a4_generic_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[GEN_SMEM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;

  const int64_t tiles_m = (g.M + BM - 1) / BM;
  const int64_t m0 = (blockIdx.x % tiles_m) * BM, n0 = (blockIdx.x / tiles_m) * BN;
  const int64_t nkt = (g.K + 127) / 128;
  const int64_t Mb = g.M / 16, Nb = g.N / 16, Kb = g.K / 16;

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
      ps = (gnb < Nb && gkb < Kb) ? g.sB[gnb * g.sB_rs + gkb] : (uint8_t)127;
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

  AccT<4, 4> acc;
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
    mfma_stage<4, 4, BM, BN>(acc, smem + cur * STAGE, wm, wn, l32, lh);
    if (kt + 1 < nkt) lstore(cur ^ 1);
    __syncthreads();
  }
  epilogue_and_store<OUT_BF16, 4, 4, 4, 256, 64>(acc, g, smem, m0, n0, tid, wave, wm, wn, l32, lh);
}

// C = sum over s of part[s], in split order (fp32 adds, so the result does not
// depend on which split finished first), stored fp32 or bf16 (nearest even).
// Four consecutive columns per work item; N is a multiple of 16.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256) split_sum_kernel(const float* __restrict__ part, int splits, int64_t M,
                                                        int64_t N, void* __restrict__ C, int64_t ldc) {
  const int64_t nq = N / 4, total = M * nq, plane = M * N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t m = i / nq, c = 4 * (i - m * nq);
    const float* p = part + m * N + c;
    v4f acc = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    for (int sp = 1; sp < splits; ++sp) {
      const v4f x = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p + sp * plane));
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    if constexpr (OUT_BF16) {
      const uint32_t lo = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
      const uint32_t hi = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
      *reinterpret_cast<v2i*>(static_cast<uint16_t*>(C) + m * ldc + c) = v2i{(int)lo, (int)hi};
    } else {
      *reinterpret_cast<v4f*>(static_cast<float*>(C) + m * ldc + c) = acc;
    }
  }
}

// dA^T and dB from the adapter workgroups' token-range partials: part[s] holds
// [r x ncols0 | r x ncols1] fp32, added in range order.  Four consecutive
// values per work item (both sizes are multiples of 16).
__global__ void __launch_bounds__(256) adapter_sum_kernel(const float* __restrict__ part, int splits, int64_t n0,
                                                          float* __restrict__ out0, int64_t n1,
                                                          float* __restrict__ out1) {
  const int64_t n = n0 + n1;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    v4f acc = *reinterpret_cast<const v4f*>(part + i);
    for (int sp = 1; sp < splits; ++sp) {
      const v4f x = *reinterpret_cast<const v4f*>(part + sp * n + i);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    if (i < n0) *reinterpret_cast<v4f*>(out0 + i) = acc;
    else *reinterpret_cast<v4f*>(out1 + (i - n0)) = acc;
  }
}

// Launch plan of the pipelined kernel.
struct GemmPlan {
  int cfg;          // 0: square 256 x 256 tiles, 1: wide 192 x 384, 2: small 128 x 128
  int splits;       // reduction splits (1: none)
  int64_t tm, tn;   // tile grid
};

// Cost model of the small-product choice, fitted to measured launches of these
// kernels (512-4608 rows, K 3072-12288): time of one 128 x 128 x 128 MFMA
// step of a workgroup on its CU with the big tiles (4 or 4.5 steps per stage)
// and with the small tile (twice the operand bytes per MFMA), the fixed cost of
// a work item (launch, pipeline fill, low-rank term, store), and that of a
// split: the partial sums' round trip through memory and the second launch.
constexpr double STEP_US = 0.294, SMALL_STEP_US = 0.42;
constexpr double ITEM_US = 13.3, SMALL_ITEM_US = 9.3;
constexpr double SPLIT_GBS = 5000.0;    // partial sums' read + write rate, GB/s
constexpr double SPLIT_US = 4.5;
// The same for the backward's dX GEMM (Q(R) read transposed), whose big tiles
// the planner weighs against the adapter workgroups beside them: fitted to the
// dX launches of 4096-4608 rows, reductions 3072-12288, square and wide tiles.
constexpr double DX_STEP_US = 0.323, DX_ITEM_US = 16.0;
constexpr int MAX_SPLITS = 8;
constexpr int MIN_SPLIT_STAGES = 4;     // 128-K stages per split, at least

bool pipelined_ok(const GemmArgs& g) {
  return g.K > 0 && g.K % 128 == 0 && BN * g.lda < ((int64_t)1 << 31) && CfgWide::BN * g.ldb < ((int64_t)1 << 31);
}

// Time of the adapter-gradient workgroups (AdaptArgs of g, dB when with_db) on
// na slots: a unit is one 64-column strip over one token range; the range count
// S minimizes the busiest workgroup's rows (AD_ROW_US per 128-byte row on one
// CU: about 20 GB/s per workgroup, as measured beside the dX GEMM in a training
// step, with X and G streamed from HBM) plus, for S > 1, the partials' round
// trip and the second launch.  *ap (if given) receives the units, ranges and
// workgroups of the minimum.
constexpr double AD_ROW_US = 0.0065;
constexpr double AD_SUM_US = 4.5;
constexpr int AD_MAX_SPLITS = 16;
constexpr int64_t AD_MIN_SPLIT_ROWS = 512;   // tokens per range when S > 1 (one 64-token chunk per wave)

struct AdaptPlan {
  int nwg, splits, units, strips0, strips1;
  int64_t rows_per_split;
};

double adapt_time(const GemmArgs& g, bool with_db, int64_t na, AdaptPlan* ap) {
  AdaptPlan best{};
  best.strips0 = (int)((g.ad.ncols[0] + AD_COLS - 1) / AD_COLS);
  best.strips1 = with_db ? (int)((g.ad.ncols[1] + AD_COLS - 1) / AD_COLS) : 0;
  const int64_t strips = best.strips0 + best.strips1;
  const int64_t n = (int64_t)g.ad.r * (g.ad.ncols[0] + (with_db ? g.ad.ncols[1] : 0));
  double best_t = 1e300;
  for (int S = 1; S <= AD_MAX_SPLITS; ++S) {
    const int64_t rps = ((g.M + S - 1) / S + 63) / 64 * 64;
    if (S > 1 && rps < AD_MIN_SPLIT_ROWS) break;
    if ((g.M + rps - 1) / rps != S) continue;   // S whole 64-token ranges do not come out
    const int64_t units = strips * S;
    const int64_t nwg = units < na ? units : na;
    // a split must save more than a tenth to be taken (the model is coarse)
    const double t = (double)((units + nwg - 1) / nwg) * (double)rps * AD_ROW_US * (S > 1 ? 1.1 : 1.0) +
                     (S > 1 ? AD_SUM_US + (double)(S + 1) * n * 4 / 5e6 : 0.0);
    if (t < best_t) {
      best_t = t;
      best.nwg = (int)nwg;
      best.splits = S;
      best.units = (int)units;
      best.rows_per_split = rps;
    }
  }
  if (ap) *ap = best;
  return best_t;
}

// Slots the adapter workgroups take beside a GEMM of W work items: those its
// last round leaves free (they start with it), or, when that is under an
// eighth, every slot (they follow it).
int64_t adapt_slots(int64_t W, int64_t slots) {
  const int64_t free_slots = (W + slots - 1) / slots * slots - W;
  return free_slots >= slots / 8 ? free_slots : slots;
}

// beside: see launch_gemm_w4a4.  can_split: a workspace for split partials exists.
// ad: the adapter gradients the same launch computes (launch_gemm_w4a4_adapt;
// with_db: dB among them), or nullptr.  splits > 1 only when can_split; the
// result depends on the shape, the CU count, these flags and ad's rank and
// column counts only.
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool beside, bool can_split, const GemmArgs* ad = nullptr,
                   bool with_db = true) {
  const int cus = num_cus();
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN, tiles = tiles_m * tiles_n;
  const int64_t wm_ = (M + CfgWide::BM - 1) / CfgWide::BM, wn_ = (N + CfgWide::BN - 1) / CfgWide::BN;
  const int64_t wide = wm_ * wn_;
  const int64_t nkt = K / 128;
  auto round_us = [&](bool w) { return (double)nkt * (w ? 4.5 : 4.0) * STEP_US + ITEM_US; };
  // Big tiles: the shape that fills the CUs in fewer partial rounds.  When other
  // kernels run beside the GEMM and both shapes take one round: with the adapter
  // workgroups in the launch, the shape whose GEMM round or adapter work (on the
  // slots it leaves) ends first; otherwise the one with fewer tiles, which
  // leaves those kernels more CUs.
  bool use_wide;
  if (beside && wide <= cus && tiles <= cus) {
    if (ad) {
      auto end_us = [&](bool w) {
        const int64_t na = adapt_slots(w ? wide : tiles, cus);
        const double ta = adapt_time(*ad, with_db, na, nullptr);
        const double tg = (double)nkt * (w ? 4.5 : 4.0) * DX_STEP_US + DX_ITEM_US;
        return na == cus ? tg + ta : (tg > ta ? tg : ta);
      };
      use_wide = end_us(true) < end_us(false);
    } else {
      use_wide = wide < tiles;
    }
  } else {
    use_wide = fill(wide, cus) > fill(tiles, cus) + 0.02;
  }
  GemmPlan p{use_wide ? 1 : 0, 1, use_wide ? wm_ : tiles_m, use_wide ? wn_ : tiles_n};
  if (tiles >= cus) return p;                                  // every CU has a big tile already
  // Fewer big tiles than CUs: compare with 128 x 128 tiles and split reductions
  // by the busiest CU's time.
  auto rounds = [&](int64_t units) { return (double)((units + cus - 1) / cus); };
  double best = rounds(p.tm * p.tn) * round_us(use_wide);
  const int64_t sm = (M + CfgSmall::BM - 1) / CfgSmall::BM, sn = (N + CfgSmall::BN - 1) / CfgSmall::BN;
  for (int S = 1; S <= (can_split ? MAX_SPLITS : 1); ++S) {
    if (S > 1 && nkt < (int64_t)S * MIN_SPLIT_STAGES) break;
    const double t = rounds(sm * sn * S) * ((double)((nkt + S - 1) / S) * SMALL_STEP_US + SMALL_ITEM_US) +
                     (S > 1 ? (double)(S + 1) * M * N * 4 / (SPLIT_GBS * 1e3) + SPLIT_US : 0.0);
    if (t < best) {
      best = t;
      p = GemmPlan{2, S, sm, sn};
    }
  }
  return p;
}

// Adapter workgroups of the backward GEMM launch (adapt_slots, adapt_time)
AdaptPlan plan_adapt(const GemmArgs& g, bool can_split, bool with_db) {
  const GemmPlan gp = plan_gemm(g.M, g.N, g.K, true, can_split, &g, with_db);
  AdaptPlan ap{};
  adapt_time(g, with_db, adapt_slots(gp.tm * gp.tn * gp.splits, (int64_t)num_cus() * cfg_occ(gp.cfg)), &ap);
  return ap;
}

}  // namespace

ft_status gemm_w4a4_plan(int64_t M, int64_t N, int64_t K, bool beside, bool can_split, int* tile_m, int* tile_n,
                         int* splits) {
  if (M < 0 || N < 0 || K < 0) return FT_ESHAPE;
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K; g.lda = K / 2; g.ldb = K / 2;
  if (!pipelined_ok(g)) {                                      // generic kernel: square tiles, whole reduction
    *tile_m = BM; *tile_n = BN; *splits = 1;
    return FT_OK;
  }
  const GemmPlan p = plan_gemm(M, N, K, beside, can_split);
  *tile_m = p.cfg == 2 ? CfgSmall::BM : p.cfg == 1 ? CfgWide::BM : BM;
  *tile_n = p.cfg == 2 ? CfgSmall::BN : p.cfg == 1 ? CfgWide::BN : BN;
  *splits = p.splits;
  return FT_OK;
}

size_t gemm_w4a4_workspace(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128) return 0;
  const GemmPlan p = plan_gemm(M, N, K, false, true);
  const GemmPlan q = plan_gemm(M, N, K, true, true);
  const int S = p.splits > q.splits ? p.splits : q.splits;
  return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

namespace {
// C from the split partials g.part (the second kernel of a split launch)
ft_status launch_split_sum(const GemmArgs& g, int splits, bool out_bf16, hipStream_t s) {
  const int64_t items = g.M * (g.N / 4);
  int64_t blocks = (items + 255) / 256;
  if (blocks > 16 * (int64_t)num_cus()) blocks = 16 * (int64_t)num_cus();
  if (out_bf16)
    hipLaunchKernelGGL((split_sum_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, s, g.part, splits, g.M, g.N,
                       g.C, g.ldc);
  else
    hipLaunchKernelGGL((split_sum_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, s, g.part, splits, g.M, g.N,
                       g.C, g.ldc);
  return launch_status();
}
}  // namespace

ft_status launch_gemm_w4a4(const GemmArgs& g_in, bool out_bf16, bool trans_b, hipStream_t s, bool beside,
                           void* ws) {
  if (g_in.M == 0 || g_in.N == 0) return FT_OK;
  const int64_t tiles_m = (g_in.M + BM - 1) / BM, tiles_n = (g_in.N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles >= ((int64_t)1 << 28)) return FT_ESHAPE;
  if (pipelined_ok(g_in)) {
    const GemmPlan p = plan_gemm(g_in.M, g_in.N, g_in.K, beside, ws != nullptr);
    GemmArgs g = g_in;
    g.splits = p.splits;
    g.part = static_cast<float*>(ws);
    const int per_xcd = (int)((p.tm * p.tn * p.splits + 7) / 8);
    const dim3 grid((unsigned)(8 * per_xcd)), block(PGT);
    const int tm = (int)p.tm, tn = (int)p.tn;
#define FT_GEMM_LAUNCH(OB, TB, C, SP) \
  hipLaunchKernelGGL((gemm_w4a4_kernel<OB, TB, C, false, 0, SP>), grid, block, 0, s, g, tm, tn, per_xcd)
    if (p.splits > 1) {   // fp32 partials, then their sum
      if (trans_b) FT_GEMM_LAUNCH(false, true, 2, true); else FT_GEMM_LAUNCH(false, false, 2, true);
      const ft_status st = launch_status();
      if (st != FT_OK) return st;
      return launch_split_sum(g, p.splits, out_bf16, s);
    } else if (p.cfg == 2) {
      if (out_bf16) { if (trans_b) FT_GEMM_LAUNCH(true, true, 2, false); else FT_GEMM_LAUNCH(true, false, 2, false); }
      else { if (trans_b) FT_GEMM_LAUNCH(false, true, 2, false); else FT_GEMM_LAUNCH(false, false, 2, false); }
    } else if (p.cfg == 1) {
      if (out_bf16) { if (trans_b) FT_GEMM_LAUNCH(true, true, 1, false); else FT_GEMM_LAUNCH(true, false, 1, false); }
      else { if (trans_b) FT_GEMM_LAUNCH(false, true, 1, false); else FT_GEMM_LAUNCH(false, false, 1, false); }
    } else {
      if (out_bf16) { if (trans_b) FT_GEMM_LAUNCH(true, true, 0, false); else FT_GEMM_LAUNCH(true, false, 0, false); }
      else { if (trans_b) FT_GEMM_LAUNCH(false, true, 0, false); else FT_GEMM_LAUNCH(false, false, 0, false); }
    }
#undef FT_GEMM_LAUNCH
    return launch_status();
  }
  const dim3 grid((unsigned)tiles), block(GT);
  if (out_bf16) hipLaunchKernelGGL((gemm_w4a4_generic_kernel<true>), grid, block, 0, s, g_in);
  else hipLaunchKernelGGL((gemm_w4a4_generic_kernel<false>), grid, block, 0, s, g_in);
  return launch_status();
}

bool gemm_w4a4_adapt_ok(const GemmArgs& g) {   // the shape (the launch checks the pointers)
  if (!(g.M > 0 && g.N > 0 && pipelined_ok(g) && g.ad.r > 0 && g.ad.r <= AD_MAX_R && g.ad.r % 16 == 0 &&
        g.ad.ncols[0] == g.N && g.ad.ncols[1] == g.K && g.ad.M == g.M && g.ad.ldp >= g.ad.poff + g.ad.r &&
        (g.M + BM - 1) / BM * ((g.N + BN - 1) / BN) < ((int64_t)1 << 28)))
    return false;
  // the adapter's 32-bit buffer offsets cover a token range of Q and of P (P's
  // row bound taken at the largest rs + r, so that the choice does not depend on rs)
  const int64_t ncmax = g.ad.ncols[0] > g.ad.ncols[1] ? g.ad.ncols[0] : g.ad.ncols[1];
  if (g.M * ncmax * 2 >= ((int64_t)1 << 31) || g.M * 128 * 4 >= ((int64_t)1 << 31)) return false;
  // two rank tiles only beside the big tiles (the small tile keeps two workgroups per CU)
  if (g.ad.r > 32 && (plan_gemm(g.M, g.N, g.K, true, false).cfg == 2 || plan_gemm(g.M, g.N, g.K, true, true).cfg == 2))
    return false;
  return true;
}

size_t gemm_w4a4_adapt_workspace(const GemmArgs& g, bool can_split) {
  if (!gemm_w4a4_adapt_ok(g)) return 0;
  size_t b = 0;
  for (int with_db = 0; with_db < 2; ++with_db) {   // with and without dB (a caller may leave it out)
    const AdaptPlan ap = plan_adapt(g, can_split, with_db != 0);
    const size_t n = (size_t)g.ad.r * (size_t)(g.ad.ncols[0] + (with_db ? g.ad.ncols[1] : 0));
    if (ap.splits > 1 && (size_t)ap.splits * n * sizeof(float) > b) b = (size_t)ap.splits * n * sizeof(float);
  }
  return b;
}

bool gemm_w4a4_adapt_plan(const GemmArgs& g, bool can_split, bool with_db, int* tile_m, int* tile_n,
                          int* gemm_splits, int* nwg, int* splits) {
  *nwg = 0;
  *splits = 1;
  if (!gemm_w4a4_adapt_ok(g)) return false;
  const GemmPlan p = plan_gemm(g.M, g.N, g.K, true, can_split, &g, with_db);
  const AdaptPlan ap = plan_adapt(g, can_split, with_db);
  *tile_m = p.cfg == 2 ? CfgSmall::BM : p.cfg == 1 ? CfgWide::BM : BM;
  *tile_n = p.cfg == 2 ? CfgSmall::BN : p.cfg == 1 ? CfgWide::BN : BN;
  *gemm_splits = p.splits;
  *nwg = ap.nwg;
  *splits = ap.splits;
  return true;
}

ft_status launch_gemm_w4a4_adapt(const GemmArgs& g_in, bool out_bf16, hipStream_t s, void* gemm_ws, void* adapt_ws) {
  if (!gemm_w4a4_adapt_ok(g_in)) return FT_ENOTSUP;
  if (!g_in.ad.P[0] || !g_in.ad.Q[0] || !g_in.ad.out[0] || (g_in.ad.out[1] && (!g_in.ad.P[1] || !g_in.ad.Q[1])))
    return FT_EINVAL;
  const bool with_db = g_in.ad.out[1] != nullptr;
  const GemmPlan p = plan_gemm(g_in.M, g_in.N, g_in.K, true, gemm_ws != nullptr, &g_in, with_db);
  const AdaptPlan ap = plan_adapt(g_in, gemm_ws != nullptr, with_db);
  if (ap.splits > 1 && !adapt_ws) return FT_EINVAL;
  GemmArgs g = g_in;
  g.splits = p.splits;
  g.part = static_cast<float*>(gemm_ws);
  g.ad.strips[0] = ap.strips0;
  g.ad.strips[1] = ap.strips1;
  g.ad.splits = ap.splits;
  g.ad.rows_per_split = ap.rows_per_split;
  g.ad.units = ap.units;
  g.ad.nwg = ap.nwg;
  g.ad.part = static_cast<float*>(adapt_ws);
  const int per_xcd = (int)((p.tm * p.tn * p.splits + 7) / 8);
  const dim3 grid((unsigned)(8 * per_xcd + ap.nwg)), block(PGT);
  const int tm = (int)p.tm, tn = (int)p.tn;
#define FT_GEMM_LAUNCH_AD(OB, C, SP, NRT) \
  hipLaunchKernelGGL((gemm_w4a4_kernel<OB, true, C, false, 0, SP, NRT>), grid, block, 0, s, g, tm, tn, per_xcd)
  const bool two = g.ad.r > 32;   // never with the small tile (gemm_w4a4_adapt_ok)
  if (p.splits > 1) FT_GEMM_LAUNCH_AD(false, 2, true, 1);
  else if (p.cfg == 2) { if (out_bf16) FT_GEMM_LAUNCH_AD(true, 2, false, 1); else FT_GEMM_LAUNCH_AD(false, 2, false, 1); }
  else if (p.cfg == 1) {
    if (two) { if (out_bf16) FT_GEMM_LAUNCH_AD(true, 1, false, 2); else FT_GEMM_LAUNCH_AD(false, 1, false, 2); }
    else { if (out_bf16) FT_GEMM_LAUNCH_AD(true, 1, false, 1); else FT_GEMM_LAUNCH_AD(false, 1, false, 1); }
  } else {
    if (two) { if (out_bf16) FT_GEMM_LAUNCH_AD(true, 0, false, 2); else FT_GEMM_LAUNCH_AD(false, 0, false, 2); }
    else { if (out_bf16) FT_GEMM_LAUNCH_AD(true, 0, false, 1); else FT_GEMM_LAUNCH_AD(false, 0, false, 1); }
  }
#undef FT_GEMM_LAUNCH_AD
  ft_status st = launch_status();
  if (st != FT_OK) return st;
  if (p.splits > 1) {
    st = launch_split_sum(g, p.splits, out_bf16, s);
    if (st != FT_OK) return st;
  }
  if (ap.splits > 1) {
    const int64_t n0 = (int64_t)g.ad.r * g.ad.ncols[0], n1 = g.ad.out[1] ? (int64_t)g.ad.r * g.ad.ncols[1] : 0;
    int64_t blocks = ((n0 + n1) / 4 + 255) / 256;
    if (blocks > 16 * (int64_t)num_cus()) blocks = 16 * (int64_t)num_cus();
    hipLaunchKernelGGL(adapter_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, s, g.ad.part, ap.splits, n0,
                       g.ad.out[0], n1, g.ad.out[1]);
    st = launch_status();
  }
  return st;
}

ft_status launch_gemm_w4a4_gelu_quant(const GemmArgs& g, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return FT_OK;
  const int64_t tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  if (tiles_m * tiles_n >= ((int64_t)1 << 28)) return FT_ESHAPE;
  if (!pipelined_ok(g)) return FT_ENOTSUP;
  const GemmPlan p = plan_gemm(g.M, g.N, g.K, false, false);
  const int per_xcd = (int)((p.tm * p.tn + 7) / 8);
  const dim3 grid((unsigned)(8 * per_xcd)), block(PGT);
  const int tm = (int)p.tm, tn = (int)p.tn;
  if (p.cfg == 2)
    hipLaunchKernelGGL((gemm_w4a4_kernel<true, false, 2, true>), grid, block, 0, s, g, tm, tn, per_xcd);
  else if (p.cfg == 1)
    hipLaunchKernelGGL((gemm_w4a4_kernel<true, false, 1, true>), grid, block, 0, s, g, tm, tn, per_xcd);
  else
    hipLaunchKernelGGL((gemm_w4a4_kernel<true, false, 0, true>), grid, block, 0, s, g, tm, tn, per_xcd);
  return launch_status();
}

ft_status launch_gemm_w4a4_groups(const GemmArgs& g, int gs, bool out_bf16, bool trans_b, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return FT_OK;
  if (gs != 16 && gs != 32) return FT_EINVAL;
  if (g.K == 0) return launch_gemm_w4a4(g, out_bf16, trans_b, s);   // no scales read: the low-rank term only
  const int64_t tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles >= ((int64_t)1 << 28)) return FT_ESHAPE;
  if (!(g.K > 0 && g.K % 128 == 0)) return FT_ENOTSUP;   // pipelined kernel only
  if (BM * g.lda >= ((int64_t)1 << 31) || BN * g.ldb >= ((int64_t)1 << 31) ||
      BM * g.sA_rs >= ((int64_t)1 << 31) || BN * g.sB_rs >= ((int64_t)1 << 31))
    return FT_ESHAPE;
  const int per_xcd = (int)((tiles + 7) / 8);
  const dim3 grid((unsigned)(8 * per_xcd)), block(PGT);
  const int tm = (int)tiles_m, tn = (int)tiles_n;
#define FT_GEMM_G(OB, TB, G) \
  hipLaunchKernelGGL((gemm_w4a4_kernel<OB, TB, 0, false, G>), grid, block, 0, s, g, tm, tn, per_xcd)
  if (gs == 16) {
    if (out_bf16) { if (trans_b) FT_GEMM_G(true, true, 16); else FT_GEMM_G(true, false, 16); }
    else { if (trans_b) FT_GEMM_G(false, true, 16); else FT_GEMM_G(false, false, 16); }
  } else {
    if (out_bf16) { if (trans_b) FT_GEMM_G(true, true, 32); else FT_GEMM_G(true, false, 32); }
    else { if (trans_b) FT_GEMM_G(false, true, 32); else FT_GEMM_G(false, false, 32); }
  }
#undef FT_GEMM_G
  return launch_status();
}

ft_status launch_gemm_m6(const GemmArgs& g, bool out_bf16, bool trans_b, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return FT_OK;
  const int64_t tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles >= ((int64_t)1 << 28)) return FT_ESHAPE;
  if (BM * g.lda >= ((int64_t)1 << 31) || BN * g.ldb >= ((int64_t)1 << 31)) return FT_ESHAPE;
  const int per_xcd = (int)((tiles + 7) / 8);
  const dim3 grid((unsigned)(8 * per_xcd)), block(PGT);
  const int tm = (int)tiles_m, tn = (int)tiles_n;
  if (out_bf16) {
    if (trans_b) hipLaunchKernelGGL((gemm_m6_kernel<true, true>), grid, block, 0, s, g, tm, tn, per_xcd);
    else hipLaunchKernelGGL((gemm_m6_kernel<true, false>), grid, block, 0, s, g, tm, tn, per_xcd);
  } else {
    if (trans_b) hipLaunchKernelGGL((gemm_m6_kernel<false, true>), grid, block, 0, s, g, tm, tn, per_xcd);
    else hipLaunchKernelGGL((gemm_m6_kernel<false, false>), grid, block, 0, s, g, tm, tn, per_xcd);
  }
  return launch_status();
}

}  // namespace ft
