// Internal launch interfaces shared between the ft entry points.
#pragma once

#include "adapter_tile.h"
#include "ft_common.h"

namespace ft {

// C[M x N] = deq(A)[M x K] deq(B)[N x K]^T + P[M x (ra+rb)] [Wa; Wb]
// A, B: packed E2M1 codes, row pitch lda / ldb bytes, reduction index contiguous.
// scale of A block (mb, kb) = sA[mb * sA_rs + kb]; of B block (nb, kb) = sB[nb * sB_rs + kb]
// (E8M0 bytes).  Wa [ra x N], Wb [rb x N] bf16 (row pitch N); P fp32 [M x (ra+rb)].
struct GemmArgs {
  int64_t M, N, K;
  const uint8_t* A; int64_t lda;
  const uint8_t* B; int64_t ldb;
  const uint8_t* sA; int64_t sA_rs;
  const uint8_t* sB; int64_t sB_rs;
  const float* P;
  const uint16_t* Wa; int ra;
  const uint16_t* Wb; int rb;
  void* C; int64_t ldc;
  // MLP fusion epilogue only: H = GELU(C) bf16 (pitch ldc), Q(H) codes row-major
  // [M][N/2] and power-of-two scale bytes [M/16][N/16]
  void* H; uint8_t* hq; uint8_t* hs;
  // split reduction (set by the launcher): split s of `splits` takes the
  // 128-K stages [s nkt / splits, (s+1) nkt / splits) and writes its fp32
  // partial tile to part[s][M][N]; the low-rank term belongs to split 0
  float* part = nullptr; int splits = 1;
  // backward only: the adapter gradients taken by extra workgroups of the launch
  // (launch_gemm_w4a4_adapt fills the plan fields)
  AdaptArgs ad{};
};

// beside: other kernels run concurrently on the device (tile choice leaves them CUs).
// ws: device scratch of at least gemm_w4a4_workspace(M, N, K) bytes, or nullptr:
// with it, a product too small to fill the CUs with whole tiles may split its
// reduction (fp32 partial tiles in ws, summed in split order by a second
// kernel); without it the reduction is never split.  The choice depends only on
// the shape and the device's CU count.
ft_status launch_gemm_w4a4(const GemmArgs& g, bool out_bf16, bool trans_b, hipStream_t s, bool beside = false,
                           void* ws = nullptr);
size_t gemm_w4a4_workspace(int64_t M, int64_t N, int64_t K);
// the tile (rows x columns) and split count launch_gemm_w4a4 takes for a shape
ft_status gemm_w4a4_plan(int64_t M, int64_t N, int64_t K, bool beside, bool can_split, int* tile_m, int* tile_n,
                         int* splits);

// The backward's dX GEMM (trans_b) with the adapter gradients of g.ad (P, Q, out,
// ncols, M, ldp, poff, r set by the caller; out[1] may be null) computed by
// extra workgroups of the same launch, plus, when the plan splits reductions,
// the kernels that add the split partials (all on stream s).  gemm_ws: as for
// launch_gemm_w4a4 (the GEMM's split partials, or nullptr); adapt_ws: at least
// gemm_w4a4_adapt_workspace bytes for the adapter's token-range partials.
// FT_ENOTSUP for shapes it does not take (no pipelined kernel, r > 64, an empty
// dimension): the caller then runs the GEMM and the adapter kernels separately.
ft_status launch_gemm_w4a4_adapt(const GemmArgs& g, bool out_bf16, hipStream_t s, void* gemm_ws, void* adapt_ws);
bool gemm_w4a4_adapt_ok(const GemmArgs& g);
size_t gemm_w4a4_adapt_workspace(const GemmArgs& g, bool can_split);
// the launch's GEMM tile and split count, adapter workgroups and token ranges
// (nothing runs); false when gemm_w4a4_adapt_ok(g) does not hold
bool gemm_w4a4_adapt_plan(const GemmArgs& g, bool can_split, bool with_db, int* tile_m, int* tile_n,
                          int* gemm_splits, int* nwg, int* splits);

// Forward GEMM (bf16 Y) with the MLP fusion epilogue: also H = GELU(Y) and Q(H)
// (g.H, g.hq, g.hs).  FT_ENOTSUP when K is not a multiple of 128 (no pipelined
// kernel for it); the caller then runs the separate kernels.
ft_status launch_gemm_w4a4_gelu_quant(const GemmArgs& g, hipStream_t s);

// The same product with scales per 1 x gs group along each row (gs 16 or 32):
// sA [M][K / gs], sB [N][K / gs] bytes (sA_rs = sB_rs = K / gs).  Square tiles,
// K a multiple of 128 (FT_ENOTSUP otherwise).
ft_status launch_gemm_w4a4_groups(const GemmArgs& g, int gs, bool out_bf16, bool trans_b, hipStream_t s);

// C[M x N] = A[M x K] deq(B)[N x K]^T + P [Wa; Wb] with a bf16 left operand:
// g.A points to bf16 [M x K] with row pitch g.lda BYTES (g.sA unused); B, its
// scales, P, W and C as for launch_gemm_w4a4.  K any multiple of 16.
ft_status launch_gemm_a16(const GemmArgs& g, bool out_bf16, bool trans_b, hipStream_t s);

// Same product from pair-merged FP6 operands (ft_quant_block16_op): A, B are
// operand bytes with row pitch lda / ldb (= groups * 96), sA / sB the operand
// scale grids with sA_rs / sB_rs = groups * 8 bytes per 16-row block.  K may be
// any multiple of 16 (the operands are zero-padded to 128).
ft_status launch_gemm_m6(const GemmArgs& g, bool out_bf16, bool trans_b, hipStream_t s);

// dW[j][c] = sum_m P[m][poff + j] Q[m][c] for j < r, c < ncols (reduction over M),
// P fp32 with row pitch ldp, Q bf16 [M x ncols].  Needs lora_grad_workspace bytes.
size_t lora_grad_workspace(int64_t M, int64_t ncols, int r);
ft_status launch_lora_grad(const float* P, int64_t ldp, int poff, int r, const uint16_t* Q,
                           int64_t M, int64_t ncols, float* dW, void* ws, hipStream_t s);

}  // namespace ft
