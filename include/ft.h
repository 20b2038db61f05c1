/*
 * ft.h -- C ABI of the W4A4G4 triple-branch quantized linear for MI355X (gfx950).
 *
 * Method: FourTune ("FourTune: Towards Fully 4-Bit Efficient Post-Training for
 * Diffusion Models").  A frozen weight is split offline as W ~= R + L1 L2
 * (section 3.1, Eq. 1).  The residual R, the activations X and the output
 * gradient G = dL/dY are quantized in 16x16 blocks (4-bit E2M1 codes plus one
 * scale per block; section 3.1 after Eq. 2, section 3.2, section 4.3 "Impact of
 * Quantization Granularity") and multiplied in 4-bit; the stabilizer L1 L2 and
 * the trainable LoRA factors A, B stay in bf16:
 *
 *   Y  = Q(X) Q(R)^T + X L1 L2 + X A B                       (Eq. 2)
 *   dX = Q(G) Q(R)   + G (L1 L2)^T + G (A B)^T               (Eq. 3)
 *   dB = (X A)^T G,   dA = X^T (G B^T)                        (section 3.2)
 *
 * Shapes: X [M x K] (tokens x in), R and W [N x K] (out x in), G and Y [M x N].
 * The low-rank factors are stored rank-major, each factor's rank index being
 * its row:  L1t = L1^T [rs x K], At = A^T [r x K], L2 [rs x N], B [r x N].
 * Gradients come back in the same layout: dAt = (dA)^T [r x K], dB [r x N].
 *
 * Conventions for every call:
 *  - All tensor pointers are device pointers owned by the caller.  The library
 *    allocates no device memory and keeps no pointer after a call returns.
 *  - Work is enqueued asynchronously on the given stream; nothing synchronizes.
 *    The backward calls fork their adapter-gradient kernels onto a stream the
 *    library keeps per device (created once, non-blocking, default priority)
 *    and join it back with events before returning, so to the caller all
 *    their work is ordered on the given stream as if it ran there.
 *  - Arguments are validated before anything is launched; on error nothing
 *    is enqueued and the status says why.  The library never aborts.
 *  - Matrices are row-major with the stated leading dimension (in elements).
 *  - bf16 data is IEEE-754 binary32's upper half (torch.bfloat16).
 *  - Results are deterministic: the same inputs give the same bits (no
 *    floating-point atomics, fixed reduction orders).
 *  - Pointers must be 16-byte aligned; leading dimensions must keep every
 *    row 16-byte aligned (FT_EALIGN otherwise).
 *  - Every matrix dimension must be a multiple of 16 (the quantization block;
 *    FT_ESHAPE otherwise).  Zero-sized dimensions are accepted: an empty output
 *    enqueues nothing, an empty reduction leaves the low-rank terms (K = 0
 *    forward, N = 0 backward), and zero tokens (M = 0) give zero adapter
 *    gradients.  Pointers to empty operands may be NULL.  Ranks: rs
 *    (stabilizer) and r (LoRA) are multiples of 16 with 0 <= rs + r <= 128.
 */
#ifndef FT_H_
#define FT_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FT_OK = 0,
  FT_EINVAL = 1,   /* null pointer where one is required, unknown enum value */
  FT_ESHAPE = 2,   /* a dimension not a multiple of 16, negative, or ranks out of range */
  FT_EALIGN = 3,   /* pointer or leading dimension breaks 16-byte alignment */
  FT_EHIP = 4,     /* a HIP launch failed (hipGetLastError after the launch) */
  FT_ENOTSUP = 5,  /* valid request that this library does not implement */
  FT_ESPACE = 6    /* workspace smaller than required */
} ft_status;

/* Block-scale rule of the quantizer (the pages fix "scale from the block
 * maximum over 6", not its number format):
 *  FT_SCALE_POW2: s = 2^E, E = min{e : 6 * 2^e >= amax}, clamped to
 *                 [-127, 127]; stored as one E8M0 byte E + 127.  This is amax/6
 *                 rounded up to the power-of-two scale format the gfx950
 *                 block-scaled MFMA consumes; no element saturates.
 *  FT_SCALE_F32:  s = fl32(amax / 6) stored as float; element ratio fl32(x / s).
 * In both rules the element code is the round-to-nearest-even E2M1 value of
 * the ratio, saturating at +-6, with the sign bit of x (so -0 -> code 8), and
 * a block of zeros gets scale 0 (byte 0 or 0.0f) and zero codes. */
typedef enum { FT_SCALE_POW2 = 0, FT_SCALE_F32 = 1 } ft_scale_mode;

typedef enum { FT_OUT_F32 = 0, FT_OUT_BF16 = 1 } ft_out_dtype;

/* ft_quant_block16 -- the 4-bit quantizer Q(.) (section 3.1: Q runs once, ahead
 * of training, on the frozen residual R, and on the fly on the activations;
 * section 3.2: 16x16 blocks whose scale serves both the matrix and its
 * transpose).
 *
 *  x         bf16 [rows x cols], leading dimension ldx (>= cols).
 *  codes_rm  out, may be NULL: row-major packed codes [rows x cols/2] bytes;
 *            element (i, j) in byte i*cols/2 + j/2, even j in the low nibble.
 *  codes_cm  out, may be NULL: column-major packed codes [cols x rows/2];
 *            element (i, j) in byte j*rows/2 + i/2, even i in the low nibble.
 *            (The codes of X^T: what the transposed GEMM of Eq. 3 reads.)
 *  scales    out: [rows/16 x cols/16] row-major, uint8 E8M0 (POW2) or float (F32).
 *  scales_cm out, may be NULL: the same scale grid stored transposed,
 *            [cols/16 x rows/16]; (codes_cm, scales_cm) is Q(x^T) in row-major form.
 *  At least one of codes_rm, codes_cm must be non-NULL.  Input and outputs
 *  must not overlap.  Codes and scales are bit-exact functions of x. */
ft_status ft_quant_block16(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                           ft_scale_mode mode, uint8_t* codes_rm, uint8_t* codes_cm,
                           void* scales, void* scales_cm, hipStream_t stream);

/* Pair-merged GEMM operand of a quantized matrix (FT_SCALE_POW2 only).
 *
 * Not a step of the method but a value-preserving re-encoding of Q(x) for
 * gfx950's block-scaled MFMA, whose 32-value fragments take ONE power-of-two
 * scale: the two 16-column blocks of each 32-column pair share a scale byte
 * where their exponent gap allows it.  Elements are FP6 E3M2 (OCP MX v1.0):
 * with block bytes e1, e2 (an all-zero block takes its partner's byte),
 * d = |e1 - e2|, hi = max, u = min(d, 2, hi): if d - u <= 3 both blocks use
 * byte H = hi - u and element values e2m1(code) * 2^(e_b - H) (exact);
 * otherwise each block keeps its byte and its E2M1 values.  So merged pairs
 * carry equal bytes and unmerged pairs different ones; dequantized values
 * are identical to those of codes + scales.
 *
 * Layout of the operand of a [rows x cols] matrix (pairs along cols):
 *  data    [rows][G * 96] bytes, G = ceil(cols / 128) groups of 4 pairs
 *          (columns past cols are zero padding).  Per row and group: the first
 *          16 bytes of each pair's 24-byte packed value (64 bytes, pairs 0..3),
 *          then the last 8 bytes of pairs 0, 2, 1, 3 in that order (32 bytes).
 *          The 24-byte value of a pair holds its 32 elements, element n in bits
 *          6n .. 6n+5, little-endian.
 *  scales  [rows/16][G * 8] bytes: entries 2p, 2p+1 are pair p's two bytes. */
size_t ft_operand_bytes(int64_t rows, int64_t cols);
size_t ft_operand_scale_bytes(int64_t rows, int64_t cols);

/* ft_quant_block16_op -- Q(x) with FT_SCALE_POW2 (as ft_quant_block16), writing
 * any subset of: E2M1 codes in either layout and the scale grid (as
 * ft_quant_block16; scales required when codes are requested), the operand of
 * x (op_rm + op_rm_scales, pairs along cols: the forward GEMM's layout) and the
 * operand of x^T (op_cm + op_cm_scales, pairs along rows: what the transposed
 * GEMM of Eq. 3 reads; sizes from ft_operand_bytes(cols, rows)).  Each operand
 * needs its scale buffer.  All pointers 16-byte aligned; at least one output. */
ft_status ft_quant_block16_op(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                              uint8_t* codes_rm, uint8_t* codes_cm, uint8_t* scales, uint8_t* scales_cm,
                              uint8_t* op_rm, uint8_t* op_rm_scales, uint8_t* op_cm, uint8_t* op_cm_scales,
                              hipStream_t stream);

/* ft_lowrank_fused -- the shared down-projection of the two low-rank branches
 * (section 3.3 "LoRA Fusion": both branches read the same input, so one pass
 * over it feeds both):
 *
 *   out[:, 0:ra]      = in . wa^T      (wa [ra x Kin], row-major, ld = Kin)
 *   out[:, ra:ra+rb]  = in . wb^T      (wb [rb x Kin])
 *
 * forward:  in = X [M x K],  wa = L1t, wb = At  -> T = [X L1 | X A]
 * backward: in = G [M x N],  wa = L2,  wb = B   -> V = [G L2^T | G B^T]
 *  in   bf16 [M x Kin], leading dimension ld_in.
 *  out  float [M x (ra+rb)], row-major, leading dimension ra+rb.
 *  workspace  device scratch of at least ft_lowrank_workspace(M, Kin, ra+rb)
 *             bytes (may be NULL when that is 0): partial sums of the split
 *             reduction, added in a fixed order.
 *  Products accumulate in fp32 from exact bf16 operands. */
ft_status ft_lowrank_fused(const void* in, int64_t M, int64_t Kin, int64_t ld_in,
                           const void* wa, int32_t ra, const void* wb, int32_t rb,
                           float* out, void* workspace, size_t ws_bytes, hipStream_t stream);

size_t ft_lowrank_workspace(int64_t M, int64_t Kin, int32_t rho);

/* ft_lowrank_plan -- how ft_lowrank_fused, ft_quant_lowrank and
 * ft_gelu_quant_lowrank launch for in [M x Kin] and rho = ra + rb ranks (for
 * tests and profiling; nothing is run).  plan holds 5 int32: plan[0] input rows
 * per workgroup (64: two 128-column groups per 256-column chunk; 128: one
 * 128-column chunk), plan[1] 1 when the input is loaded in whole 128-byte lines
 * and re-laid out through LDS, 0 for loads in the MFMA fragment layout, plan[2]
 * reduction splits (their partials go to the workspace when above 1), plan[3]
 * chunks per split along the reduction (a chunk is 128 columns per column
 * group: 256 columns at 64-row blocks, 128 at 128-row blocks), plan[4] LDS
 * bytes per workgroup.  All zero for an empty input.  FT_ESHAPE for M or
 * Kin not a multiple of 16, or rho not one of 0, 16, ..., 128. */
ft_status ft_lowrank_plan(int64_t M, int64_t Kin, int32_t rho, int32_t* plan);

/* ft_quant_lowrank -- ft_lowrank_fused and the quantizer Q(in) (FT_SCALE_POW2,
 * row-major codes) in one read of the input: the LoRA fusion of section 3.3
 * extended to the quantizer, which reads the same activations (forward: X) or
 * gradient (backward: G).  out / workspace as ft_lowrank_fused (out may be NULL
 * when ra + rb == 0); codes_rm [M x Kin/2] and scales [M/16 x Kin/16] E8M0 bytes
 * as ft_quant_block16's codes_rm and scales, bit for bit. */
ft_status ft_quant_lowrank(const void* in, int64_t M, int64_t Kin, int64_t ld_in,
                           const void* wa, int32_t ra, const void* wb, int32_t rb, float* out,
                           uint8_t* codes_rm, uint8_t* scales, void* workspace, size_t ws_bytes,
                           hipStream_t stream);

/* ft_quant_lowrank_db -- the backward's pass over G with the LoRA gradient
 * folded in (section 3.3 "LoRA Fusion": every branch reads the same G; section
 * 3.2: dB = (X A)^T G).  From one read of g = G [M x N]:
 *
 *   V      = [G L2^T | G B^T]           (as ft_quant_lowrank with wa = L2, wb = B)
 *   Q(G)   codes_rm + scales            (as ft_quant_lowrank)
 *   dB     = T[:, rs:rs+r]^T G          (T: the forward's [X L1 | X A], [M x (rs+r)])
 *
 *  g bf16 [M x N], leading dimension ld_g; L2 [rs x N], B [r x N] bf16; V float
 *  [M x (rs+r)]; T float [M x (rs+r)]; dB float [r x N]; r <= 64.
 *  workspace  at least ft_quant_lowrank_db_workspace(M, N, rs + r, r) bytes: the
 *             V reduction's partials and one dB partial per 128-token block,
 *             added in block order (deterministic).
 * V, codes and scales equal ft_quant_lowrank's bit for bit; dB is the same sum
 * as ft_linear_bwd's in another order (fp32, equal to within rounding).  Follow
 * it with ft_linear_bwd(..., dB = NULL, ...). */
ft_status ft_quant_lowrank_db(const void* g, int64_t M, int64_t N, int64_t ld_g, const void* L2, int32_t rs,
                              const void* B, int32_t r, float* V, uint8_t* codes_rm, uint8_t* scales,
                              const float* T, float* dB, void* workspace, size_t ws_bytes, hipStream_t stream);
size_t ft_quant_lowrank_db_workspace(int64_t M, int64_t N, int32_t rho, int32_t r);

/* ft_gelu_quant_lowrank -- the MLP fusion of section 3.3 ("MLP Fusion": the
 * activation and the second linear's input quantization go with a pass the
 * intermediate already makes, so it is not read back by separate kernels),
 * placed in the second linear's quantize + down-projection pass: from one read
 * of the first linear's output y,
 *
 *   h      = GELU(y)                        (bf16, as ft_gelu_fwd)
 *   Q(h)   codes_rm + scales                (as ft_quant_block16, FT_SCALE_POW2)
 *   out    = [h wa^T | h wb^T]              (as ft_lowrank_fused; the second
 *                                            linear's T with wa = L1t, wb = At)
 *
 *  y, h  bf16 [M x Kin], contiguous rows (leading dimension Kin)
 *  Other arguments and the workspace as ft_quant_lowrank.  All three outputs
 *  equal, bit for bit, ft_gelu_fwd followed by ft_quant_lowrank on h. */
ft_status ft_gelu_quant_lowrank(const void* y, int64_t M, int64_t Kin, const void* wa, int32_t ra,
                                const void* wb, int32_t rb, void* h, float* out, uint8_t* codes_rm,
                                uint8_t* scales, void* workspace, size_t ws_bytes, hipStream_t stream);

/* ft_linear_fwd -- Eq. 2 with the LoRA-fusion epilogue (section 3.3: the
 * backbone GEMM and the up-projections are accumulated in one kernel):
 *
 *   Y = deq(Xq) deq(Rq)^T + T[:, 0:rs] L2 + T[:, rs:rs+r] B
 *
 *  xq_codes   row-major codes of X [M x K/2], xq_scales [M/16 x K/16]
 *  rq_codes   row-major codes of R [N x K/2], rq_scales [N/16 x K/16]
 *  T          float [M x (rs+r)] from ft_lowrank_fused(X, L1t, At)
 *  L2 [rs x N], B [r x N] bf16
 *  Y          [M x N] float or bf16 (round-to-nearest-even of the fp32 result).
 * Only FT_SCALE_POW2 operands are supported by the GEMM (FT_ENOTSUP otherwise):
 * the block-scaled MFMA applies power-of-two scales in hardware. */
ft_status ft_linear_fwd(int64_t M, int64_t N, int64_t K, ft_scale_mode mode,
                        const uint8_t* xq_codes, const void* xq_scales,
                        const uint8_t* rq_codes, const void* rq_scales,
                        const float* T, const void* L2, int32_t rs, const void* B, int32_t r,
                        void* Y, ft_out_dtype ydt, hipStream_t stream);

/* ft_linear_fwd_ws -- ft_linear_fwd with a workspace, for products too small to
 * give every compute unit a whole output tile (few tokens, e.g. the 512 text
 * tokens of a FLUX block): their reduction over K may be split into fp32
 * partial products in the workspace, which a second kernel adds in split order
 * (deterministic: no atomics).  Y equals ft_linear_fwd's up to fp32 summation
 * order.
 *  workspace  device scratch of at least ft_linear_fwd_workspace(M, N, K)
 *             bytes, 16-byte aligned; may be NULL when that is 0 (the shape
 *             does not split; the call is then ft_linear_fwd).  FT_ESPACE when
 *             ws_bytes is smaller.
 * Other arguments as ft_linear_fwd.  The split depends only on the shape and the
 * device's compute-unit count. */
ft_status ft_linear_fwd_ws(int64_t M, int64_t N, int64_t K, ft_scale_mode mode,
                           const uint8_t* xq_codes, const void* xq_scales,
                           const uint8_t* rq_codes, const void* rq_scales,
                           const float* T, const void* L2, int32_t rs, const void* B, int32_t r,
                           void* Y, ft_out_dtype ydt, void* workspace, size_t ws_bytes, hipStream_t stream);

size_t ft_linear_fwd_workspace(int64_t M, int64_t N, int64_t K);

/* ft_linear_plan -- how the 4-bit GEMM of a call is launched (for tests and
 * profiling; nothing is run): plan[0] x plan[1] output tile per workgroup,
 * plan[2] reduction splits.  backward 0: the GEMM of ft_linear_fwd (with_ws 0)
 * or ft_linear_fwd_ws (with_ws 1); backward 1: the dX GEMM of a backward whose
 * adapter gradients run as separate kernels beside it (the _op, _g16 and _grp
 * backwards, and ranks ft_linear_bwd does not take into its launch; with_ws 1:
 * they always have their workspace).  ft_linear_bwd_plan gives ft_linear_bwd's
 * own launch.  M, N, K as in those calls; plan holds 3 int32. */
ft_status ft_linear_plan(int64_t M, int64_t N, int64_t K, int32_t backward, int32_t with_ws, int32_t* plan);

/* ft_linear_bwd -- Eq. 3 and the adapter gradients of section 3.2:
 *
 *   dX  = deq(Gq) deq(Rq) + V[:, 0:rs] L1t + V[:, rs:rs+r] At
 *   dAt = V[:, rs:rs+r]^T X          ( = (X^T G B^T)^T )
 *   dB  = T[:, rs:rs+r]^T G          ( = (X A)^T G )
 *
 *  gq_codes     row-major codes of G [M x N/2], gq_scales [M/16 x N/16]
 *  rq_codes_cm  column-major codes of R [K x N/2] (ft_quant_block16 codes_cm of R)
 *  rq_scales_cm R's scale grid transposed, [K/16 x N/16] (ft_quant_block16
 *               scales_cm of R): the forward's block scales, read transposed
 *  V            float [M x (rs+r)] from ft_lowrank_fused(G, L2, B)
 *  L1t [rs x K], At [r x K] bf16
 *  X  bf16 [M x K], G bf16 [M x N] (unquantized), T float [M x (rs+r)] (forward)
 *  dX [M x K] float or bf16; dAt float [r x K]; dB float [r x N], or NULL to
 *     skip dB (a caller that took it in the pass over G, ft_quant_lowrank_db)
 *  workspace  device scratch of at least ft_linear_bwd_workspace(M, N, K, r)
 *             bytes (partial sums of the reductions over M, and, for few
 *             tokens, of the dX GEMM's split reduction over N as in
 *             ft_linear_fwd_ws).
 * For r <= 64 (r <= 32 where the dX GEMM takes 128 x 128 tiles) and K a
 * multiple of 128 the adapter gradients are computed by extra workgroups of the
 * dX GEMM's own launch: the call enqueues that kernel (plus, where reductions
 * are split, the kernels that add the partials) on `stream` only.  Otherwise
 * they run on a second stream the library creates once per device (default
 * priority) that forks from and joins `stream` through two events.  Either way
 * the results are complete in `stream`'s order when the call's work is; they
 * depend only on the shape and the device's compute-unit count
 * (ft_linear_bwd_plan). */
ft_status ft_linear_bwd(int64_t M, int64_t N, int64_t K, ft_scale_mode mode,
                        const uint8_t* gq_codes, const void* gq_scales,
                        const uint8_t* rq_codes_cm, const void* rq_scales_cm,
                        const float* V, const void* L1t, int32_t rs, const void* At, int32_t r,
                        const void* X, const void* G, const float* T,
                        void* dX, ft_out_dtype dxdt, float* dAt, float* dB,
                        void* workspace, size_t ws_bytes, hipStream_t stream);

/* Bytes of workspace for ft_linear_bwd and for the _op, _g16 and _grp backwards
 * (one size serves them all). */
size_t ft_linear_bwd_workspace(int64_t M, int64_t N, int64_t K, int32_t r);

/* ft_linear_bwd_plan -- how ft_linear_bwd launches (for tests and profiling;
 * nothing is run).  plan holds 5 int32: plan[0] x plan[1] the dX GEMM's output
 * tile, plan[2] its reduction splits, plan[3] the adapter-gradient workgroups in
 * the same launch (0: the adapter gradients run as separate kernels on the
 * side stream), plan[4] the token ranges those workgroups split the reductions
 * over M into.  with_db 0: the plan of a call with dB = NULL. */
ft_status ft_linear_bwd_plan(int64_t M, int64_t N, int64_t K, int32_t r, int32_t with_db, int32_t* plan);

/* ft_linear_bwd_noalloc -- ft_linear_bwd for callers that cannot allocate device
 * memory (code under stream capture, tight loops, harnesses that forbid
 * allocation): the same arguments without the workspace, the same kernels and
 * the same results bit for bit.  The reduction partials live in a fixed scratch
 * area of FT_NOALLOC_SCRATCH_BYTES that the library keeps per GPU (a device
 * array, resident until the process ends; its address is looked up on the first
 * call on each device).  The call allocates nothing and creates no stream or
 * event: where ft_linear_bwd would use its side stream, the adapter gradients
 * run after the dX GEMM on the given stream.
 *  - FT_ESPACE when ft_linear_bwd_workspace(M, N, K, r) exceeds
 *    FT_NOALLOC_SCRATCH_BYTES (every config of the method needs at most 27 MiB).
 *  - Every call on a GPU shares that GPU's scratch: calls that overlap in time
 *    on one GPU (different streams, or host threads) race and must not be
 *    issued.  Nothing in the scratch needs to start at zero; it keeps the last
 *    call's partials. */
#define FT_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
ft_status ft_linear_bwd_noalloc(int64_t M, int64_t N, int64_t K, ft_scale_mode mode,
                                const uint8_t* gq_codes, const void* gq_scales,
                                const uint8_t* rq_codes_cm, const void* rq_scales_cm,
                                const float* V, const void* L1t, int32_t rs, const void* At, int32_t r,
                                const void* X, const void* G, const float* T,
                                void* dX, ft_out_dtype dxdt, float* dAt, float* dB, hipStream_t stream);

/* ft_linear_fwd_op / ft_linear_bwd_op -- the same Eq. 2 and Eq. 3 (and adapter
 * gradients) with the 4-bit operands given as pair-merged operands
 * (ft_quant_block16_op), FT_SCALE_POW2 only.  Results equal those of
 * ft_linear_fwd / ft_linear_bwd on the same Q(.) up to fp32 summation order:
 * the operands carry exactly the same values, but every 32-K MFMA fragment is
 * filled instead of half of it.
 *
 *  fwd:  x_op, x_op_scales   operand of X  [M x K] (op_rm of X)
 *        r_op, r_op_scales   operand of R  [N x K] (op_rm of R)
 *  bwd:  g_op, g_op_scales   operand of G  [M x N] (op_rm of G)
 *        rt_op, rt_op_scales operand of R^T [K x N] (op_cm of R)
 * Other arguments, layouts and the workspace are those of ft_linear_fwd / _bwd. */
ft_status ft_linear_fwd_op(int64_t M, int64_t N, int64_t K, const uint8_t* x_op, const uint8_t* x_op_scales,
                           const uint8_t* r_op, const uint8_t* r_op_scales,
                           const float* T, const void* L2, int32_t rs, const void* B, int32_t r,
                           void* Y, ft_out_dtype ydt, hipStream_t stream);
ft_status ft_linear_bwd_op(int64_t M, int64_t N, int64_t K, const uint8_t* g_op, const uint8_t* g_op_scales,
                           const uint8_t* rt_op, const uint8_t* rt_op_scales,
                           const float* V, const void* L1t, int32_t rs, const void* At, int32_t r,
                           const void* X, const void* G, const float* T,
                           void* dX, ft_out_dtype dxdt, float* dAt, float* dB,
                           void* workspace, size_t ws_bytes, hipStream_t stream);

/* ft_linear_fwd_gelu -- the first linear of an MLP block with the MLP fusion of
 * section 3.3 ("MLP Fusion": the first linear's GEMM carries the activation and
 * the quantization of the second linear's input, so the intermediate is not read
 * back by separate kernels).  Eq. 2 as ft_linear_fwd with a bf16 Y, and from the
 * same epilogue:
 *
 *   H  = GELU(Y)  (bf16; fp32 math on the bf16 Y, as ft_gelu_fwd)
 *   Hq = Q(H)     (row-major codes and power-of-two scales, as ft_quant_block16)
 *
 *  Y, H        bf16 [M x N] (Y is kept for the GELU backward, H for the second
 *              linear's adapter gradient dA)
 *  hq_codes    row-major codes of H [M x N/2]; hq_scales [M/16 x N/16] E8M0 bytes
 * All three equal, bit for bit, ft_linear_fwd (bf16) -> ft_gelu_fwd ->
 * ft_quant_block16 (codes_rm, scales).  Operands and T, L2, B as ft_linear_fwd;
 * FT_SCALE_POW2 only.  When K is not a multiple of 128 the three steps run as
 * those separate kernels. */
ft_status ft_linear_fwd_gelu(int64_t M, int64_t N, int64_t K, ft_scale_mode mode,
                             const uint8_t* xq_codes, const void* xq_scales,
                             const uint8_t* rq_codes, const void* rq_scales,
                             const float* T, const void* L2, int32_t rs, const void* B, int32_t r,
                             void* Y, void* H, uint8_t* hq_codes, void* hq_scales, hipStream_t stream);

/* ft_linear_fwd_a16 / ft_linear_bwd_g16 -- the precision variants of section
 * 4.3 ("Impact of Precision Configurations", Table 4).  W4A16 keeps the
 * activations in bf16, G16 the output gradient; the weight residual stays
 * quantized (same Q(R), same codes and block scales as the W4A4G4 calls), and
 * the low-rank branches and adapter gradients are unchanged.  With ft_linear_fwd
 * and ft_linear_bwd they make up the four settings of the table:
 *   W4A4G4 = fwd + bwd,  W4A16G4 = fwd_a16 + bwd,
 *   W4A4G16 = fwd + bwd_g16,  W4A16G16 = fwd_a16 + bwd_g16.
 *
 *   fwd_a16:  Y  = X deq(Rq)^T + T[:, 0:rs] L2 + T[:, rs:rs+r] B     (Eq. 2, X for Q(X))
 *   bwd_g16:  dX = G deq(Rq)   + V[:, 0:rs] L1t + V[:, rs:rs+r] At   (Eq. 3, G for Q(G))
 *             dAt = V[:, rs:rs+r]^T X,  dB = T[:, rs:rs+r]^T G
 *
 *  X  bf16 [M x K] (leading dimension K), G bf16 [M x N] (leading dimension N)
 *  rq_codes, rq_scales         as ft_linear_fwd (FT_SCALE_POW2 bytes)
 *  rq_codes_cm, rq_scales_cm   as ft_linear_bwd (FT_SCALE_POW2 bytes)
 * All other arguments, layouts, the workspace and the stream behaviour are those
 * of ft_linear_fwd / ft_linear_bwd.  The backbone product runs on bf16 matrix
 * instructions with Q(R) dequantized exactly to bf16 and fp32 accumulation. */
ft_status ft_linear_fwd_a16(int64_t M, int64_t N, int64_t K, const void* X,
                            const uint8_t* rq_codes, const void* rq_scales,
                            const float* T, const void* L2, int32_t rs, const void* B, int32_t r,
                            void* Y, ft_out_dtype ydt, hipStream_t stream);
ft_status ft_linear_bwd_g16(int64_t M, int64_t N, int64_t K, const void* G,
                            const uint8_t* rq_codes_cm, const void* rq_scales_cm,
                            const float* V, const void* L1t, int32_t rs, const void* At, int32_t r,
                            const void* X, const float* T,
                            void* dX, ft_out_dtype dxdt, float* dAt, float* dB,
                            void* workspace, size_t ws_bytes, hipStream_t stream);

/* Other quantization granularities -- section 4.3 ("Impact of Quantization
 * Granularity", Table 5) compares the 16x16 blocks with group-wise 1 x 16
 * scales; 1 x 32 is the group one scale covers in gfx950's block-scaled matrix
 * instruction.  Same element and scale rules as FT_SCALE_POW2 (E2M1 codes,
 * scale 2^E with E = min{e : 6 * 2^e >= group max} clamped to [-127, 127],
 * stored as the byte E + 127), over 1 x group elements along each row.
 *
 * ft_quant_group -- Q(x) in 1 x group groups (group 16 or 32).
 *  x       bf16 [rows x cols], leading dimension ldx (elements, rows 16-byte aligned)
 *  codes   out: row-major packed codes [rows x cols/2] (as ft_quant_block16 codes_rm)
 *  scales  out: [rows x cols/group] bytes
 *  cols must be a multiple of group (FT_ESHAPE).  Bit-exact function of x.
 *
 * ft_requant_group_t -- the backward's right operand under group scales
 * (section 3.2: group scales of a row lie along the reduction axis once the
 * matrix is transposed, so Q(R)^T cannot be read in place): the values of
 * Q(R) = (codes, scales) [rows x cols] transposed and quantized again in
 * 1 x group groups, Q(deq(Q(R))^T).
 *  codes_t  out: row-major codes [cols x rows/2];  scales_t out: [cols x rows/group]
 *  rows and cols must be multiples of group.  Exact (bit-exact function of the input).
 *
 * ft_linear_fwd_grp / ft_linear_bwd_grp -- Eq. 2 and Eq. 3 (and the adapter
 * gradients) with group-scaled operands: xq / rq from ft_quant_group of X and R
 * (scales [M x K/group], [N x K/group]); gq from ft_quant_group of G (scales
 * [M x N/group]); rtq from ft_requant_group_t of Q(R) (codes [K x N/2],
 * scales [K x N/group]).  Other arguments as ft_linear_fwd / ft_linear_bwd.
 * The reduction length (K forward, N backward) must be a multiple of 128
 * (FT_ENOTSUP otherwise).  With group 32 every 32-element fragment of the
 * block-scaled MFMA carries data; with group 16 half of it does, as in the
 * 16x16 path. */
ft_status ft_quant_group(const void* x, int64_t rows, int64_t cols, int64_t ldx, int32_t group,
                         uint8_t* codes, uint8_t* scales, hipStream_t stream);
ft_status ft_requant_group_t(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                             int32_t group, uint8_t* codes_t, uint8_t* scales_t, hipStream_t stream);
ft_status ft_linear_fwd_grp(int64_t M, int64_t N, int64_t K, int32_t group,
                            const uint8_t* xq_codes, const uint8_t* xq_scales,
                            const uint8_t* rq_codes, const uint8_t* rq_scales,
                            const float* T, const void* L2, int32_t rs, const void* B, int32_t r,
                            void* Y, ft_out_dtype ydt, hipStream_t stream);
ft_status ft_linear_bwd_grp(int64_t M, int64_t N, int64_t K, int32_t group,
                            const uint8_t* gq_codes, const uint8_t* gq_scales,
                            const uint8_t* rtq_codes, const uint8_t* rtq_scales,
                            const float* V, const void* L1t, int32_t rs, const void* At, int32_t r,
                            const void* X, const void* G, const float* T,
                            void* dX, ft_out_dtype dxdt, float* dAt, float* dB,
                            void* workspace, size_t ws_bytes, hipStream_t stream);

/* GELU between the two linears of an MLP (section 3.3 "MLP Fusion" names the
 * activation; the exact erf form x * Phi(x) is used).  h = GELU(y) in bf16;
 * dy = GELU'(y) * dh in bf16.  y, dh, h, dy are bf16 [n] (n a multiple of 8). */
ft_status ft_gelu_fwd(const void* y, int64_t n, void* h, hipStream_t stream);
ft_status ft_gelu_bwd(const void* y, const void* dh, int64_t n, void* dy, hipStream_t stream);

/* ft_stream_2to1 -- a measurement reference, not a step of the method: reads n
 * 16-bit values and writes one byte per value (its high byte), the same 2 : 1
 * read : write byte ratio as ft_quant_block16 with both code layouts, as plain
 * streaming with 16-byte accesses.  Its rate is the same-run HBM ceiling the
 * quantizer is compared with.  in [n] 16-bit, out [n] bytes; n a multiple of 16;
 * pointers 16-byte aligned. */
ft_status ft_stream_2to1(const void* in, int64_t n, void* out, hipStream_t stream);

const char* ft_status_str(ft_status s);

#ifdef __cplusplus
}
#endif
#endif /* FT_H_ */
