// Entry points of the triple-branch linear: ft_linear_fwd (Eq. 2) and
// ft_linear_bwd (Eq. 3 plus the adapter gradients of section 3.2), taking the
// 4-bit operands either as E2M1 codes + block scales or as the pair-merged
// operands of ft_quant_block16_op (the _op variants).
#include <mutex>

#include "ft_internal.h"

namespace ft {
namespace {

bool ranks_ok(int rs, int r) { return rs >= 0 && r >= 0 && rs % 16 == 0 && r % 16 == 0 && rs + r <= 128; }
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
int64_t op_groups(int64_t k) { return (k + 127) / 128; }

// dA^T = V[:, rs:]^T X ;  dB = T[:, rs:]^T G  (reductions over the M tokens)
ft_status adapter_grads(int64_t M, int64_t N, int64_t K, const float* V, int rs, int r, const void* X,
                        const void* G, const float* T, float* dAt, float* dB, void* workspace, hipStream_t stream);

// The adapter gradients do not depend on the dX GEMM.  Where the GEMM kernel
// takes them in its own launch (launch_gemm_w4a4_adapt: r <= 64, K a multiple
// of 128) they run on the CUs its last round leaves free.  Otherwise they run
// on a second stream that forks from the caller's stream after the GEMM is
// enqueued and joins it again before the call returns, so the memory-bound
// reductions still use the CUs the GEMM leaves idle instead of following it.  Per device, the library creates once (on first use) one side
// stream (default priority) and one fork and one join event.  An event may be
// recorded again as soon as a wait on it has been enqueued (the wait takes the
// record that precedes it), so the pair is reused by every call; a mutex keeps
// each record + wait pair of concurrent host threads together.
struct SideCtx {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool tried = false;
};

std::mutex side_mu;

SideCtx* side_ctx() {
  static SideCtx ctx[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideCtx& c = ctx[dev];
  if (!c.tried) {
    c.tried = true;
    if (hipStreamCreateWithFlags(&c.stream, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&c.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c.join, hipEventDisableTiming) != hipSuccess)
      c.stream = nullptr;   // no side stream: run everything on the caller's stream
  }
  return c.stream ? &c : nullptr;
}

// enqueue `gemm` on `stream` and the adapter gradients concurrently beside it
// (gemm(stream, beside): beside tells it that other kernels share the device)
template <class F>
ft_status gemm_with_adapter_grads(F gemm, int64_t M, int64_t N, int64_t K, const float* V, int rs, int r,
                                  const void* X, const void* G, const float* T, float* dAt, float* dB,
                                  void* workspace, hipStream_t stream) {
  std::unique_lock<std::mutex> lock(side_mu);
  SideCtx* side = r ? side_ctx() : nullptr;
  if (!side) {  // no side stream: one after the other on the caller's stream
    lock.unlock();
    ft_status st = gemm(stream, false);
    if (st != FT_OK) return st;
    return adapter_grads(M, N, K, V, rs, r, X, G, T, dAt, dB, workspace, stream);
  }
  ft_status st = FT_OK;
  if (hipEventRecord(side->fork, stream) != hipSuccess) st = FT_EHIP;
  if (st == FT_OK) st = gemm(stream, true);
  if (st == FT_OK && hipStreamWaitEvent(side->stream, side->fork, 0) != hipSuccess) st = FT_EHIP;
  if (st == FT_OK) st = adapter_grads(M, N, K, V, rs, r, X, G, T, dAt, dB, workspace, side->stream);
  if (st == FT_OK && hipEventRecord(side->join, side->stream) != hipSuccess) st = FT_EHIP;
  if (st == FT_OK && hipStreamWaitEvent(stream, side->join, 0) != hipSuccess) st = FT_EHIP;
  return st;
}

}  // namespace
}  // namespace ft

namespace ft {
namespace {
// ft_linear_fwd (with_ws false: no workspace, the reduction is never split) and
// ft_linear_fwd_ws
ft_status linear_fwd_impl(int64_t M, int64_t N, int64_t K, ft_scale_mode mode, const uint8_t* xq_codes,
                          const void* xq_scales, const uint8_t* rq_codes, const void* rq_scales, const float* T,
                          const void* L2, int32_t rs, const void* B, int32_t r, void* Y, ft_out_dtype ydt,
                          bool with_ws, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (mode != FT_SCALE_POW2 && mode != FT_SCALE_F32) return FT_EINVAL;
  if (ydt != FT_OUT_F32 && ydt != FT_OUT_BF16) return FT_EINVAL;
  if (!mult16(M) || !mult16(N) || !mult16(K) || !ranks_ok(rs, r)) return FT_ESHAPE;
  if (mode != FT_SCALE_POW2) return FT_ENOTSUP;
  if (M == 0 || N == 0) return FT_OK;
  const int rho = rs + r;
  if (!Y || (K && (!xq_codes || !xq_scales || !rq_codes || !rq_scales)) || (rho && !T) ||
      (rs && !L2) || (r && !B))
    return FT_EINVAL;
  if (!aligned16(Y) || (K && (!aligned16(xq_codes) || !aligned16(rq_codes))) || (rho && !aligned16(T)) ||
      (rs && !aligned16(L2)) || (r && !aligned16(B)))
    return FT_EALIGN;
  const size_t need = with_ws ? gemm_w4a4_workspace(M, N, K) : 0;
  if (need && !workspace) return FT_EINVAL;
  if (need && !aligned16(workspace)) return FT_EALIGN;
  if (need && ws_bytes < need) return FT_ESPACE;
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.A = xq_codes; g.lda = K / 2;
  g.B = rq_codes; g.ldb = K / 2;
  g.sA = static_cast<const uint8_t*>(xq_scales); g.sA_rs = K / 16;
  g.sB = static_cast<const uint8_t*>(rq_scales); g.sB_rs = K / 16;
  g.P = T;
  g.Wa = static_cast<const uint16_t*>(L2); g.ra = rs;
  g.Wb = static_cast<const uint16_t*>(B); g.rb = r;
  g.C = Y; g.ldc = N;
  return launch_gemm_w4a4(g, ydt == FT_OUT_BF16, false, stream, false, need ? workspace : nullptr);
}
}  // namespace
}  // namespace ft

extern "C" ft_status ft_linear_fwd(int64_t M, int64_t N, int64_t K, ft_scale_mode mode,
                                   const uint8_t* xq_codes, const void* xq_scales,
                                   const uint8_t* rq_codes, const void* rq_scales,
                                   const float* T, const void* L2, int32_t rs, const void* B, int32_t r,
                                   void* Y, ft_out_dtype ydt, hipStream_t stream) {
  return ft::linear_fwd_impl(M, N, K, mode, xq_codes, xq_scales, rq_codes, rq_scales, T, L2, rs, B, r, Y, ydt,
                             false, nullptr, 0, stream);
}

extern "C" size_t ft_linear_fwd_workspace(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return 0;
  return ft::gemm_w4a4_workspace(M, N, K);
}

extern "C" ft_status ft_linear_plan(int64_t M, int64_t N, int64_t K, int32_t backward, int32_t with_ws,
                                    int32_t* plan) {
  using namespace ft;
  if (!plan) return FT_EINVAL;
  if (!mult16(M) || !mult16(N) || !mult16(K)) return FT_ESHAPE;
  int tm = 0, tn = 0, sp = 1;
  // the backward's dX GEMM: M x K output, reduction over N, planned as with the
  // adapter gradients on the side stream beside it
  const ft_status st = backward ? gemm_w4a4_plan(M, K, N, true, with_ws != 0, &tm, &tn, &sp)
                                : gemm_w4a4_plan(M, N, K, false, with_ws != 0, &tm, &tn, &sp);
  plan[0] = tm;
  plan[1] = tn;
  plan[2] = sp;
  return st;
}

extern "C" ft_status ft_linear_fwd_ws(int64_t M, int64_t N, int64_t K, ft_scale_mode mode,
                                      const uint8_t* xq_codes, const void* xq_scales,
                                      const uint8_t* rq_codes, const void* rq_scales,
                                      const float* T, const void* L2, int32_t rs, const void* B, int32_t r,
                                      void* Y, ft_out_dtype ydt, void* workspace, size_t ws_bytes,
                                      hipStream_t stream) {
  return ft::linear_fwd_impl(M, N, K, mode, xq_codes, xq_scales, rq_codes, rq_scales, T, L2, rs, B, r, Y, ydt,
                             true, workspace, ws_bytes, stream);
}

extern "C" ft_status ft_linear_fwd_gelu(int64_t M, int64_t N, int64_t K, ft_scale_mode mode,
                                        const uint8_t* xq_codes, const void* xq_scales,
                                        const uint8_t* rq_codes, const void* rq_scales,
                                        const float* T, const void* L2, int32_t rs, const void* B, int32_t r,
                                        void* Y, void* H, uint8_t* hq_codes, void* hq_scales, hipStream_t stream) {
  using namespace ft;
  if (mode != FT_SCALE_POW2 && mode != FT_SCALE_F32) return FT_EINVAL;
  if (!mult16(M) || !mult16(N) || !mult16(K) || !ranks_ok(rs, r)) return FT_ESHAPE;
  if (mode != FT_SCALE_POW2) return FT_ENOTSUP;
  if (M == 0 || N == 0) return FT_OK;
  const int rho = rs + r;
  if (!Y || !H || !hq_codes || !hq_scales || (K && (!xq_codes || !xq_scales || !rq_codes || !rq_scales)) ||
      (rho && !T) || (rs && !L2) || (r && !B))
    return FT_EINVAL;
  if (!aligned16(Y) || !aligned16(H) || !aligned16(hq_codes) || !aligned16(hq_scales) ||
      (K && (!aligned16(xq_codes) || !aligned16(rq_codes))) || (rho && !aligned16(T)) ||
      (rs && !aligned16(L2)) || (r && !aligned16(B)))
    return FT_EALIGN;
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.A = xq_codes; g.lda = K / 2;
  g.B = rq_codes; g.ldb = K / 2;
  g.sA = static_cast<const uint8_t*>(xq_scales); g.sA_rs = K / 16;
  g.sB = static_cast<const uint8_t*>(rq_scales); g.sB_rs = K / 16;
  g.P = T;
  g.Wa = static_cast<const uint16_t*>(L2); g.ra = rs;
  g.Wb = static_cast<const uint16_t*>(B); g.rb = r;
  g.C = Y; g.ldc = N;
  g.H = H; g.hq = hq_codes; g.hs = static_cast<uint8_t*>(hq_scales);
  const ft_status st = launch_gemm_w4a4_gelu_quant(g, stream);
  if (st != FT_ENOTSUP) return st;
  // no pipelined kernel for this K: the same three results from the separate kernels
  ft_status s2 = launch_gemm_w4a4(g, true, false, stream);
  if (s2 == FT_OK) s2 = ft_gelu_fwd(Y, M * N, H, stream);
  if (s2 == FT_OK) s2 = ft_quant_block16(H, M, N, N, FT_SCALE_POW2, hq_codes, nullptr, hq_scales, nullptr, stream);
  return s2;
}

namespace ft {
namespace {
// The dX GEMM of the backward: M x K output, reduction over N.  With the
// adapter gradients in the same launch (bwd_gemm_args(...).ad set), the
// backward's workspace is [adapter token-range partials | the GEMM's split
// partials]; otherwise [dA partials | dB partials | the GEMM's split partials].
GemmArgs bwd_shape(int64_t M, int64_t N, int64_t K, int rs, int r) {
  GemmArgs g{};
  g.M = M; g.N = K; g.K = N;
  g.lda = N / 2; g.ldb = N / 2;
  g.ad.M = M; g.ad.ldp = rs + r; g.ad.poff = rs; g.ad.r = r;
  g.ad.ncols[0] = K; g.ad.ncols[1] = N;
  return g;
}
size_t bwd_adapt_bytes(const GemmArgs& g) {
  return align256(gemm_w4a4_adapt_workspace(g, gemm_w4a4_workspace(g.M, g.N, g.K) > 0));
}
}  // namespace
}  // namespace ft

// One size for every backward entry point: the larger of the two layouts (the
// _op, _g16 and _grp backwards always take the separate adapter kernels).
extern "C" size_t ft_linear_bwd_workspace(int64_t M, int64_t N, int64_t K, int32_t r) {
  using namespace ft;
  if (M < 0 || N < 0 || K < 0 || r < 0) return 0;
  const size_t sep = align256(lora_grad_workspace(M, K, r)) + align256(lora_grad_workspace(M, N, r)) +
                     gemm_w4a4_workspace(M, K, N);
  const GemmArgs g = bwd_shape(M, N, K, 0, r);   // the plan does not depend on rs
  const size_t one = gemm_w4a4_adapt_ok(g) ? bwd_adapt_bytes(g) + gemm_w4a4_workspace(M, K, N) : 0;
  return sep > one ? sep : one;
}

extern "C" ft_status ft_linear_bwd_plan(int64_t M, int64_t N, int64_t K, int32_t r, int32_t with_db,
                                        int32_t* plan) {
  using namespace ft;
  if (!plan) return FT_EINVAL;
  if (!mult16(M) || !mult16(N) || !mult16(K) || r < 0 || r % 16 || r > 128) return FT_ESHAPE;
  const GemmArgs g = bwd_shape(M, N, K, 0, r);
  const bool split = gemm_w4a4_workspace(M, K, N) > 0;
  int tm = 0, tn = 0, sp = 1, nwg = 0, asp = 1;
  ft_status st = FT_OK;
  if (!gemm_w4a4_adapt_plan(g, split, with_db != 0, &tm, &tn, &sp, &nwg, &asp))
    st = gemm_w4a4_plan(M, K, N, true, split, &tm, &tn, &sp);   // the GEMM beside the side stream
  plan[0] = tm;
  plan[1] = tn;
  plan[2] = sp;
  plan[3] = nwg;
  plan[4] = asp;
  return st;
}

namespace ft {
namespace {
// ft_linear_bwd with its workspace given; side: the adapter gradients may run on
// the library's side stream (otherwise after the GEMM on the caller's stream)
ft_status linear_bwd_impl(int64_t M, int64_t N, int64_t K, ft_scale_mode mode,
                          const uint8_t* gq_codes, const void* gq_scales,
                          const uint8_t* rq_codes_cm, const void* rq_scales_cm,
                          const float* V, const void* L1t, int32_t rs, const void* At, int32_t r,
                          const void* X, const void* G, const float* T,
                          void* dX, ft_out_dtype dxdt, float* dAt, float* dB,
                          void* workspace, size_t ws_bytes, hipStream_t stream, bool side) {
  if (mode != FT_SCALE_POW2 && mode != FT_SCALE_F32) return FT_EINVAL;
  if (dxdt != FT_OUT_F32 && dxdt != FT_OUT_BF16) return FT_EINVAL;
  if (!mult16(M) || !mult16(N) || !mult16(K) || !ranks_ok(rs, r)) return FT_ESHAPE;
  if (mode != FT_SCALE_POW2) return FT_ENOTSUP;
  const int rho = rs + r;
  const size_t need = ft_linear_bwd_workspace(M, N, K, r);
  if (M && K && !dX) return FT_EINVAL;
  if (M && N && K && (!gq_codes || !gq_scales || !rq_codes_cm || !rq_scales_cm)) return FT_EINVAL;
  if (M && rho && !V) return FT_EINVAL;
  if ((rs && K && !L1t) || (r && K && (!At || !dAt))) return FT_EINVAL;   // dB may be NULL: not computed
  if (r && M && ((K && !X) || (N && !G) || !T)) return FT_EINVAL;
  if (need && (!workspace || ws_bytes < need)) return workspace ? FT_ESPACE : FT_EINVAL;
  const void* ptrs[] = {gq_codes, rq_codes_cm, V, L1t, At, X, G, T, dX, dAt, dB, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FT_EALIGN;

  // dX = deq(Gq) deq(Rq) + V [L1^T; A^T]: GEMM over the output features N, with
  // R's column-major codes and transposed scale grid as the B operand.
  GemmArgs g{};
  g.M = M; g.N = K; g.K = N;
  g.A = gq_codes; g.lda = N / 2;
  g.B = rq_codes_cm; g.ldb = N / 2;
  g.sA = static_cast<const uint8_t*>(gq_scales); g.sA_rs = N / 16;
  g.sB = static_cast<const uint8_t*>(rq_scales_cm); g.sB_rs = N / 16;
  g.P = V;
  g.Wa = static_cast<const uint16_t*>(L1t); g.ra = rs;
  g.Wb = static_cast<const uint16_t*>(At); g.rb = r;
  g.C = dX; g.ldc = K;
  const bool out_bf16 = dxdt == FT_OUT_BF16;
  // the adapter gradients in the GEMM's launch (one kernel on the caller's stream)
  GemmArgs ga = bwd_shape(M, N, K, rs, r);
  if (gemm_w4a4_adapt_ok(ga)) {
    g.ad = ga.ad;
    g.ad.P[0] = V; g.ad.Q[0] = static_cast<const uint16_t*>(X); g.ad.out[0] = dAt;
    if (dB) { g.ad.P[1] = T; g.ad.Q[1] = static_cast<const uint16_t*>(G); g.ad.out[1] = dB; }
    uint8_t* w = static_cast<uint8_t*>(workspace);
    const size_t a_bytes = bwd_adapt_bytes(ga);
    void* gemm_ws = gemm_w4a4_workspace(M, K, N) ? w + a_bytes : nullptr;
    return launch_gemm_w4a4_adapt(g, out_bf16, stream, gemm_ws, a_bytes ? w : nullptr);
  }
  void* split_ws = nullptr;   // the last part of the workspace, when the GEMM splits its reduction
  if (gemm_w4a4_workspace(M, K, N))
    split_ws = static_cast<uint8_t*>(workspace) + align256(lora_grad_workspace(M, K, r)) +
               align256(lora_grad_workspace(M, N, r));
  auto gemm = [&](hipStream_t s, bool beside) {
    return (M && K) ? launch_gemm_w4a4(g, out_bf16, true, s, beside, split_ws) : FT_OK;
  };
  if (!side) {
    // the GEMM planned as when the adapter gradients run beside it, so that both
    // ways run the same kernels and give the same results bit for bit
    ft_status st = gemm(stream, true);
    if (st != FT_OK) return st;
    return adapter_grads(M, N, K, V, rs, r, X, G, T, dAt, dB, workspace, stream);
  }
  return gemm_with_adapter_grads(gemm, M, N, K, V, rs, r, X, G, T, dAt, dB, workspace, stream);
}

// Scratch of ft_linear_bwd_noalloc: a file-scope device array (each GPU the
// library runs on holds its own copy until the process ends).  In host code
// `scratch` names a host-side stand-in, not device memory: its device address
// is looked up once per device with hipGetSymbolAddress and only that address
// is handed to kernels.
static __device__ __align__(256) uint8_t scratch[FT_NOALLOC_SCRATCH_BYTES];

// the device address of `scratch` on the current device (nullptr on failure)
void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}
}  // namespace
}  // namespace ft

extern "C" ft_status ft_linear_bwd(int64_t M, int64_t N, int64_t K, ft_scale_mode mode,
                                   const uint8_t* gq_codes, const void* gq_scales,
                                   const uint8_t* rq_codes_cm, const void* rq_scales_cm,
                                   const float* V, const void* L1t, int32_t rs, const void* At, int32_t r,
                                   const void* X, const void* G, const float* T,
                                   void* dX, ft_out_dtype dxdt, float* dAt, float* dB,
                                   void* workspace, size_t ws_bytes, hipStream_t stream) {
  return ft::linear_bwd_impl(M, N, K, mode, gq_codes, gq_scales, rq_codes_cm, rq_scales_cm, V, L1t, rs, At, r, X,
                             G, T, dX, dxdt, dAt, dB, workspace, ws_bytes, stream, true);
}

extern "C" ft_status ft_linear_bwd_noalloc(int64_t M, int64_t N, int64_t K, ft_scale_mode mode,
                                           const uint8_t* gq_codes, const void* gq_scales,
                                           const uint8_t* rq_codes_cm, const void* rq_scales_cm,
                                           const float* V, const void* L1t, int32_t rs, const void* At,
                                           int32_t r, const void* X, const void* G, const float* T,
                                           void* dX, ft_out_dtype dxdt, float* dAt, float* dB,
                                           hipStream_t stream) {
  using namespace ft;
  if (M < 0 || N < 0 || K < 0 || r < 0) return FT_ESHAPE;
  const size_t need = ft_linear_bwd_workspace(M, N, K, r);
  if (need > FT_NOALLOC_SCRATCH_BYTES) return FT_ESPACE;
  void* ws = nullptr;
  if (need) {
    // validate everything else before touching the device
    const ft_status pre = linear_bwd_impl(M, N, K, mode, gq_codes, gq_scales, rq_codes_cm, rq_scales_cm, V, L1t,
                                          rs, At, r, X, G, T, dX, dxdt, dAt, dB, nullptr, 0, stream, false);
    if (pre != FT_EINVAL) return pre;   // the missing workspace is the only complaint expected here
    ws = scratch_ptr();
    if (!ws) return FT_EHIP;
  }
  return linear_bwd_impl(M, N, K, mode, gq_codes, gq_scales, rq_codes_cm, rq_scales_cm, V, L1t, rs, At, r, X, G,
                         T, dX, dxdt, dAt, dB, ws, need, stream, false);
}

namespace ft {
namespace {
ft_status adapter_grads(int64_t M, int64_t N, int64_t K, const float* V, int rs, int r, const void* X,
                        const void* G, const float* T, float* dAt, float* dB, void* workspace, hipStream_t stream) {
  if (!r) return FT_OK;
  const int rho = rs + r;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const size_t wa = align256(lora_grad_workspace(M, K, r));
  ft_status st = launch_lora_grad(V, rho, rs, r, static_cast<const uint16_t*>(X), M, K, dAt, ws, stream);
  if (st != FT_OK || !dB) return st;   // dB NULL: taken in the G pass (ft_quant_lowrank_db)
  return launch_lora_grad(T, rho, rs, r, static_cast<const uint16_t*>(G), M, N, dB, ws + wa, stream);
}
}  // namespace
}  // namespace ft

extern "C" ft_status ft_linear_fwd_op(int64_t M, int64_t N, int64_t K, const uint8_t* x_op,
                                      const uint8_t* x_op_scales, const uint8_t* r_op, const uint8_t* r_op_scales,
                                      const float* T, const void* L2, int32_t rs, const void* B, int32_t r,
                                      void* Y, ft_out_dtype ydt, hipStream_t stream) {
  using namespace ft;
  if (ydt != FT_OUT_F32 && ydt != FT_OUT_BF16) return FT_EINVAL;
  if (!mult16(M) || !mult16(N) || !mult16(K) || !ranks_ok(rs, r)) return FT_ESHAPE;
  if (M == 0 || N == 0) return FT_OK;
  const int rho = rs + r;
  if (!Y || (K && (!x_op || !x_op_scales || !r_op || !r_op_scales)) || (rho && !T) || (rs && !L2) || (r && !B))
    return FT_EINVAL;
  const void* ptrs[] = {Y, x_op, x_op_scales, r_op, r_op_scales, T, L2, B};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FT_EALIGN;
  const int64_t gk = op_groups(K);
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.A = x_op; g.lda = gk * 96;
  g.B = r_op; g.ldb = gk * 96;
  g.sA = x_op_scales; g.sA_rs = gk * 8;
  g.sB = r_op_scales; g.sB_rs = gk * 8;
  g.P = T;
  g.Wa = static_cast<const uint16_t*>(L2); g.ra = rs;
  g.Wb = static_cast<const uint16_t*>(B); g.rb = r;
  g.C = Y; g.ldc = N;
  return launch_gemm_m6(g, ydt == FT_OUT_BF16, false, stream);
}

extern "C" ft_status ft_linear_bwd_op(int64_t M, int64_t N, int64_t K, const uint8_t* g_op,
                                      const uint8_t* g_op_scales, const uint8_t* rt_op, const uint8_t* rt_op_scales,
                                      const float* V, const void* L1t, int32_t rs, const void* At, int32_t r,
                                      const void* X, const void* G, const float* T,
                                      void* dX, ft_out_dtype dxdt, float* dAt, float* dB,
                                      void* workspace, size_t ws_bytes, hipStream_t stream) {
  using namespace ft;
  if (dxdt != FT_OUT_F32 && dxdt != FT_OUT_BF16) return FT_EINVAL;
  if (!mult16(M) || !mult16(N) || !mult16(K) || !ranks_ok(rs, r)) return FT_ESHAPE;
  const int rho = rs + r;
  const size_t need = ft_linear_bwd_workspace(M, N, K, r);
  if (M && K && !dX) return FT_EINVAL;
  if (M && N && K && (!g_op || !g_op_scales || !rt_op || !rt_op_scales)) return FT_EINVAL;
  if (M && rho && !V) return FT_EINVAL;
  if ((rs && K && !L1t) || (r && K && (!At || !dAt))) return FT_EINVAL;   // dB may be NULL: not computed
  if (r && M && ((K && !X) || (N && !G) || !T)) return FT_EINVAL;
  if (need && (!workspace || ws_bytes < need)) return workspace ? FT_ESPACE : FT_EINVAL;
  const void* ptrs[] = {g_op, g_op_scales, rt_op, rt_op_scales, V, L1t, At, X, G, T, dX, dAt, dB, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FT_EALIGN;
  // dX = deq(Gq) deq(Rq) + V [L1^T; A^T]: reduction over the N output features;
  // the right operand is R^T's operand (pairs along N)
  const int64_t gn = op_groups(N);
  GemmArgs g{};
  g.M = M; g.N = K; g.K = N;
  g.A = g_op; g.lda = gn * 96;
  g.B = rt_op; g.ldb = gn * 96;
  g.sA = g_op_scales; g.sA_rs = gn * 8;
  g.sB = rt_op_scales; g.sB_rs = gn * 8;
  g.P = V;
  g.Wa = static_cast<const uint16_t*>(L1t); g.ra = rs;
  g.Wb = static_cast<const uint16_t*>(At); g.rb = r;
  g.C = dX; g.ldc = K;
  const bool out_bf16 = dxdt == FT_OUT_BF16;
  auto gemm = [&](hipStream_t s, bool) { return (M && K) ? launch_gemm_m6(g, out_bf16, true, s) : FT_OK; };
  return gemm_with_adapter_grads(gemm, M, N, K, V, rs, r, X, G, T, dAt, dB, workspace, stream);
}

// Precision variants (section 4.3 "Impact of Precision Configurations", Table 4):
// the backbone GEMM with the unquantized bf16 activations (W4A16: Eq. 2 with X in
// place of Q(X)) or output gradient (G16: Eq. 3 with G in place of Q(G)); R stays
// quantized.  The low-rank branches and adapter gradients are those of the
// W4A4G4 calls.
extern "C" ft_status ft_linear_fwd_a16(int64_t M, int64_t N, int64_t K, const void* X,
                                       const uint8_t* rq_codes, const void* rq_scales,
                                       const float* T, const void* L2, int32_t rs, const void* B, int32_t r,
                                       void* Y, ft_out_dtype ydt, hipStream_t stream) {
  using namespace ft;
  if (ydt != FT_OUT_F32 && ydt != FT_OUT_BF16) return FT_EINVAL;
  if (!mult16(M) || !mult16(N) || !mult16(K) || !ranks_ok(rs, r)) return FT_ESHAPE;
  if (M == 0 || N == 0) return FT_OK;
  const int rho = rs + r;
  if (!Y || (K && (!X || !rq_codes || !rq_scales)) || (rho && !T) || (rs && !L2) || (r && !B))
    return FT_EINVAL;
  const void* ptrs[] = {Y, X, rq_codes, rq_scales, T, L2, B};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FT_EALIGN;
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.A = static_cast<const uint8_t*>(X); g.lda = 2 * K;
  g.B = rq_codes; g.ldb = K / 2;
  g.sB = static_cast<const uint8_t*>(rq_scales); g.sB_rs = K / 16;
  g.P = T;
  g.Wa = static_cast<const uint16_t*>(L2); g.ra = rs;
  g.Wb = static_cast<const uint16_t*>(B); g.rb = r;
  g.C = Y; g.ldc = N;
  return launch_gemm_a16(g, ydt == FT_OUT_BF16, false, stream);
}

extern "C" ft_status ft_linear_bwd_g16(int64_t M, int64_t N, int64_t K, const void* G,
                                       const uint8_t* rq_codes_cm, const void* rq_scales_cm,
                                       const float* V, const void* L1t, int32_t rs, const void* At, int32_t r,
                                       const void* X, const float* T,
                                       void* dX, ft_out_dtype dxdt, float* dAt, float* dB,
                                       void* workspace, size_t ws_bytes, hipStream_t stream) {
  using namespace ft;
  if (dxdt != FT_OUT_F32 && dxdt != FT_OUT_BF16) return FT_EINVAL;
  if (!mult16(M) || !mult16(N) || !mult16(K) || !ranks_ok(rs, r)) return FT_ESHAPE;
  const int rho = rs + r;
  const size_t need = ft_linear_bwd_workspace(M, N, K, r);
  if (M && K && !dX) return FT_EINVAL;
  if (M && N && K && (!G || !rq_codes_cm || !rq_scales_cm)) return FT_EINVAL;
  if (M && rho && !V) return FT_EINVAL;
  if ((rs && K && !L1t) || (r && K && (!At || !dAt))) return FT_EINVAL;   // dB may be NULL: not computed
  if (r && M && ((K && !X) || (N && !G) || !T)) return FT_EINVAL;
  if (need && (!workspace || ws_bytes < need)) return workspace ? FT_ESPACE : FT_EINVAL;
  const void* ptrs[] = {G, rq_codes_cm, rq_scales_cm, V, L1t, At, X, T, dX, dAt, dB, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FT_EALIGN;
  // dX = G deq(Rq) + V [L1^T; A^T]: reduction over the N output features, R's
  // column-major codes and transposed scale grid as the right operand
  GemmArgs g{};
  g.M = M; g.N = K; g.K = N;
  g.A = static_cast<const uint8_t*>(G); g.lda = 2 * N;
  g.B = rq_codes_cm; g.ldb = N / 2;
  g.sB = static_cast<const uint8_t*>(rq_scales_cm); g.sB_rs = N / 16;
  g.P = V;
  g.Wa = static_cast<const uint16_t*>(L1t); g.ra = rs;
  g.Wb = static_cast<const uint16_t*>(At); g.rb = r;
  g.C = dX; g.ldc = K;
  const bool out_bf16 = dxdt == FT_OUT_BF16;
  auto gemm = [&](hipStream_t s, bool) { return (M && K) ? launch_gemm_a16(g, out_bf16, true, s) : FT_OK; };
  return gemm_with_adapter_grads(gemm, M, N, K, V, rs, r, X, G, T, dAt, dB, workspace, stream);
}

// Other quantization granularities (section 4.3 "Impact of Quantization
// Granularity", Table 5): Eq. 2 and Eq. 3 with every 4-bit operand scaled per
// 1 x group elements along its reduction axis (ft_quant_group); the backward's
// right operand is the re-quantized transpose of Q(R) (ft_requant_group_t).
extern "C" ft_status ft_linear_fwd_grp(int64_t M, int64_t N, int64_t K, int32_t group,
                                       const uint8_t* xq_codes, const uint8_t* xq_scales,
                                       const uint8_t* rq_codes, const uint8_t* rq_scales,
                                       const float* T, const void* L2, int32_t rs, const void* B, int32_t r,
                                       void* Y, ft_out_dtype ydt, hipStream_t stream) {
  using namespace ft;
  if (ydt != FT_OUT_F32 && ydt != FT_OUT_BF16) return FT_EINVAL;
  if (group != 16 && group != 32) return FT_EINVAL;
  if (!mult16(M) || !mult16(N) || !mult16(K) || !ranks_ok(rs, r)) return FT_ESHAPE;
  if (M == 0 || N == 0) return FT_OK;
  if (K % 128 != 0) return FT_ENOTSUP;
  const int rho = rs + r;
  if (!Y || (K && (!xq_codes || !xq_scales || !rq_codes || !rq_scales)) || (rho && !T) || (rs && !L2) || (r && !B))
    return FT_EINVAL;
  const void* ptrs[] = {Y, xq_codes, xq_scales, rq_codes, rq_scales, T, L2, B};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FT_EALIGN;
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.A = xq_codes; g.lda = K / 2;
  g.B = rq_codes; g.ldb = K / 2;
  g.sA = xq_scales; g.sA_rs = K / group;
  g.sB = rq_scales; g.sB_rs = K / group;
  g.P = T;
  g.Wa = static_cast<const uint16_t*>(L2); g.ra = rs;
  g.Wb = static_cast<const uint16_t*>(B); g.rb = r;
  g.C = Y; g.ldc = N;
  return launch_gemm_w4a4_groups(g, group, ydt == FT_OUT_BF16, false, stream);
}

extern "C" ft_status ft_linear_bwd_grp(int64_t M, int64_t N, int64_t K, int32_t group,
                                       const uint8_t* gq_codes, const uint8_t* gq_scales,
                                       const uint8_t* rtq_codes, const uint8_t* rtq_scales,
                                       const float* V, const void* L1t, int32_t rs, const void* At, int32_t r,
                                       const void* X, const void* G, const float* T,
                                       void* dX, ft_out_dtype dxdt, float* dAt, float* dB,
                                       void* workspace, size_t ws_bytes, hipStream_t stream) {
  using namespace ft;
  if (dxdt != FT_OUT_F32 && dxdt != FT_OUT_BF16) return FT_EINVAL;
  if (group != 16 && group != 32) return FT_EINVAL;
  if (!mult16(M) || !mult16(N) || !mult16(K) || !ranks_ok(rs, r)) return FT_ESHAPE;
  if (M && K && N % 128 != 0) return FT_ENOTSUP;
  const int rho = rs + r;
  const size_t need = ft_linear_bwd_workspace(M, N, K, r);
  if (M && K && !dX) return FT_EINVAL;
  if (M && N && K && (!gq_codes || !gq_scales || !rtq_codes || !rtq_scales)) return FT_EINVAL;
  if (M && rho && !V) return FT_EINVAL;
  if ((rs && K && !L1t) || (r && K && (!At || !dAt))) return FT_EINVAL;   // dB may be NULL: not computed
  if (r && M && ((K && !X) || (N && !G) || !T)) return FT_EINVAL;
  if (need && (!workspace || ws_bytes < need)) return workspace ? FT_ESPACE : FT_EINVAL;
  const void* ptrs[] = {gq_codes, gq_scales, rtq_codes, rtq_scales, V, L1t, At, X, G, T, dX, dAt, dB, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FT_EALIGN;
  GemmArgs g{};
  g.M = M; g.N = K; g.K = N;
  g.A = gq_codes; g.lda = N / 2;
  g.B = rtq_codes; g.ldb = N / 2;
  g.sA = gq_scales; g.sA_rs = N / group;
  g.sB = rtq_scales; g.sB_rs = N / group;
  g.P = V;
  g.Wa = static_cast<const uint16_t*>(L1t); g.ra = rs;
  g.Wb = static_cast<const uint16_t*>(At); g.rb = r;
  g.C = dX; g.ldc = K;
  const bool out_bf16 = dxdt == FT_OUT_BF16;
  auto gemm = [&](hipStream_t s, bool) {
    return (M && K) ? launch_gemm_w4a4_groups(g, group, out_bf16, true, s) : FT_OK;
  };
  return gemm_with_adapter_grads(gemm, M, N, K, V, rs, r, X, G, T, dAt, dB, workspace, stream);
}
