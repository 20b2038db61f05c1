// GELU between the two linears of an MLP block: bf16 in, fp32 math (gelu_f),
// bf16 out (round to nearest even).
#include "ft_device.h"

namespace ft {
namespace {

__global__ void gelu_fwd_kernel(const v4i* __restrict__ y, int64_t n8, v4i* __restrict__ h) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const v4i v = y[i];
  const uint32_t w[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = f32_to_bf16_rne(gelu_f(bf16lo_to_f32(w[k]))) | (f32_to_bf16_rne(gelu_f(bf16hi_to_f32(w[k]))) << 16);
  h[i] = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
}

__global__ void gelu_bwd_kernel(const v4i* __restrict__ y, const v4i* __restrict__ dh, int64_t n8,
                                v4i* __restrict__ dy) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const v4i v = y[i], g = dh[i];
  const uint32_t w[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
  const uint32_t d[4] = {(uint32_t)g.x, (uint32_t)g.y, (uint32_t)g.z, (uint32_t)g.w};
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo = gelu_grad_f(bf16lo_to_f32(w[k])) * bf16lo_to_f32(d[k]);
    const float hi = gelu_grad_f(bf16hi_to_f32(w[k])) * bf16hi_to_f32(d[k]);
    o[k] = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
  }
  dy[i] = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
}

}  // namespace
}  // namespace ft

extern "C" ft_status ft_gelu_fwd(const void* y, int64_t n, void* h, hipStream_t stream) {
  using namespace ft;
  if (n < 0 || n % 8) return FT_ESHAPE;
  if (n == 0) return FT_OK;
  if (!y || !h) return FT_EINVAL;
  if (!aligned16(y) || !aligned16(h)) return FT_EALIGN;
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(gelu_fwd_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const v4i*>(y), n8, static_cast<v4i*>(h));
  return launch_status();
}

extern "C" ft_status ft_gelu_bwd(const void* y, const void* dh, int64_t n, void* dy, hipStream_t stream) {
  using namespace ft;
  if (n < 0 || n % 8) return FT_ESHAPE;
  if (n == 0) return FT_OK;
  if (!y || !dh || !dy) return FT_EINVAL;
  if (!aligned16(y) || !aligned16(dh) || !aligned16(dy)) return FT_EALIGN;
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(gelu_bwd_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const v4i*>(y), static_cast<const v4i*>(dh), n8, static_cast<v4i*>(dy));
  return launch_status();
}
