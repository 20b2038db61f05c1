// Small utility kernels shared by the entry points.
#include "ft_common.h"

namespace ft {

__global__ void fill_zero_f32_kernel(float* __restrict__ p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = 0.0f;
}

ft_status fill_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return FT_OK;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return launch_status();
}

}  // namespace ft
