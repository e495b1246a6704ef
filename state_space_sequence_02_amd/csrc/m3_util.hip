// m3_util.hip -- small device utilities shared by the entry points.
#include "m3_internal.h"

namespace m3 {
namespace {

__global__ void copy_or_zero_kernel(float* dst, const float* src, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace

hipError_t launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t stream) {
  if (n == 0 || dst == src) return hipSuccess;
  hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     dst, src, n);
  return hipGetLastError();
}

}  // namespace m3
