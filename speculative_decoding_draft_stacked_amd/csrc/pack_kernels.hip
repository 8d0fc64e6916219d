// One-time pack helpers: widening the k_norm weights to fp32 and comparing two
// rotary tables bit for bit on the device.
#include "internal.h"

namespace dspark {
namespace {

__global__ void widen_kernel(const void* src, int dtype, float* dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (dtype == DSPARK_FP32) {
    dst[i] = static_cast<const float*>(src)[i];
  } else {
    const uint32_t b = static_cast<const uint16_t*>(src)[i];
    dst[i] = dtype == DSPARK_BF16 ? __uint_as_float(b << 16)
                                  : (float)__builtin_bit_cast(_Float16, (uint16_t)b);
  }
}

__global__ void compare_kernel(const uint32_t* a, const uint32_t* b, int64_t n, int* differ) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n && a[i] != b[i]) *differ = 1;  // every writer stores the same value
}

}  // namespace

hipError_t launch_widen_to_f32(const void* src, int dtype, float* dst, int64_t n,
                               hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(widen_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, stream, src,
                     dtype, dst, n);
  return hipGetLastError();
}

hipError_t launch_compare_f32(const float* a, const float* b, int64_t n, int* differ,
                              hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(compare_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(a), reinterpret_cast<const uint32_t*>(b), n,
                     differ);
  return hipGetLastError();
}

}  // namespace dspark
