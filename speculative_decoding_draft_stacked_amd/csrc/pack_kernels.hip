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

// Blocked weight layout (see dspark_pack_buffers in dspark.h): block (rt, c)
// holds rows [128 rt, 128 rt + 128) x columns [64 c, 64 c + 64) as 1024
// pieces of 8 elements; piece q = (g * 4 + s) * 64 + l is row 128 rt + 32 g +
// l % 32, columns 64 c + 32 (l / 32) + 8 s + [0, 8). Columns past H are zero.
__global__ void block_weight_kernel(const uint16_t* plain, int64_t H, int64_t nk, int64_t pieces,
                                    uint16_t* blk) {
  const int64_t P = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (P >= pieces) return;
  const int64_t rt = P / (nk * 1024);
  const int64_t c = (P / 1024) % nk;
  const int q = (int)(P % 1024);
  const int g = q / 256, s = (q / 64) % 4, l = q % 64;
  const int64_t row = rt * 128 + 32 * g + (l % 32);
  const int64_t k = 64 * c + 32 * (l / 32) + 8 * s;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (k < H) v = *reinterpret_cast<const uint4*>(plain + row * H + k);  // H % 8 == 0
  *reinterpret_cast<uint4*>(blk + P * 8) = v;
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

hipError_t launch_block_weight(const uint16_t* plain, int64_t rows, int64_t H, uint16_t* blk,
                               hipStream_t stream) {
  const int64_t nk = (H + 63) / 64;
  const int64_t pieces = rows / 128 * nk * 1024;
  if (pieces <= 0) return hipSuccess;
  hipLaunchKernelGGL(block_weight_kernel, dim3((uint32_t)((pieces + 255) / 256)), dim3(256), 0,
                     stream, plain, H, nk, pieces, blk);
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
