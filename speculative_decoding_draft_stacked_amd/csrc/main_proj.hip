// Row RMSNorm that completes the DSpark context producer,
// ctx_hidden = main_norm(main_proj(aux)), for gfx950.
//
// Method: vLLM PR #46995 ("[Spec Decode] DSpark", key source snippets:
// combine_hidden_states applies the RMSNorm main_norm over the hidden size to
// the output of the bias-free projection main_proj). The projection runs as
// the write kernels' GEMM with a row-output epilogue: it stores the rounded
// outputs and the sum of squares of each 128-feature group of each token. This
// kernel adds a token's group sums in a fixed order (deterministic), forms
// inv = 1 / sqrt(sum / H + eps) and rewrites the row in place as
// round(y * inv * g), in fp32 with the weight widened to fp32 at pack time.
//
// When the projection is split over K for small batches, its workgroups leave
// fp32 partial sums instead, and the norm kernel first adds a token's parts in
// a fixed order and rounds them (the projection's output rounding).
//
// Mapping: one wave per token row (a workgroup of four waves per token in the
// K-split form, which has few tokens), 16-byte accesses, 8 features per lane
// per pass (a pass covers 512 features); sums across the wave use a butterfly,
// which leaves the same bits in every lane.
#include "internal.h"

namespace dspark {
namespace {

constexpr int kThreads = 256;

template <bool FP16>
__device__ __forceinline__ float to_f(uint32_t b) {
  if (FP16) return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
  return __uint_as_float(b << 16);
}

template <bool FP16>
__device__ __forceinline__ uint32_t from_f(float f) {
  if (FP16) return __builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
  return __builtin_bit_cast(uint16_t, (__bf16)f);               // round to nearest even
}

template <bool FP16>
__global__ __launch_bounds__(kThreads) void row_norm_kernel(uint16_t* y, int64_t y_stride,
                                                             const float* partial, int64_t T,
                                                             int64_t groups, const float* g,
                                                             float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform over the wave
  float ss = 0.0f;
  for (int64_t r = lane; r < groups; r += 64) ss += partial[r * T + t];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  const int64_t H = groups * 128;
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);
  uint16_t* row = y + t * y_stride;
  for (int64_t c = lane * 8; c < H; c += 64 * 8) {
    const uint4 u = *reinterpret_cast<const uint4*>(row + c);
    const float4 g0 = *reinterpret_cast<const float4*>(g + c);
    const float4 g1 = *reinterpret_cast<const float4*>(g + c + 4);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    const float gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = to_f<FP16>(w[i] & 0xFFFFu) * inv * gw[2 * i];
      const float hi = to_f<FP16>(w[i] >> 16) * inv * gw[2 * i + 1];
      o[i] = from_f<FP16>(lo) | (from_f<FP16>(hi) << 16);
    }
    *reinterpret_cast<uint4*>(row + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// K-split form: partial holds ksplits fp32 partial projections [ks, T, H].
// A workgroup of 4 waves takes one token: each wave adds the parts of a
// quarter of the features in order (deterministic), rounds them to the dtype
// (the linear's output rounding) and keeps them in registers (H <= 8192: up to
// 4 passes of 512 features per wave); the four partial sums of squares are
// added in wave order through LDS, and each wave writes round(y * inv * g).
constexpr int kMaxPasses = 4;

template <bool FP16>
__global__ __launch_bounds__(kThreads) void row_norm_split_kernel(uint16_t* y, int64_t y_stride,
                                                                   const float* partial,
                                                                   int64_t T, int64_t H, int ks,
                                                                   const float* g, float eps) {
  __shared__ float wsum[kThreads / 64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t = blockIdx.x;
  const int64_t quarter = H / 4;  // H % 512 == 0, so a quarter is whole passes of 128
  uint32_t yv[kMaxPasses][4];
  float ss = 0.0f;
#pragma unroll
  for (int pp = 0; pp < kMaxPasses; ++pp) {
    const int64_t c = wave * quarter + (int64_t)pp * 512 + lane * 8;
    if ((int64_t)pp * 512 + lane * 8 < quarter) {
      float sum[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      for (int q = 0; q < ks; ++q) {
        const float* src = partial + ((int64_t)q * T + t) * H + c;
        const float4 a0 = *reinterpret_cast<const float4*>(src);
        const float4 a1 = *reinterpret_cast<const float4*>(src + 4);
        sum[0] += a0.x, sum[1] += a0.y, sum[2] += a0.z, sum[3] += a0.w;
        sum[4] += a1.x, sum[5] += a1.y, sum[6] += a1.z, sum[7] += a1.w;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = from_f<FP16>(sum[2 * i]), hi = from_f<FP16>(sum[2 * i + 1]);
        const float flo = to_f<FP16>(lo), fhi = to_f<FP16>(hi);
        ss += flo * flo + fhi * fhi;
        yv[pp][i] = lo | (hi << 16);
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  if (lane == 0) wsum[wave] = ss;
  __syncthreads();
  const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  uint16_t* row = y + t * y_stride;
#pragma unroll
  for (int pp = 0; pp < kMaxPasses; ++pp) {
    const int64_t c = wave * quarter + (int64_t)pp * 512 + lane * 8;
    if ((int64_t)pp * 512 + lane * 8 < quarter) {
      const float4 g0 = *reinterpret_cast<const float4*>(g + c);
      const float4 g1 = *reinterpret_cast<const float4*>(g + c + 4);
      const float gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = to_f<FP16>(yv[pp][i] & 0xFFFFu) * inv * gw[2 * i];
        const float hi = to_f<FP16>(yv[pp][i] >> 16) * inv * gw[2 * i + 1];
        o[i] = from_f<FP16>(lo) | (from_f<FP16>(hi) << 16);
      }
      *reinterpret_cast<uint4*>(row + c) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

}  // namespace

hipError_t launch_row_norm(uint16_t* y, int64_t y_stride, const float* partial, int64_t T,
                           int64_t groups, int ksplits, const float* g, float eps, bool is_fp16,
                           hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int64_t blocks = (T + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)blocks), block(kThreads);
  if (ksplits > 1) {
    // a workgroup per token; a wave per quarter of the features
    const int64_t H = groups * 128;
    if (H > 4 * kMaxPasses * 512 || H % 512 != 0 || T > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (is_fp16)
      hipLaunchKernelGGL(row_norm_split_kernel<true>, dim3((uint32_t)T), block, 0, stream, y,
                         y_stride, partial, T, H, ksplits, g, eps);
    else
      hipLaunchKernelGGL(row_norm_split_kernel<false>, dim3((uint32_t)T), block, 0, stream, y,
                         y_stride, partial, T, H, ksplits, g, eps);
  } else if (is_fp16) {
    hipLaunchKernelGGL(row_norm_kernel<true>, grid, block, 0, stream, y, y_stride, partial, T,
                       groups, g, eps);
  } else {
    hipLaunchKernelGGL(row_norm_kernel<false>, grid, block, 0, stream, y, y_stride, partial, T,
                       groups, g, eps);
  }
  return hipGetLastError();
}

}  // namespace dspark
