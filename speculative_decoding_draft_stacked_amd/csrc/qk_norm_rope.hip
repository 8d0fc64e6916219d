// In-place table QK-RMSNorm + neox RoPE on a fused QKV tensor for gfx950.
//
// Method: sglang PR #31847 ("[spec decoding] support inkling dspark", key
// source snippets: table_qk_norm_rope_ / _table_qk_norm_rope_kernel). Row t of
// the tensor is [NHQ query heads | NHK key heads | value heads | padding], each
// head D wide, so query head h and key head j both start at column h * D with
// h = NHQ + j for a key head. Each of the NHQ + NHK heads is normalised in
// fp32 (mean of squares over D, plus eps, reciprocal square root, times the
// query or key norm weight), rounded to the dtype, rotated neox-style over the
// pairs (i, i + D/2) with the cos | sin row of the token's position, rounded
// again and stored back in place. Value heads and padding are not touched.
//
// Mapping. The op moves every byte of the query and key heads through HBM once
// in each direction, so it is laid out for coalescing only: D / 16 lanes take
// one (token, head), lane j owning elements [8j, 8j + 8) of the first half and
// their rotation partners 8j + D/2 + [0, 8), read and written as 16-byte
// vectors. A wave covers 64 / (D / 16) consecutive heads of a row, i.e. one
// contiguous run of memory; the sum of squares needs log2(D / 16) lane swaps.
// The table row of a token (D fp32 values) is shared by its heads through the
// caches.
#include "internal.h"

namespace dspark {
namespace {

constexpr int kThreads = 256;

template <bool FP16>
struct Half16;

template <>
struct Half16<false> {  // bf16
  static __device__ __forceinline__ float to_f(uint32_t b) { return __uint_as_float(b << 16); }
  static __device__ __forceinline__ uint32_t from_f(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);  // round to nearest even
  }
};

template <>
struct Half16<true> {  // fp16
  static __device__ __forceinline__ float to_f(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
  }
  static __device__ __forceinline__ uint32_t from_f(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
  }
};

template <typename E>
__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = E::to_f(w[i] & 0xFFFFu);
    f[2 * i + 1] = E::to_f(w[i] >> 16);
  }
}

template <typename E>
__device__ __forceinline__ uint4 pack8(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = E::from_f(f[2 * i]) | (E::from_f(f[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// 8 consecutive norm-weight entries as fp32: the dtype's 16-bit patterns, or fp32.
template <typename E, bool WF32>
__device__ __forceinline__ void load_weight8(const void* w, int off, float* f) {
  if (WF32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(w) + off);
    const float4 a = p[0], b = p[1];
    f[0] = a.x, f[1] = a.y, f[2] = a.z, f[3] = a.w, f[4] = b.x, f[5] = b.y, f[6] = b.z, f[7] = b.w;
  } else {
    unpack8<E>(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + off), f);
  }
}

template <bool FP16, int D, bool WF32>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(const QkArgs a) {
  using E = Half16<FP16>;
  constexpr int TPH = D / 16;             // lanes per (token, head)
  constexpr int HPB = kThreads / TPH;     // heads per workgroup
  const int tid = threadIdx.x;
  const int j = tid % TPH;
  const int64_t task = (int64_t)blockIdx.x * HPB + tid / TPH;
  if (task >= a.T * a.NHT) return;  // uniform over the TPH lanes of a task
  const int64_t t = task / a.NHT;
  const int h = (int)(task % a.NHT);
  const int64_t p = a.pos[t];
  if (p < 0 || p >= a.P) {
    if (h == 0 && j == 0 && a.err) atomicAdd(a.err, 1ull);  // once per token
    return;
  }
  uint16_t* row = a.qkv + t * a.row_stride + (int64_t)h * D + j * 8;
  // each head is read and rewritten once: nontemporal accesses (10% faster
  // than default ones on an 8k-token batch)
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 q1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row));
  const u32x4 q2 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + D / 2));
  const uint4 u1 = make_uint4(q1[0], q1[1], q1[2], q1[3]);
  const uint4 u2 = make_uint4(q2[0], q2[1], q2[2], q2[3]);
  float x1[8], x2[8];
  unpack8<E>(u1, x1);
  unpack8<E>(u2, x2);
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += x1[i] * x1[i] + x2[i] * x2[i];
#pragma unroll
  for (int m = 1; m < TPH; m <<= 1) ss += __shfl_xor(ss, m);
  const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
  const void* w = h < a.NHQ ? a.qw : a.kw;
  float w1[8], w2[8];
  load_weight8<E, WF32>(w, j * 8, w1);
  load_weight8<E, WF32>(w, D / 2 + j * 8, w2);
  const float4* cs = reinterpret_cast<const float4*>(a.table + p * D + j * 8);
  const float4* sn = reinterpret_cast<const float4*>(a.table + p * D + D / 2 + j * 8);
  const float4 c0 = cs[0], c1 = cs[1], s0 = sn[0], s1 = sn[1];
  const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  float o1[8], o2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float n1 = E::to_f(E::from_f(x1[i] * inv * w1[i]));
    const float n2 = E::to_f(E::from_f(x2[i] * inv * w2[i]));
    o1[i] = n1 * c[i] - n2 * s[i];
    o2[i] = n2 * c[i] + n1 * s[i];
  }
  const uint4 p1 = pack8<E>(o1), p2 = pack8<E>(o2);
  __builtin_nontemporal_store((u32x4){p1.x, p1.y, p1.z, p1.w}, reinterpret_cast<u32x4*>(row));
  __builtin_nontemporal_store((u32x4){p2.x, p2.y, p2.z, p2.w},
                              reinterpret_cast<u32x4*>(row + D / 2));
}

template <bool FP16, int D, bool WF32>
hipError_t launch(const QkArgs& a, hipStream_t stream) {
  constexpr int HPB = kThreads / (D / 16);
  const int64_t blocks = (a.T * a.NHT + HPB - 1) / HPB;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((qk_norm_rope_kernel<FP16, D, WF32>), dim3((uint32_t)blocks),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool FP16, int D>
hipError_t launch_w(const QkArgs& a, bool weight_fp32, hipStream_t stream) {
  return weight_fp32 ? launch<FP16, D, true>(a, stream) : launch<FP16, D, false>(a, stream);
}

template <bool FP16>
hipError_t launch_d(const QkArgs& a, int head_dim, bool weight_fp32, hipStream_t stream) {
  if (head_dim == 128) return launch_w<FP16, 128>(a, weight_fp32, stream);
  if (head_dim == 64) return launch_w<FP16, 64>(a, weight_fp32, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_qk_norm_rope(const QkArgs& a, int head_dim, bool is_fp16, bool weight_fp32,
                               hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  return is_fp16 ? launch_d<true>(a, head_dim, weight_fp32, stream)
                 : launch_d<false>(a, head_dim, weight_fp32, stream);
}

}  // namespace dspark
