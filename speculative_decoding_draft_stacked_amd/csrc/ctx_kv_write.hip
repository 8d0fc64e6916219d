// Fused context-KV write for gfx950: one MFMA GEMM of ctx_hidden [T, H] against
// the stacked KV weight [N_tot, H], whose epilogue rounds the projection to the
// activation dtype, applies the per-head K RMSNorm and the neox table rotation,
// and scatters K and V into every layer's pool.
//
// Method: sglang PR #31986 (one GEMM over the stacked KV rows of all draft
// layers, then per-head K RMSNorm and shared RoPE) and sglang PR #31847 (the
// same norm/rotation arithmetic in "_table_qk_norm_rope_kernel", and the
// write's validity rule: loc < 0 skipped, commit_lens truncating a flattened
// [B, W] window).
//
// Tiling. The GEMM is computed transposed, Y^T = W_stacked * X^T: weight rows
// run along the MFMA M axis and tokens along N, so both operands are K-major
// in memory and no transpose is needed. A workgroup (4 waves) owns BN = 128
// weight rows, i.e. one head of 128 or two heads of 64, so a tile never
// straddles a head and the norm and the (d, d + D/2) rotation pairs are local
// to it, and BT tokens. The K loop stages 64-wide slices of both operands
// through double-buffered LDS with rows padded to 144 bytes so that the
// 16-byte fragment reads of 8 consecutive rows fall on distinct banks.
// MFMA: v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation.
//
// Epilogue. Accumulators (+ bias) are rounded once to the dtype (the GEMM's
// output dtype) into an LDS tile [BT][BN]. Each (token, head) is then handled
// by D/16 lanes: every lane owns 8 elements of the first half and their 8
// rotation partners in the second half, so the rotation needs no exchange and
// the sum of squares needs log2(D/16) lane swaps. K is normalised in fp32
// (x * inv * w), rounded, rotated in fp32 and rounded; V is copied. Stores are
// 16-byte vectors into the pool row of the token's slot.
#include "internal.h"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BN = 128;       // weight rows per tile
constexpr int BK = 64;        // K slice per pipeline stage
constexpr int LDK = BK + 8;   // padded LDS row of an operand tile (elements)
constexpr int NTHREADS = 256;

template <bool FP16>
struct Elem;

template <>
struct Elem<false> {  // bf16
  using vec8 = bf16x8;
  static __device__ __forceinline__ float to_f(uint32_t b) { return __uint_as_float(b << 16); }
  static __device__ __forceinline__ uint32_t from_f(float f) {
    __bf16 h = (__bf16)f;  // round to nearest even
    return __builtin_bit_cast(uint16_t, h);
  }
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Elem<true> {  // fp16
  using vec8 = f16x8;
  static __device__ __forceinline__ float to_f(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
  }
  static __device__ __forceinline__ uint32_t from_f(float f) {
    _Float16 h = (_Float16)f;  // round to nearest even
    return __builtin_bit_cast(uint16_t, h);
  }
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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

template <bool FP16, int D, bool BIAS, bool COMMIT, int BT, int WAVES_N>
__global__ __launch_bounds__(NTHREADS) void ctx_kv_write_kernel(const WriteArgs a) {
  using E = Elem<FP16>;
  using vec8 = typename E::vec8;
  constexpr int WAVES_T = 4 / WAVES_N;
  constexpr int MB = BN / 32 / WAVES_N;  // 32-row blocks per wave
  constexpr int NB = BT / 32 / WAVES_T;  // 32-token blocks per wave
  constexpr int CPR = BK / 8;            // 16-byte chunks per operand row slice
  constexpr int W_CHUNKS = BN * CPR / NTHREADS;
  constexpr int X_CHUNKS = BT * CPR / NTHREADS;
  static_assert(MB >= 1 && NB >= 1 && W_CHUNKS >= 1 && X_CHUNKS >= 1, "tile shape");
  static_assert(BN % D == 0, "a tile holds whole heads");

  constexpr int SW = BN * LDK;
  constexpr int SX = BT * LDK;
  constexpr int LDO = BN + 4;  // output tile row: 264 bytes, 8-byte aligned rows
  constexpr int OPER = 2 * (SW + SX);
  constexpr int OUT = BT * LDO;
  __shared__ __align__(16) uint16_t smem[OPER > OUT ? OPER : OUT];
  uint16_t* sW = smem;
  uint16_t* sX = smem + 2 * SW;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_n = wave / WAVES_T;
  const int wave_t = wave % WAVES_T;

  const int64_t T = a.T;
  const int H = a.H;
  const int64_t t_tiles = (T + BT - 1) / BT;
  const int64_t bid = blockIdx.x;
  const int64_t t_blk = bid % t_tiles;
  const int64_t n_blk = bid / t_tiles;
  const int64_t n0 = n_blk * BN;
  const int64_t t0 = t_blk * BT;
  const int nk = (H + BK - 1) / BK;

  uint4 rw[W_CHUNKS];
  uint4 rx[X_CHUNKS];
  const uint4 zero = make_uint4(0, 0, 0, 0);

  auto load = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < W_CHUNKS; ++i) {
      const int c = tid + i * NTHREADS;
      const int row = c / CPR;
      const int k = k0 + (c % CPR) * 8;
      rw[i] = (k < H) ? *reinterpret_cast<const uint4*>(a.w + (n0 + row) * (int64_t)H + k) : zero;
    }
#pragma unroll
    for (int i = 0; i < X_CHUNKS; ++i) {
      const int c = tid + i * NTHREADS;
      const int row = c / CPR;
      const int k = k0 + (c % CPR) * 8;
      const int64_t t = t0 + row;
      rx[i] = (k < H && t < T) ? *reinterpret_cast<const uint4*>(a.x + t * a.x_stride + k) : zero;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < W_CHUNKS; ++i) {
      const int c = tid + i * NTHREADS;
      *reinterpret_cast<uint4*>(sW + buf * SW + (c / CPR) * LDK + (c % CPR) * 8) = rw[i];
    }
#pragma unroll
    for (int i = 0; i < X_CHUNKS; ++i) {
      const int c = tid + i * NTHREADS;
      *reinterpret_cast<uint4*>(sX + buf * SX + (c / CPR) * LDK + (c % CPR) * 8) = rx[i];
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
    const uint16_t* cw = sW + cur * SW;
    const uint16_t* cx = sX + cur * SX;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      // lane l supplies row (l % 32) and the 8 consecutive k at 8 * (l / 32)
      const int kof = kk * 16 + (lane >> 5) * 8;
      vec8 af[MB], bfr[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[mb] = *reinterpret_cast<const vec8*>(
            cw + (wave_n * MB * 32 + mb * 32 + (lane & 31)) * LDK + kof);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        bfr[nb] = *reinterpret_cast<const vec8*>(
            cx + (wave_t * NB * 32 + nb * 32 + (lane & 31)) * LDK + kof);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = E::mfma(af[mb], bfr[nb], acc[mb][nb]);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue 1: accumulators (+ bias) -> dtype, into the LDS tile [BT][LDO].
  // 32x32 accumulator layout: lane l holds column (token) l % 32 and, in
  // register r, row 8 * (r / 4) + 4 * (l / 32) + r % 4.
  uint16_t* sO = smem;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int tok = wave_t * NB * 32 + nb * 32 + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = wave_n * MB * 32 + mb * 32 + 8 * q + 4 * (lane >> 5);
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = acc[mb][nb][4 * q + i];
          if (BIAS) v[i] += E::to_f(a.bias[n0 + row + i]);
        }
        uint2 packed;
        packed.x = E::from_f(v[0]) | (E::from_f(v[1]) << 16);
        packed.y = E::from_f(v[2]) | (E::from_f(v[3]) << 16);
        *reinterpret_cast<uint2*>(sO + tok * LDO + row) = packed;
      }
    }
  }
  __syncthreads();

  // ---- epilogue 2: per (token, head): norm + rotation for K, copy for V, scatter.
  constexpr int TPH = D / 16;  // lanes per (token, head)
  constexpr int HPT = BN / D;  // heads per tile
  constexpr int ROUNDS = BT * HPT * TPH / NTHREADS;
  static_assert(ROUNDS * NTHREADS == BT * HPT * TPH, "epilogue work split");
  const int two_nh = 2 * a.NH;
#pragma unroll 1
  for (int r = 0; r < ROUNDS; ++r) {
    const int idx = r * NTHREADS + tid;
    const int task = idx / TPH;
    const int j = idx % TPH;
    const int tt = task / HPT;
    const int hd = task % HPT;
    const int64_t t = t0 + tt;
    if (t >= T) continue;  // uniform over the TPH lanes of a task
    const int64_t loc = a.locs[t];
    bool valid = loc >= 0;
    if (COMMIT) valid = valid && (t % a.W) < a.commit[t / a.W];
    if (!valid) continue;
    const int64_t g = (n0 + hd * D) / D;  // global head: layer-major, K heads then V heads
    const int layer = (int)(g / two_nh);
    const int jj = (int)(g % two_nh);
    const bool is_k = jj < a.NH;
    const int n = is_k ? jj : jj - a.NH;
    const int64_t p = a.pos[t];
    if (p < 0 || p >= a.P || loc >= a.slots[layer]) {
      if (j == 0 && jj == 0) atomicAdd(a.err, 1ull);  // once per (row, layer)
      continue;
    }
    const uint16_t* src = sO + tt * LDO + hd * D + j * 8;
    const uint4 u1 = *reinterpret_cast<const uint4*>(src);
    const uint4 u2 = *reinterpret_cast<const uint4*>(src + D / 2);
    if (is_k) {
      float x1[8], x2[8];
      unpack8<E>(u1, x1);
      unpack8<E>(u2, x2);
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += x1[i] * x1[i] + x2[i] * x2[i];
#pragma unroll
      for (int m = 1; m < TPH; m <<= 1) ss += __shfl_xor(ss, m);
      const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
      const float* gw = a.knw + (int64_t)layer * D + j * 8;
      const float* cs = a.table + p * D + j * 8;
      float o1[8], o2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float n1 = E::to_f(E::from_f(x1[i] * inv * gw[i]));
        const float n2 = E::to_f(E::from_f(x2[i] * inv * gw[i + D / 2]));
        const float c = cs[i];
        const float s = cs[i + D / 2];
        o1[i] = n1 * c - n2 * s;
        o2[i] = n2 * c + n1 * s;
      }
      uint16_t* dst = a.pk[layer] + loc * a.ks0[layer] + n * D + j * 8;
      *reinterpret_cast<uint4*>(dst) = pack8<E>(o1);
      *reinterpret_cast<uint4*>(dst + D / 2) = pack8<E>(o2);
    } else {
      uint16_t* dst = a.pv[layer] + loc * a.vs0[layer] + n * D + j * 8;
      *reinterpret_cast<uint4*>(dst) = u1;
      *reinterpret_cast<uint4*>(dst + D / 2) = u2;
    }
  }
}

template <bool FP16, int D, bool BIAS, bool COMMIT, int BT, int WAVES_N>
hipError_t launch_tile(const WriteArgs& a, hipStream_t stream) {
  const int64_t n_tiles = (int64_t)a.L * 2 * a.NH * D / BN;
  const int64_t t_tiles = (a.T + BT - 1) / BT;
  const int64_t grid = n_tiles * t_tiles;
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((ctx_kv_write_kernel<FP16, D, BIAS, COMMIT, BT, WAVES_N>), dim3((uint32_t)grid),
                     dim3(NTHREADS), 0, stream, a);
  return hipGetLastError();
}

template <bool FP16, int D, bool BIAS, bool COMMIT>
hipError_t launch_by_rows(const WriteArgs& a, hipStream_t stream) {
  if (a.T <= 32) return launch_tile<FP16, D, BIAS, COMMIT, 32, 4>(a, stream);
  if (a.T <= 512) return launch_tile<FP16, D, BIAS, COMMIT, 64, 2>(a, stream);
  return launch_tile<FP16, D, BIAS, COMMIT, 128, 2>(a, stream);
}

template <bool FP16, int D, bool BIAS>
hipError_t launch_commit(const WriteArgs& a, bool has_commit, hipStream_t stream) {
  return has_commit ? launch_by_rows<FP16, D, BIAS, true>(a, stream)
                    : launch_by_rows<FP16, D, BIAS, false>(a, stream);
}

template <bool FP16, int D>
hipError_t launch_bias(const WriteArgs& a, bool has_bias, bool has_commit, hipStream_t stream) {
  return has_bias ? launch_commit<FP16, D, true>(a, has_commit, stream)
                  : launch_commit<FP16, D, false>(a, has_commit, stream);
}

template <bool FP16>
hipError_t launch_dim(const WriteArgs& a, int head_dim, bool has_bias, bool has_commit,
                      hipStream_t stream) {
  if (head_dim == 128) return launch_bias<FP16, 128>(a, has_bias, has_commit, stream);
  if (head_dim == 64) return launch_bias<FP16, 64>(a, has_bias, has_commit, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_ctx_kv_write(const WriteArgs& a, int head_dim, bool is_fp16, bool has_bias,
                               bool has_commit, hipStream_t stream) {
  return is_fp16 ? launch_dim<true>(a, head_dim, has_bias, has_commit, stream)
                 : launch_dim<false>(a, head_dim, has_bias, has_commit, stream);
}

}  // namespace dspark
