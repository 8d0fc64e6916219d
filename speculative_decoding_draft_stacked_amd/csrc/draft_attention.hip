// DSpark draft attention over the KV pool for gfx950: bidirectional
// grouped-query attention of each request's block of queries over its prefix
// (gathered from a layer's pool through the request's slot list) and the
// block's own keys.
//
// Method: sglang PR #35499 ("K3 DSpark draft attention via verify_shared_kv on
// ROCm gfx95", implementation breakdown and key source snippets): a split-KV
// stage over the prefix, query head h reading KV head h // G, and a combine
// stage with the causal mask off for the draft. Here the block's own keys are
// one more split of the first stage, and the second stage only merges.
//
// Stage 1: one wave per (request, KV head, tile of 32 rows, key split), the
// heads of a record launched together on one XCD (see the record order). A row
// is a (block token j, query head g of the group) pair, row = j * G + g. For
// every 32 keys of the split:
//   - S^T = K * Q^T on v_mfma_f32_32x32x16: keys on M (each lane gathers its
//     key's row from the pool, 16 bytes per step, and its V row the same way),
//     rows on N (Q fragments stay in registers). Lane l then holds row l % 32 and 16 of the 32 keys, so
//     the online softmax (base-2, scores scaled by sm_scale * log2 e) is
//     lane-local apart from one swap with lane l ^ 32.
//   - O^T += V^T * P^T: the probabilities are the B operand straight from the
//     score registers (the k-slots of a lane are exactly the keys it holds),
//     and V^T comes from a transposed 32-key tile in LDS, read in the same key
//     order. O^T's lane column is again the lane's row, so rescaling is
//     lane-local.
//   The split leaves fp32 (O, m, l) per row in the workspace.
// Stage 2: per row, M = max m, L = sum l * 2^(m - M), O = sum O * 2^(m - M) / L,
// rounded once to the dtype; 4 or 8 threads per (row, 8 features), each
// merging a share of the splits. Keys past a request's prefix, and slots outside the
// pool (counted), are masked with a zero value row.
#include "internal.h"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
// LDS row of the V^T tile (elements): 72 bytes keeps 8-byte reads aligned, and
// 32 consecutive rows start in 32 distinct even banks (18 d mod 64).
constexpr int KS = 32 + 4;

template <bool FP16>
struct AE;

template <>
struct AE<false> {
  using vec8 = bf16x8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t from_f(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);  // round to nearest even
  }
};

template <>
struct AE<true> {
  using vec8 = f16x8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t from_f(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
  }
};

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
  const u32x4 v = *(global_u32x4*)p;
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <bool FP16, int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void draft_attn_stage1(const AttnArgs a) {
  using E = AE<FP16>;
  using vec8 = typename E::vec8;
  constexpr int DS = D / 16;          // MFMA steps over the head dimension
  constexpr int DB = D / 32;          // 32-wide blocks of O^T
  __shared__ __align__(16) uint16_t vt[D * KS];

  const int lane = threadIdx.x;
  const int r32 = lane & 31;
  const int hh = lane >> 5;
  // Record order: the KV heads of one (request, row tile, split) are launched
  // back to back on one XCD (workgroup w runs on XCD w % 8), so the pieces of
  // each gathered pool row, one per head, reach HBM together and mostly hit an
  // open DRAM row, rather than 256-byte reads scattered in time.
  int64_t wg = blockIdx.x;
  const int nsp = a.n_splits + 1;
  const int64_t nrec = a.B * a.row_tiles * nsp;  // records per KV head
  int kh;
  if (nrec % 8 == 0) {
    const int64_t q = wg / 8;
    kh = (int)(q % a.nhk);
    wg = (q / a.nhk) * 8 + wg % 8;
  } else {
    kh = (int)(wg % a.nhk);
    wg /= a.nhk;
  }
  const int split = (int)(wg % nsp);
  wg /= nsp;
  const int rtile = (int)(wg % a.row_tiles);
  const int64_t b = wg / a.row_tiles;

  // this lane's row (N index of S^T and O^T)
  const int row = rtile * 32 + r32;
  const bool row_ok = row < a.M;
  const int tj = row_ok ? row / a.G : 0;
  const int tg = row_ok ? row % a.G : 0;
  const int64_t qtok = b * a.block + tj;
  vec8 qf[DS];
  {
    const uint16_t* qrow = a.q + qtok * a.q_stride0 + (int64_t)(kh * a.G + tg) * a.q_stride1;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const uint4 u = row_ok ? ld16(qrow + 16 * s + 8 * hh) : make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(vec8, u);
    }
  }

  const bool ext = split == a.n_splits;  // the block's own keys
  const int64_t p0 = a.kv_indptr[b];
  const int64_t plen = a.kv_indptr[b + 1] - p0;
  const int64_t kbeg = ext ? 0 : (int64_t)split * a.split_len;
  int64_t kend = ext ? a.block : kbeg + a.split_len;
  // prefix keys past max_prefix are never attended (and counted below)
  if (!ext) kend = min(kend, min(plen, a.max_prefix));
  const uint16_t* kbase = ext ? a.k_ext : a.k_pool;
  const uint16_t* vbase = ext ? a.v_ext : a.v_pool;
  const bool counter = !ext && kh == 0 && rtile == 0 && a.err != nullptr;
  // a prefix longer than max_prefix is counted once per request
  if (ext && kh == 0 && rtile == 0 && a.err != nullptr && lane == 0 && plen > a.max_prefix)
    atomicAdd(a.err, 1ull);
  const float scale2 = a.sm_scale * kLog2e;

  float m = -INFINITY, lsum = 0.0f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;

  // Keys go in windows of 8 steps of 32: the window's slot indices are loaded
  // at once, and each step's K and V gathers are issued during the previous
  // step (see load_k / load_v below), so they overlap its math.
  constexpr int WSTEPS = 8;
  // K and V are gathered alike: lane (key r32, half h) takes features
  // 16s + 8h + [0, 8) of its key's row, which is the MFMA A layout for K and,
  // written to the transposed tile, puts 32 consecutive keys of one feature
  // row in one instruction (no bank conflicts between the 16-lane groups).
  // One register buffer each for K and V: the next step's K rows are
  // gathered as soon as this step's S MFMAs have read the current ones, and
  // its V rows once the current ones are in the LDS tile, so both stay one
  // step ahead with half the registers of a double buffer. With that the
  // kernel fits 256 registers, two waves per SIMD at head_dim 128, so the
  // block-key waves run alongside the prefix splits instead of after them.
  uint4 kf[DS], vu[DS];
  auto load_k = [&](int64_t krow) {
#pragma unroll
    for (int s = 0; s < DS; ++s) kf[s] = ld16(kbase + krow + 16 * s + 8 * hh);
  };
  auto load_v = [&](int64_t krow) {
#pragma unroll
    for (int s = 0; s < DS; ++s) vu[s] = ld16(vbase + krow + 16 * s + 8 * hh);
  };
  auto step = [&](unsigned long long vmask, bool more, int64_t knext) {
    // S^T = K * Q^T over the head dimension
    f32x16 st;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < DS; ++s) st = E::mfma(__builtin_bit_cast(vec8, kf[s]), qf[s], st);
    if (more) load_k(knext);  // uniform

    // V^T tile into LDS: vt[d][key], zero rows for masked keys
    const bool vok = (vmask >> r32) & 1ull;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const uint4 u = vok ? vu[s] : make_uint4(0, 0, 0, 0);
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
      uint16_t* col = vt + (16 * s + 8 * hh) * KS + r32;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        col[(2 * e) * KS] = (uint16_t)(w4[e] & 0xFFFFu);
        col[(2 * e + 1) * KS] = (uint16_t)(w4[e] >> 16);
      }
    }
    if (more) load_v(knext);

    // online softmax of this lane's row over the 32 keys (16 here, 16 in lane ^ 32)
    float sv[16];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 8 * (r / 4) + 4 * hh + (r % 4);
      sv[r] = ((vmask >> kr) & 1ull) ? st[r] * scale2 : -INFINITY;
      mx = fmaxf(mx, sv[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float alpha = mnew == -INFINITY ? 1.0f : exp2f(m - mnew);
    float ps = 0.0f;
    uint32_t pk[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float pa = sv[r] == -INFINITY ? 0.0f : exp2f(sv[r] - mnew);
      const float pb = sv[r + 1] == -INFINITY ? 0.0f : exp2f(sv[r + 1] - mnew);
      ps += pa + pb;
      pk[r / 2] = (uint32_t)E::from_f(pa) | ((uint32_t)E::from_f(pb) << 16);
    }
    ps += __shfl_xor(ps, 32);
    lsum = lsum * alpha + ps;
    m = mnew;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

    // O^T += V^T * P^T: k-step s takes this lane's score registers 8s .. 8s + 7,
    // i.e. keys 16s + 4h + [0, 4) and 16s + 8 + 4h + [0, 4)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const vec8 pf = __builtin_bit_cast(
          vec8, make_uint4(pk[4 * s], pk[4 * s + 1], pk[4 * s + 2], pk[4 * s + 3]));
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vr = vt + (db * 32 + r32) * KS + 16 * s + 4 * hh;
        const uint2 x0 = *reinterpret_cast<const uint2*>(vr);
        const uint2 x1 = *reinterpret_cast<const uint2*>(vr + 8);
        const vec8 af = __builtin_bit_cast(vec8, make_uint4(x0.x, x0.y, x1.x, x1.y));
        o[db] = E::mfma(af, pf, o[db]);
      }
    }
  };

  for (int64_t w0 = kbeg; w0 < kend; w0 += 32 * WSTEPS) {
    // this lane's key of every step in the window (M index of S^T): its row
    int64_t krow[WSTEPS];
    unsigned long long vmask[WSTEPS];
#pragma unroll
    for (int j = 0; j < WSTEPS; ++j) {
      const int64_t key = w0 + 32 * j + r32;
      bool kvalid = key < kend;
      if (ext) {
        krow[j] = (b * a.block + (kvalid ? key : 0)) * a.ext_stride0 +
                  (int64_t)kh * a.ext_stride1;
      } else {
        int64_t slot = kvalid ? a.kv_indices[p0 + key] : 0;
        if (slot < 0 || slot >= a.num_slots) {
          if (kvalid && counter && hh == 0) atomicAdd(a.err, 1ull);
          kvalid = false;
          slot = 0;
        }
        krow[j] = slot * a.pool_stride0 + (int64_t)kh * a.pool_stride1;
      }
      vmask[j] = __ballot(kvalid);
    }
    load_k(krow[0]);
    load_v(krow[0]);
#pragma unroll
    for (int j = 0; j < WSTEPS; ++j) {
      if (w0 + 32 * j < kend) {  // uniform over the wave
        const bool more = j + 1 < WSTEPS && w0 + 32 * (j + 1) < kend;
        step(vmask[j], more, more ? krow[j + 1] : 0);
      }
    }
  }

  // partial record: O [32 rows][D] fp32, then m [32], then l [32]
  float* rec = a.part + (((b * a.nhk + kh) * a.row_tiles + rtile) * nsp + split) *
                            (int64_t)(32 * (D + 2));
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(rec + r32 * D + db * 32 + 8 * q + 4 * hh) =
          make_float4(o[db][4 * q], o[db][4 * q + 1], o[db][4 * q + 2], o[db][4 * q + 3]);
  if (hh == 0) {
    rec[32 * D + r32] = m;
    rec[32 * D + 32 + r32] = lsum;
  }
}

// Stage 2: P threads per (row, 8 features) of a (request, KV head, row tile)
// record (P = 4 at head_dim 128, 8 at 64, where records have twice the
// splits), each merging every P-th split online (running max M, sum L and
// weighted O, rescaled as each split arrives, so its loads of all its splits
// are independent and go out together); the P partial merges are then
// combined by lane swaps in a fixed order. An empty split has m = -inf, l = 0
// and O = 0 and adds nothing. A workgroup takes 256 / (P * D / 8) rows of a
// record, so short records still spread over many workgroups.
template <int D>
constexpr int kMergeParts = D <= 64 ? 8 : 4;

template <bool FP16, int D>
__global__ __launch_bounds__(256) void draft_attn_stage2(const AttnArgs a) {
  using E = AE<FP16>;
  constexpr int FG = D / 8;                     // 8-feature groups of a row
  constexpr int P = kMergeParts<D>;
  constexpr int RPW = 256 / (P * FG);           // rows per workgroup
  constexpr int64_t REC = 32 * (D + 2);
  static_assert(32 % RPW == 0, "row groups tile the 32-row record");
  const int tid = threadIdx.x;
  const int part = tid % P;
  const int fg = (tid / P) % FG;
  int64_t wg = blockIdx.x;
  const int rgrp = (int)(wg % (32 / RPW));
  wg /= 32 / RPW;
  const int rtile = (int)(wg % a.row_tiles);
  wg /= a.row_tiles;
  const int kh = (int)(wg % a.nhk);
  const int64_t b = wg / a.nhk;
  const int nsp = a.n_splits + 1;
  const float* base = a.part + ((b * a.nhk + kh) * a.row_tiles + rtile) * nsp * REC;
  const int r32 = rgrp * RPW + tid / (P * FG);
  const int row = rtile * 32 + r32;
  float M = -INFINITY, L = 0.0f;
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
  for (int s = part; s < nsp; s += P) {
    const float* rec = base + s * REC;
    const float ms = rec[32 * D + r32];
    const float ls = rec[32 * D + 32 + r32];
    const float4 x0 = *reinterpret_cast<const float4*>(rec + r32 * D + fg * 8);
    const float4 x1 = *reinterpret_cast<const float4*>(rec + r32 * D + fg * 8 + 4);
    const float mn = fmaxf(M, ms);
    const float wa = M == -INFINITY ? 0.0f : exp2f(M - mn);   // rescale what is merged
    const float wb = ms == -INFINITY ? 0.0f : exp2f(ms - mn);  // weight of this split
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    L = L * wa + ls * wb;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * wa + xs[e] * wb;
    M = mn;
  }
  // combine the P partial merges (lanes part = 0..P-1 are adjacent)
#pragma unroll
  for (int mask = 1; mask < P; mask <<= 1) {
    const float Mo = __shfl_xor(M, mask);
    const float Lo = __shfl_xor(L, mask);
    const float mn = fmaxf(M, Mo);
    const float wa = M == -INFINITY ? 0.0f : exp2f(M - mn);
    const float wb = Mo == -INFINITY ? 0.0f : exp2f(Mo - mn);
    L = L * wa + Lo * wb;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * wa + __shfl_xor(acc[e], mask) * wb;
    M = mn;
  }
  if (part != 0 || row >= a.M) return;
  const float invL = 1.0f / L;
  const int tj = row / a.G, tg = row % a.G;
  uint16_t* out = a.out + (b * a.block + tj) * a.out_stride0 +
                  (int64_t)(kh * a.G + tg) * a.out_stride1 + fg * 8;
  uint32_t w4[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w4[e] = (uint32_t)E::from_f(acc[2 * e] * invL) |
            ((uint32_t)E::from_f(acc[2 * e + 1] * invL) << 16);
  *reinterpret_cast<uint4*>(out) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
}

template <bool FP16, int D>
hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  const int64_t g1 = (int64_t)a.B * a.nhk * a.row_tiles * (a.n_splits + 1);
  const int64_t g2 = (int64_t)a.B * a.nhk * a.row_tiles * (32 / (256 / (kMergeParts<D> * (D / 8))));
  if (g1 > 0x7FFFFFFF || g2 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((draft_attn_stage1<FP16, D>), dim3((uint32_t)g1), dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((draft_attn_stage2<FP16, D>), dim3((uint32_t)g2), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_draft_attention(const AttnArgs& a, int head_dim, bool is_fp16,
                                  hipStream_t stream) {
  if (a.B <= 0) return hipSuccess;
  if (head_dim == 128) return is_fp16 ? launch<true, 128>(a, stream) : launch<false, 128>(a, stream);
  if (head_dim == 64) return is_fp16 ? launch<true, 64>(a, stream) : launch<false, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dspark
