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
// in memory and no transpose is needed. Weight tiles are 128 rows, i.e. one
// head of 128 or two heads of 64, so a tile never straddles a head and the
// norm and the (d, d + D/2) rotation pairs are local to it. The weight comes
// from the pack in a blocked layout where each wave's MFMA A fragment for one
// 16-wide K step is one contiguous KiB. The regimes:
//   - ctx_kv_stream_kernel, small T: one 128-row tile x up to 128 tokens per
//     workgroup, the weight streamed from HBM into registers;
//   - the same kernel with K split over workgroups, when few weight tiles
//     would leave the device idle (e.g. one GPU's share of the KV heads): fp32
//     part sums to the caller's workspace, then ctx_kv_stream_reduce adds
//     them in part order and runs the epilogue;
//   - ctx_kv_tiled_kernel, large T: 256 rows x 128/192/256 tokens per
//     workgroup, both operands staged through an LDS ring by direct-to-LDS
//     loads.
// MFMA: v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation.
//
// Epilogue. Accumulators (+ bias) are rounded once to the dtype (the GEMM's
// output dtype) into an LDS tile [BT][rows]. Each (token, head) is then handled
// by D/16 lanes: every lane owns 8 elements of the first half and their 8
// rotation partners in the second half, so the rotation needs no exchange and
// the sum of squares needs log2(D/16) lane swaps. K is normalised in fp32
// (x * inv * w), rounded, rotated in fp32 and rounded; V is copied. Stores are
// 16-byte vectors into the pool row of the token's slot.
#include "internal.h"

#include <type_traits>

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BN = 128;       // weight rows per tile
constexpr int BK = 64;        // K slice per pipeline stage
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

// 16-byte nontemporal load of a streamed weight fragment: on a pure HBM
// stream this reaches about 9% more bandwidth than a default load. The
// pointer is cast to the global address space so that the compiler emits
// global_load (counted by vmcnt only) rather than flat_load, which would also
// hold up every LDS wait behind outstanding memory loads.
__device__ __forceinline__ uint4 ldg16_nt(const uint16_t* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
  const u32x4 v = __builtin_nontemporal_load((global_u32x4*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

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

// Epilogue shared by both kernels: from the dtype-rounded LDS tile [BT][LDO]
// (tokens x the tile's ROWS weight rows), normalise + rotate each K head, copy
// each V head, and scatter both into the token's slot of the head's layer pool.
// D/16 lanes handle a (token, head), lane j owning elements [8j, 8j+8) of the
// first half and their rotation partners 8j + D/2 + [0, 8). The tile's heads
// are split into HS groups, HS as small as keeps every thread busy: a thread
// walks tokens TSTEP apart, each over the heads of its group, so where tokens
// are plentiful (the tiled kernel) a token's slot, position and table row are
// loaded once for all of its heads. Every global load a thread needs is issued
// before its first pool store: vmcnt counts loads and stores in issue order,
// so a load issued after a store could not be waited for without also waiting
// for that store to complete.
// With a row map (rmap != nullptr), tile token tt is row rmap[tt] (< 0: none).
template <typename E, int D, int BT, bool COMMIT, int LDO, int NT = NTHREADS, int ROWS = BN>
__device__ __forceinline__ void scatter_tile(const WriteArgs& a, const uint16_t* sO, int64_t n0,
                                             int64_t t0, int tid, const int* rmap = nullptr) {
  constexpr int TPH = D / 16;    // lanes per (token, head)
  constexpr int HPT = ROWS / D;  // heads per tile
  constexpr int HS_FILL = (NT + BT * TPH - 1) / (BT * TPH);
  constexpr int HS = HPT < HS_FILL ? HPT : HS_FILL;  // head groups
  constexpr int HPG = HPT / HS;                      // heads per group
  static_assert(HPT % HS == 0 && NT % 64 == 0 && (NT / TPH) % HS == 0,
                "a thread keeps one lane slot and head group");
  constexpr int TASK_LANES = BT * HS * TPH;
  constexpr int ITERS = (TASK_LANES + NT - 1) / NT;
  constexpr int TSTEP = NT / TPH / HS;  // tile tokens between a thread's iterations
  const int j = tid % TPH;
  const int hs = (tid / TPH) % HS;
  const int tt0 = tid / TPH / HS;
  const int two_nh = 2 * a.NH;
  const int64_t T = a.T;

  // the group's heads: pool, row stride and size of the head's layer, read
  // once (a kernel-argument array with a run-time index is read by a vector
  // load, which must not follow a store)
  bool live[HPG], is_k[HPG], counts[HPG];
  uint16_t* pool[HPG];
  int64_t rstride[HPG], nslots[HPG];
  int hlayer[HPG];
  bool any_k = false;
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    const int64_t g = (n0 + (hs * HPG + h) * D) / D;  // global head: layer-major, K then V
    live[h] = g < (int64_t)a.L * two_nh;  // false: rows past the stacked weight (last tile)
    const int layer = live[h] ? (int)(g / two_nh) : 0;
    const int jj = (int)(g % two_nh);
    is_k[h] = live[h] && jj < a.NH;
    counts[h] = live[h] && jj == 0;  // the layer's first K head counts range errors
    any_k = any_k || is_k[h];
    hlayer[h] = layer;
    const int n = jj < a.NH ? jj : jj - a.NH;
    pool[h] = (is_k[h] ? a.pk[layer] : a.pv[layer]) + n * D + j * 8;
    rstride[h] = is_k[h] ? a.ks0[layer] : a.vs0[layer];
    nslots[h] = a.slots[layer];
  }

  // indices of every token this thread stores
  int64_t loc[ITERS], pos[ITERS];
  int tts[ITERS];
#pragma unroll
  for (int k = 0; k < ITERS; ++k) {
    const int tt = tt0 + k * TSTEP;
    tts[k] = tt;
    loc[k] = -1;
    pos[k] = 0;
    if (tid + k * NT >= TASK_LANES) continue;  // ragged last pass (uniform per lane group)
    const int64_t t = rmap ? (int64_t)rmap[tt] : t0 + tt;
    if (t < 0 || t >= T) continue;
    int64_t l = a.locs[t];
    if (COMMIT && (t % a.W) >= a.commit[t / a.W]) l = -1;
    loc[k] = l;
    pos[k] = a.pos[t];
  }
  bool pos_ok[ITERS];
#pragma unroll
  for (int k = 0; k < ITERS; ++k) pos_ok[k] = loc[k] >= 0 && pos[k] >= 0 && pos[k] < a.P;

  // K heads: norm weights of their layers and the tokens' table rows (row 0
  // for tokens not stored: always inside the table)
  float gw1[HPG][8], gw2[HPG][8];
  float cc[ITERS][8], ss[ITERS][8];
  if (any_k) {
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      const float* gwp = a.knw + (int64_t)hlayer[h] * D + j * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        gw1[h][i] = gwp[i];
        gw2[h][i] = gwp[i + D / 2];
      }
    }
#pragma unroll
    for (int k = 0; k < ITERS; ++k) {
      const float* cs = a.table + (pos_ok[k] ? pos[k] : 0) * D + j * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        cc[k][i] = cs[i];
        ss[k][i] = cs[i + D / 2];
      }
    }
  }

#pragma unroll
  for (int k = 0; k < ITERS; ++k) {
    if (loc[k] < 0) continue;  // not stored (uniform over the TPH lanes of a token)
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      if (!live[h]) continue;
      if (!pos_ok[k] || loc[k] >= nslots[h]) {
        if (counts[h] && j == 0 && a.err) atomicAdd(a.err, 1ull);  // once per (row, layer)
        continue;
      }
      const uint16_t* src = sO + tts[k] * LDO + (hs * HPG + h) * D + j * 8;
      const uint4 u1 = *reinterpret_cast<const uint4*>(src);
      const uint4 u2 = *reinterpret_cast<const uint4*>(src + D / 2);
      uint16_t* dst = pool[h] + loc[k] * rstride[h];
      if (is_k[h]) {
        float x1[8], x2[8];
        unpack8<E>(u1, x1);
        unpack8<E>(u2, x2);
        float sq = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) sq += x1[i] * x1[i] + x2[i] * x2[i];
#pragma unroll
        for (int m = 1; m < TPH; m <<= 1) sq += __shfl_xor(sq, m);
        const float inv = 1.0f / sqrtf(sq / (float)D + a.eps);
        float o1[8], o2[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float n1 = E::to_f(E::from_f(x1[i] * inv * gw1[h][i]));
          const float n2 = E::to_f(E::from_f(x2[i] * inv * gw2[h][i]));
          o1[i] = n1 * cc[k][i] - n2 * ss[k][i];
          o2[i] = n2 * cc[k][i] + n1 * ss[k][i];
        }
        *reinterpret_cast<uint4*>(dst) = pack8<E>(o1);
        *reinterpret_cast<uint4*>(dst + D / 2) = pack8<E>(o2);
      } else {
        *reinterpret_cast<uint4*>(dst) = u1;
        *reinterpret_cast<uint4*>(dst + D / 2) = u2;
      }
    }
  }
}

// Head dimension value that selects the context producer's epilogue instead
// of the K/V scatter: the tile's rows are plain output features.
constexpr int kRowsOut = 0;

// Producer epilogue: from the dtype-rounded LDS tile [BT][LDO] (tokens x ROWS
// output features), store each token's features to its output row and write
// the sum of squares of every 128-feature group (in fp32, of the rounded
// values) to partial[group * T + token] for the row norm that follows. 16
// lanes per (token, group), 8 features each.
template <typename E, int BT, int LDO, int NT, int ROWS>
__device__ __forceinline__ void rows_out_tile(const WriteArgs& a, const uint16_t* sO, int64_t n0,
                                              int64_t t0, int tid) {
  constexpr int GROUPS = ROWS / BN;
  constexpr int LPG = BN / 8;
  constexpr int TASK_LANES = BT * GROUPS * LPG;
  static_assert(NT % 64 == 0 && TASK_LANES % LPG == 0, "lane groups stay inside a wave");
#pragma unroll 1
  for (int idx = tid; idx < TASK_LANES; idx += NT) {
    const int task = idx / LPG;
    const int j = idx % LPG;
    const int tt = task / GROUPS;
    const int g = task % GROUPS;
    const int64_t t = t0 + tt;
    const int64_t rt = n0 / BN + g;
    if (t >= a.T || rt >= a.R) continue;  // uniform over the LPG lanes of a task
    const uint4 u = *reinterpret_cast<const uint4*>(sO + tt * LDO + g * BN + j * 8);
    float f[8];
    unpack8<E>(u, f);
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += f[i] * f[i];
#pragma unroll
    for (int m = 1; m < LPG; m <<= 1) ss += __shfl_xor(ss, m);
    *reinterpret_cast<uint4*>(a.y + t * a.y_stride + rt * BN + j * 8) = u;
    if (j == 0) a.partial[rt * a.T + t] = ss;
  }
}

// 16-byte direct-to-LDS load (gfx950 global_load_lds_dwordx4): lane i of the
// wave writes its 16 bytes to lds_wave_base + 16 * i; lds_wave_base must be
// the same for the whole wave.
__device__ __forceinline__ void ldg16_to_lds(const uint16_t* src, uint16_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)lds_wave_base, 16, 0,
                                   0);
}

// Plain workgroup barrier. The caller has already waited (vmcnt) for its own
// direct-to-LDS loads; a fence here would wait for all of them, including the
// prefetches that must stay in flight. The memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void raw_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt vmcnt(N) lgkmcnt(0): before a ring barrier, this wave's loads of
// the next stage have landed and its own LDS reads of the stage about to be
// refilled have completed (the compiler may issue them late, right before the
// barrier), so no direct-to-LDS write issued after the barrier can overtake one.
template <int N>
__device__ __forceinline__ void wait_ring() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

// LDS-tiled kernel for large T. A workgroup owns a 256-row x BT-token tile
// (two 128-row weight tiles; the second may lie past the stacked weight when
// the number of 128-row tiles is odd). Eight waves, two per SIMD, form a 4 x 2
// grid of 64-row x (BT/2)-token wave tiles (2 x BT/64 MFMA blocks each).
// Operands reach the LDS by direct-to-LDS loads, every load instruction of a
// wave fetching eight whole 128-byte lines:
//   - weight: a ring of four 32-wide K sub-chunks (16 KiB each), issued three
//     sub-chunks ahead; the blocked layout holds, per 64-column chunk, each
//     32-row group's A fragment for one MFMA step as one contiguous KiB, and a
//     sub-chunk copies the two steps it needs linearly;
//   - X: a ring of two 64-wide K chunks (BT x 128 bytes each), issued two
//     sub-chunks ahead: one token's 64 columns are one line, fetched by eight
//     consecutive lanes whose 16-byte pieces land at slot s of the token's LDS
//     row, holding piece s ^ ((t / 2) % 8). A B fragment read (16 lanes, 16
//     consecutive tokens, one piece) then covers all 64 banks once.
// The fragments of an MFMA step are read while the MFMAs of the previous step
// run (software pipeline, one barrier per sub-chunk between the two steps).
// Wait counts per sub-chunk (loads complete in issue order): with the issue
// order X(j), W(2j+1) at sub-chunk 2j - 2 and W(2j+2) at 2j - 1, an even
// sub-chunk finds its X chunk behind at most two weight sub-chunks' loads and
// an odd one its weight sub-chunk behind one X chunk and two weight
// sub-chunks.
template <bool FP16, int D, bool BIAS, bool COMMIT, int BT>
__global__ __launch_bounds__(512) void ctx_kv_tiled_kernel(const WriteArgs a, int t_tiles) {
  using E = Elem<FP16>;
  using vec8 = typename E::vec8;
  constexpr int NT = 512;
  constexpr int ROWS = 2 * BN;              // 256 weight rows per workgroup
  constexpr int MB = 2;                     // 32-row blocks per wave
  constexpr int NB = BT / 64;               // 32-token blocks per wave
  static_assert(BT % 64 == 0 && BT <= 256, "token tile");
  constexpr int SK = 32;                    // weight K per sub-chunk
  constexpr int WSTAGES = 4;
  constexpr int WLOOK = WSTAGES - 1;        // weight sub-chunks in flight ahead
  constexpr int SW = ROWS * SK;             // weight elements per stage
  constexpr int SX = BT * BK;               // X elements per stage (one 64-wide chunk)
  constexpr int W_PER_THREAD = SW / 8 / NT;   // 2 direct loads per sub-chunk
  constexpr int X_PER_THREAD = SX / 8 / NT;   // BT / 64 direct loads per chunk
  static_assert(SX == X_PER_THREAD * NT * 8, "X chunk split");
  constexpr int XOFF = WSTAGES * SW;          // X ring after the weight ring
  constexpr int RING = XOFF + 2 * SX;
  constexpr int LDO = ROWS + 4;
  constexpr int SMEM = (RING > BT * LDO ? RING : BT * LDO);
  // + the tile's bias rows, past both the ring and the output tile
  __shared__ __align__(16) uint16_t smem[SMEM + (BIAS ? ROWS : 0)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_n = wave >> 1;  // 64-row group
  const int wave_t = wave & 1;   // token half
  const int r32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t T = a.T;
  const int H = a.H;
  const int nk = (H + BK - 1) / BK;

  // Tile order: groups of 4 row pairs x all token tiles, walked row-fastest,
  // and each XCD (workgroup b runs on XCD b % 8) takes a contiguous run of
  // that order, so the workgroups resident on one XCD share weight and token
  // tiles through its L2.
  const int64_t R = a.R;  // 128-row weight tiles
  const int64_t RP = (R + 1) / 2;                       // 256-row tiles
  const int64_t ntiles = RP * t_tiles;
  const int64_t b = blockIdx.x;
  const int64_t j = ntiles % 8 == 0 ? (b % 8) * (ntiles / 8) + b / 8 : b;
  constexpr int64_t G = 4;
  const int64_t gsz = G * t_tiles;
  const int64_t g0 = (j / gsz) * G;
  const int64_t rows_in_group = RP - g0 < G ? RP - g0 : G;
  const int64_t jr = j % gsz;
  const int64_t rp = g0 + jr % rows_in_group;
  const int64_t tt = jr / rows_in_group;
  const int64_t n0 = rp * ROWS;
  const int64_t t0 = tt * BT;

  // Per-lane source offsets: weight stage piece q = i * NT + tid is (block i,
  // group tid / 128, step (tid / 64) % 2, lane tid % 64); X slot i * NT + tid
  // is token i * 64 + tid / 8, LDS piece tid % 8 holding global piece
  // (tid % 8) ^ ((tid / 16) % 8) (the same column offset for every i).
  const int wl = ((tid / 128) * 4 + (tid % 128) / 64) * 512 + (tid % 64) * 8;
  const int xt = tid / 8;
  const int xcol = 8 * ((tid & 7) ^ ((xt >> 1) & 7));
  // weight sub-chunk u (half u % 2 of 64-column chunk u / 2) into stage u % 4;
  // the second half takes MFMA steps 2 and 3
  auto issue_w = [&](int u) {
    uint16_t* base = smem + (u % WSTAGES) * SW;
    const int c = u >> 1, h = u & 1;
    const bool live = c < nk;  // sub-chunks past the end read the zero page
#pragma unroll
    for (int i = 0; i < W_PER_THREAD; ++i) {
      const int64_t rt = 2 * rp + i;
      const uint16_t* src =
          live && rt < R ? a.w + (rt * nk + c) * 8192 + h * 1024 + wl : a.zeros;
      ldg16_to_lds(src, base + (i * NT + wave * 64) * 8);
    }
  };
  // X chunk c (64 columns of every token of the tile) into stage c % 2
  auto issue_x = [&](int c) {
    uint16_t* base = smem + XOFF + (c & 1) * SX;
    const int k = c * BK + xcol;
    const bool live = c < nk && k < H;
#pragma unroll
    for (int i = 0; i < X_PER_THREAD; ++i) {
      const int64_t t = t0 + i * 64 + xt;
      const int64_t tok = t < T ? t : T - 1;  // rows past T are never stored
      const uint16_t* src = live ? a.x + tok * a.x_stride + k : a.zeros;
      ldg16_to_lds(src, base + (i * NT + wave * 64) * 8);
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  // Software pipeline over MFMA steps: the fragments of a step are read
  // from the LDS while the MFMAs of the previous step run, so no MFMA waits
  // on a fragment read issued right before it. Per sub-chunk u:
  //   read step-1 fragments of u | 8 MFMAs on the step-0 fragments of u
  //   issue the loads of weight sub-chunk u + 3 (into the stage of u - 1)
  //     and, for even u, of X chunk u / 2 + 1 (into that of chunk u / 2 - 1)
  //   wait for the loads of u + 1, barrier
  //   read step-0 fragments of u + 1 | 8 MFMAs on the step-1 fragments of u
  // The loads go out behind the wave's MFMAs, so a wave held up issuing them
  // holds up none of its own MFMAs (with the loads placed between the
  // fragment reads and the MFMAs, prefill took 715 us instead of 588 us;
  // right after the barrier, 588 us; here, 584 us). A step's fragment reads
  // are interleaved one per MFMA with the previous step's MFMAs, and the
  // load addresses are formed from the tile's scalars at each issue rather
  // than kept in per-lane arrays (230-238 VGPRs instead of 248: 573 against
  // 580 us on prefill; placing all six reads ahead of the MFMAs instead
  // needs 256 VGPRs and took 608 us). Whole turns of four
  // sub-chunks (two X chunks) with no branches (sub-chunks past the end read
  // the zero page), so stage indices are compile-time constants and every
  // wait count is exact.
  auto read_a = [&](int stage, int sp, vec8(&fa)[MB]) {
    const uint16_t* ws = smem + stage * SW;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = wave_n * 64 + mb * 32;  // first row of the 32-row block
      const int blk = r / BN;               // which of the two weight blocks
      const int grp = (r % BN) / 32;        // 32-row group inside the block
      fa[mb] = *reinterpret_cast<const vec8*>(ws + blk * (BN * SK) +
                                              ((grp * 2 + sp) * 64 + lane) * 8);
    }
  };
  auto read_b = [&](int u, int sp, vec8(&fb)[NB]) {
    const uint16_t* xs = smem + XOFF + ((u >> 1) & 1) * SX;
    const int h = u & 1;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int t = wave_t * (BT / 2) + nb * 32 + r32;
      // MFMA step s = 2h + sp, lane half hh: columns 32 hh + 8 s + [0, 8)
      // (the weight's blocked layout pairs the same columns)
      const int piece = 4 * hh + 2 * h + sp;
      const int slot = piece ^ ((t >> 1) & 7);
      fb[nb] = *reinterpret_cast<const vec8*>(xs + (t * 8 + slot) * 8);
    }
  };
  auto mfmas = [&](const vec8(&fa)[MB], const vec8(&fb)[NB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = E::mfma(fa[mb], fb[nb], acc[mb][nb]);
  };
  const int nsub = 2 * nk;
  const int nsub_ring = (nsub + WSTAGES - 1) / WSTAGES * WSTAGES;
  vec8 a0[MB], b0[NB], a1[MB], b1[NB];
  // the tile's bias rows, loaded once by 32 threads and kept in registers
  // until the epilogue (a load older than every ring load: the ring's first
  // wait covers it)
  const int64_t n_tot = R * BN;
  uint4 bias8 = make_uint4(0, 0, 0, 0);
  if (BIAS && tid < ROWS / 8 && n0 + tid * 8 < n_tot)
    bias8 = *reinterpret_cast<const uint4*>(a.bias + n0 + tid * 8);
  issue_x(0);
#pragma unroll
  for (int u = 0; u < WLOOK; ++u) issue_w(u);
  wait_ring<2 * W_PER_THREAD>();  // X chunk 0 and weight sub-chunk 0
  raw_barrier();
  read_a(0, 0, a0);
  read_b(0, 0, b0);
  for (int c0 = 0; c0 < nsub_ring; c0 += WSTAGES) {
#pragma unroll
    for (int uu = 0; uu < WSTAGES; ++uu) {
      const int u = c0 + uu;
      __builtin_amdgcn_sched_barrier(0);
      read_a(uu, 1, a1);
      read_b(uu, 1, b1);
      mfmas(a0, b0);
#pragma unroll
      for (int g = 0; g < MB + NB; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, MB * NB - (MB + NB), 0);
      __builtin_amdgcn_sched_barrier(0);
      // the stages of sub-chunk u - 1 (X: chunk u / 2 - 1) were freed by the
      // previous barrier
      if (uu % 2 == 0) issue_x((u >> 1) + 1);
      issue_w(u + WLOOK);
      __builtin_amdgcn_sched_barrier(0);
      // the loads of sub-chunk u + 1 landed (odd: its X chunk, behind at
      // most two weight sub-chunks; even: its weight sub-chunk, behind one X
      // chunk and two weight sub-chunks), this wave's reads of u are done
      if ((uu + 1) % 2 == 0)
        wait_ring<2 * W_PER_THREAD>();
      else
        wait_ring<2 * W_PER_THREAD + X_PER_THREAD>();
      raw_barrier();  // ... everyone's: the stages of sub-chunk u are free
      read_a((uu + 1) % WSTAGES, 0, a0);
      read_b(u + 1, 0, b0);
      mfmas(a1, b1);
#pragma unroll
      for (int g = 0; g < MB + NB; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, MB * NB - (MB + NB), 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  wait_ring<0>();  // the prefetches past the end (zero page) are done, LDS reads too
  uint16_t* const sbias = smem + SMEM;
  if (BIAS && tid < ROWS / 8) *reinterpret_cast<uint4*>(sbias + tid * 8) = bias8;
  raw_barrier();

  // accumulators (+ bias) -> dtype, into the LDS tile [BT][LDO]
  uint16_t* sO = smem;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int tok = wave_t * (BT / 2) + nb * 32 + r32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = wave_n * 64 + mb * 32 + 8 * q + 4 * hh;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = acc[mb][nb][4 * q + i];
          if (BIAS) v[i] += E::to_f(sbias[row + i]);  // zero past the stacked weight
        }
        uint2 packed;
        packed.x = E::from_f(v[0]) | (E::from_f(v[1]) << 16);
        packed.y = E::from_f(v[2]) | (E::from_f(v[3]) << 16);
        *reinterpret_cast<uint2*>(sO + tok * LDO + row) = packed;
      }
    }
  }
  __syncthreads();
  if constexpr (D == kRowsOut)
    rows_out_tile<E, BT, LDO, NT, ROWS>(a, sO, n0, t0, tid);
  else
    scatter_tile<E, D, BT, COMMIT, LDO, NT, ROWS>(a, sO, n0, t0, tid);
}

// Row compaction for commit windows. Only rows that are written (slot >= 0
// and inside the request's committed prefix) need projecting, so the rows of
// a commit window are first numbered in row order over the valid ones, and
// valid row j goes to token split j % splits, tile slot j / splits: the splits
// share the valid rows evenly without the host knowing their count. Every
// workgroup runs the same scan (T is small on this path). map[slot] = row, or
// -1 where the slot holds none; returns this split's number of rows. The scan
// costs every workgroup a pass per 512 rows, so longer windows (up to 32768
// rows reach this kernel when there are few weight tiles) keep contiguous
// splits instead.
template <int BT>
__device__ int compact_rows(const WriteArgs& a, int64_t sp, int splits, int* map, int* wcnt,
                            int tid) {
  constexpr int NT = 512;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < BT; i += NT) map[i] = -1;
  int base = 0;
  for (int64_t c = 0; c < a.T; c += NT) {
    const int64_t t = c + tid;
    bool v = false;
    if (t < a.T) {
      const int64_t loc = a.locs[t];
      const int64_t committed = a.commit[t / a.W];
      v = (loc >= 0) & ((t % a.W) < committed);
    }
    const unsigned long long m = __ballot(v);
    if (lane == 0) wcnt[wave] = __popcll(m);
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      const int n = wcnt[i];
      pre += i < wave ? n : 0;
      tot += n;
    }
    if (v) {
      const int j = base + pre + __popcll(m & ((1ull << lane) - 1ull));
      if (j % splits == sp && j / splits < BT) map[j / splits] = (int)t;
    }
    base += tot;
    __syncthreads();
  }
  return base > sp ? (int)((base - sp + splits - 1) / splits) : 0;
}

// Row compaction of the adaptive K-split plan (windows of at most 2 * NT
// rows): the valid rows are counted first. When they fit the `splits` token
// splits (BT slots each), valid row j goes to split j % splits as above and
// the K parts stay (this workgroup serves split sp_split); otherwise K is
// kept whole and the splits x ks workgroups of a row tile become as many
// token splits, row j going to split j % (splits * ks) (this workgroup then
// serves split sp_whole). A negative split serves no rows. *whole tells which
// mode; returns this workgroup's row count.
template <int BT>
__device__ int compact_rows_adaptive(const WriteArgs& a, int sp_split, int sp_whole, int splits,
                                     int ks, int* map, int* wcnt, int tid, bool* whole) {
  constexpr int NT = 512;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < BT; i += NT) map[i] = -1;
  bool v[2];
  unsigned long long mask[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int64_t t = (int64_t)c * NT + tid;
    v[c] = false;
    if (t < a.T) {
      const int64_t loc = a.locs[t];
      const int64_t committed = a.commit[t / a.W];
      v[c] = (loc >= 0) & ((t % a.W) < committed);
    }
    mask[c] = __ballot(v[c]);
    if (lane == 0) wcnt[c * (NT / 64) + wave] = __popcll(mask[c]);
  }
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int i = 0; i < 2 * (NT / 64); ++i) total += wcnt[i];
  const bool kwhole = total > splits * BT;
  const int m = kwhole ? splits * ks : splits;
  const int me = kwhole ? sp_whole : sp_split;
  int base = 0;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    int pre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      const int n = wcnt[c * (NT / 64) + i];
      pre += i < wave ? n : 0;
      tot += n;
    }
    if (v[c]) {
      const int j = base + pre + __popcll(mask[c] & ((1ull << lane) - 1ull));
      if (j % m == me && j / m < BT) map[j / m] = c * NT + tid;
    }
    base += tot;
  }
  __syncthreads();
  *whole = kwhole;
  return me >= 0 && base > me ? (base - me + m - 1) / m : 0;
}

// Weight-streaming kernel for small T (decode-sized batches). A workgroup
// owns one 128-row tile of the stacked weight and BT = 32*NB tokens; the host
// picks the number of token splits so that the whole grid is one round of
// workgroups. Eight waves, two per SIMD: wave (w, par) owns weight rows
// [32w, 32w+32) of the tile and the K chunks of parity par (K is split
// inside the workgroup; the two halves are added through LDS at the end), so
// each SIMD interleaves two instruction streams. ADAPT (compacted windows,
// K split): the workgroups keep K whole when the window's written rows do not
// fit the K-split plan's token splits (compact_rows_adaptive).
//   - Weight: streamed from HBM straight into a per-wave register ring (the
//     blocked layout gives each MFMA A fragment as one contiguous KiB), with
//     nontemporal loads.
//   - X: direct-to-LDS loads into an 8-stage ring, rows XOR-swizzled for
//     conflict-free 16-lane B fragment reads; no register staging.
//   - Chunks are consumed in groups of two (one per parity) with one barrier
//     per group; loads run LOOK groups ahead, so each wait covers only the
//     group about to be used.
//   - Commit windows: the workgroup's tokens are its share of the written rows
//     (compact_rows); 32-token blocks past that share skip their MFMAs, and
//     tile slots without a row load from the zero page.
template <bool FP16, int D, bool BIAS, bool COMMIT, int NB, bool ADAPT = false>
__global__ __launch_bounds__(512) void ctx_kv_stream_kernel(const WriteArgs a, int splits) {
  using E = Elem<FP16>;
  using vec8 = typename E::vec8;
  constexpr int NT = 512;
  constexpr int BT = 32 * NB;
  constexpr int LOOK = 3;             // groups issued ahead of the one being computed
  static_assert(LOOK == 3, "the commit-window prologue waits below assume three groups ahead");
  constexpr int SLOTS = LOOK + 1;     // per-wave weight ring slots (one chunk per group)
  constexpr int XSTAGES = 2 * SLOTS;  // X stages (one chunk each)
  constexpr int SXE = BT * BK;        // X stage elements
  constexpr int XPW = SXE / 8 / 256;  // X direct loads per thread per chunk (= NB)
  constexpr int LOADS = 4 + XPW;      // per thread per group
  constexpr int LDO = BN + 4;         // rounded output tile row (elements)
  constexpr int RS = BN + 4;          // fp32 partial row (floats): 528 bytes, conflict-free
  constexpr int XBYTES = XSTAGES * SXE * 2;
  constexpr int EBYTES = BT * RS * 4 + BT * LDO * 2;
  static_assert(XPW * 256 * 8 == SXE, "X chunk split");
  static_assert(!ADAPT || (COMMIT && D != kRowsOut), "adaptive K split: compacted writes");
  constexpr int MBYTES = COMMIT ? (BT + (ADAPT ? 2 : 1) * NT / 64) * 4 : 0;  // row map + counts
  __shared__ __align__(16) uint16_t smem[((XBYTES > EBYTES ? XBYTES : EBYTES) + MBYTES) / 2];
  int* const rmap = reinterpret_cast<int*>(smem + (XBYTES > EBYTES ? XBYTES : EBYTES) / 2);
  int* const wcnt = rmap + BT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int w = wave & 3;     // 32-row group
  const int par = wave >> 2;  // K-chunk parity
  const int r32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t T = a.T;
  const int H = a.H;
  const int64_t R = a.R;
  // Workgroup b runs on XCD b % 8. When the row tiles divide evenly, the
  // `splits` workgroups sharing a weight tile are placed on one XCD and
  // dispatched back to back, so its L2 serves the tile to all of them.
  // K may also be split over workgroups (a.ksplits > 1): workgroup b takes K
  // part b / (R * splits) and writes fp32 partial sums instead of the
  // epilogue; the producer's row-norm kernel, or ctx_kv_stream_reduce for the
  // write, adds the parts.
  int ks = a.ksplits > 1 ? a.ksplits : 1;
  int64_t kq = (int64_t)blockIdx.x / (R * splits);
  const int64_t b = (int64_t)blockIdx.x % (R * splits);
  int64_t rt, sp;
  if (D != kRowsOut && ks > 1) {
    // the write's K parts: the token splits of one (row tile, K part) slice
    // are 8 workgroups apart, i.e. on one XCD, whose L2 then fetches the
    // weight slice once for all of them; the grid is padded to whole groups
    // of 8 slices
    if constexpr (!ADAPT) {
      const int64_t slice = ((int64_t)blockIdx.x / (8 * splits)) * 8 + blockIdx.x % 8;
      if (slice >= R * ks) return;  // padding
      sp = ((int64_t)blockIdx.x / 8) % splits;
      rt = slice / ks;
      kq = slice % ks;
    } else {  // padding takes part in the scan (it may serve rows with K whole)
      const int64_t slice = ((int64_t)blockIdx.x / (8 * splits)) * 8 + blockIdx.x % 8;
      const bool pad = slice >= R * ks;
      sp = pad ? -1 : ((int64_t)blockIdx.x / 8) % splits;
      rt = pad ? 0 : slice / ks;
      kq = pad ? 0 : slice % ks;
    }
  } else if (R % 8 == 0) {
    const int64_t i = b / 8;
    rt = 8 * (i / splits) + b % 8;
    sp = i % splits;
  } else {
    rt = b / splits;
    sp = b % splits;
  }
  int64_t n0 = rt * BN;
  const int64_t t0 = sp * BT;
  const int nk_all = (H + BK - 1) / BK;
  int kc0 = (int)(kq * nk_all / ks);         // this part's chunks [kc0, kc1)
  int nk = (int)((kq + 1) * nk_all / ks) - kc0;
  int ng = (nk + 1) / 2;
  int ng_ring = (ng + SLOTS - 1) / SLOTS * SLOTS;
  // this wave's pieces of weight block (rt, c): one contiguous KiB per MFMA step
  const uint16_t* wblk = a.w + (rt * nk_all + kc0) * 8192 + (w * 4 * 64 + lane) * 8;
  // X direct loads: instruction i of wave (w, par) fills LDS slots
  // [256 i + 64 w, +64) of its chunk's stage; slot s holds piece
  // (s % 8) ^ ((t / 2) % 8) of token t = s / 8. Per-lane source offsets are
  // the same for every chunk.
  int64_t xoff[XPW];
  int xcol[XPW];
  bool xrow[XPW];  // the slot holds a row (else it loads zeros)

  uint4 wq[SLOTS][4];
  auto issue_w = [&](int g, uint4(&wd)[4]) {
    const int c = 2 * g + par;  // chunk of this part (the stage follows it)
    const bool live = c < nk;   // chunks past the end read the zero page
    const uint16_t* wsrc = live ? wblk + (int64_t)c * 8192 : a.zeros;
    const int wstep = live ? 512 : 0;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) wd[kk] = ldg16_nt(wsrc + kk * wstep);
  };
  auto issue_x = [&](int g) {
    const int c = 2 * g + par;
    const bool live = c < nk;
    uint16_t* stage = smem + ((c % XSTAGES) * SXE);
    const int kbase = (kc0 + c) * BK;
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
      const bool ok = live && xrow[i] && kbase + xcol[i] < H;
      ldg16_to_lds(ok ? a.x + xoff[i] + kbase : a.zeros, stage + (i * 256 + w * 64) * 8);
    }
  };

  // Commit windows: the weight loads of the first LOOK groups go out before
  // the row scan, whose latency they then cover; the X loads follow it.
  int nbe = NB;  // 32-token blocks that hold rows
  if constexpr (COMMIT) {
#pragma unroll
    for (int g = 0; g < LOOK; ++g) issue_w(g, wq[g]);
    int mine;
    if (ADAPT && T <= kCompactMaxRows) {
      // K whole: the R * splits * ks workgroups take the row tiles and token
      // splits the plain streaming plan would give them (a tile's splits on
      // one XCD); the others, and the padding, serve no rows
      const int sw = splits * ks;
      const int64_t bw = blockIdx.x;
      const bool in_whole = bw < R * sw;
      const int64_t rt_w = !in_whole ? 0 : R % 8 == 0 ? 8 * ((bw / 8) / sw) + bw % 8 : bw / sw;
      const int sp_w = !in_whole ? -1 : (int)(R % 8 == 0 ? (bw / 8) % sw : bw % sw);
      bool whole;
      mine = compact_rows_adaptive<BT>(a, (int)sp, sp_w, splits, ks, rmap, wcnt, tid, &whole);
      if (whole) {  // no part sums: the reduce launch finds no rows
        if (blockIdx.x == 0)
          for (int i = tid; i < splits * BT; i += NT) a.rowmap[i] = -1;
        ks = 1;
        kq = 0;
        rt = rt_w;
        sp = sp_w;
        n0 = rt * BN;
        kc0 = 0;
        nk = nk_all;
        ng = (nk + 1) / 2;
        ng_ring = (ng + SLOTS - 1) / SLOTS * SLOTS;
        wblk = a.w + rt * nk_all * 8192 + (w * 4 * 64 + lane) * 8;
        if (mine > 0) {  // this tile's K from the start (the scan's loads, issued
                         // after the ones above, have completed)
#pragma unroll
          for (int g = 0; g < LOOK; ++g) issue_w(g, wq[g]);
        }
      }
    } else if (T <= kCompactMaxRows) {
      mine = compact_rows<BT>(a, sp, splits, rmap, wcnt, tid);
    } else {  // the split's contiguous rows; the epilogue applies the window
      for (int i = tid; i < BT; i += NT) rmap[i] = t0 + i < T ? (int)(t0 + i) : -1;
      __syncthreads();
      mine = (int)(T - t0 < BT ? T - t0 : BT);
    }
    nbe = (mine + 31) / 32;
    if (D != kRowsOut && ks > 1 && kq == 0 && rt == 0 && (!ADAPT || sp >= 0))  // for the reduce
      for (int i = tid; i < BT; i += NT) a.rowmap[sp * BT + i] = rmap[i];
    if (mine == 0) {  // uniform: nothing of this split is written
      wait_vmcnt<0>();
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < XPW; ++i) {
    const int slot = i * 256 + w * 64 + lane;
    const int t = slot / 8;
    const int piece = (slot % 8) ^ ((t >> 1) & 7);
    int64_t tok;
    if constexpr (COMMIT) {
      tok = rmap[t];
      xrow[i] = tok >= 0;
      tok = xrow[i] ? tok : 0;
    } else {
      tok = t0 + t < T ? t0 + t : T - 1;  // rows past T are never stored
      xrow[i] = true;
    }
    xoff[i] = tok * a.x_stride + piece * 8;
    xcol[i] = piece * 8;
  }

  f32x16 acc[NB];
#pragma unroll
  for (int tb = 0; tb < NB; ++tb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[tb][r] = 0.0f;

#pragma unroll
  for (int g = 0; g < LOOK; ++g) {
    if constexpr (!COMMIT) issue_w(g, wq[g]);
    issue_x(g);
  }
  // Main loop, instantiated for the number of 32-token blocks that hold rows
  // (commit windows may fill fewer than NB): empty blocks issue no MFMAs.
  auto main_loop = [&](auto nbe_c) {
    constexpr int NBE = decltype(nbe_c)::value;
    for (int g0 = 0; g0 < ng_ring; g0 += SLOTS) {
#pragma unroll
      for (int u = 0; u < SLOTS; ++u) {
        // this thread's loads of group g0 + u have landed (in issue order: the
        // first two waits of a commit-window prologue, which issued its weight
        // loads ahead of all X loads, leave fewer loads outstanding)
        if (COMMIT && u == 0 && g0 == 0)
          wait_ring<(LOOK - 1) * XPW>();
        else if (COMMIT && u == 1 && g0 == 0)
          wait_ring<(LOOK - 2) * XPW + LOADS>();
        else
          wait_ring<(LOOK - 1) * LOADS>();
        raw_barrier();  // ... and everyone's; group g0 + u - 1 is free
        issue_w(g0 + u + LOOK, wq[(u + LOOK) % SLOTS]);
        issue_x(g0 + u + LOOK);
        const uint16_t* xs = smem + ((2 * u + par) % XSTAGES) * SXE;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
          const vec8 av = __builtin_bit_cast(vec8, wq[u][kk]);
#pragma unroll
          for (int tb = 0; tb < NBE; ++tb) {
            const int t = tb * 32 + r32;
            const int slot = (4 * hh + kk) ^ ((t >> 1) & 7);
            const vec8 bv = *reinterpret_cast<const vec8*>(xs + (t * 8 + slot) * 8);
            acc[tb] = E::mfma(av, bv, acc[tb]);
          }
        }
      }
    }
  };
  if constexpr (COMMIT) {
    if (NB >= 4 && nbe >= 4) main_loop(std::integral_constant<int, NB>{});
    else if (NB >= 3 && nbe == 3) main_loop(std::integral_constant<int, NB >= 3 ? 3 : NB>{});
    else if (NB >= 2 && nbe == 2) main_loop(std::integral_constant<int, NB >= 2 ? 2 : NB>{});
    else main_loop(std::integral_constant<int, 1>{});
  } else {
    main_loop(std::integral_constant<int, NB>{});
  }
  wait_ring<0>();  // prefetches past the end (zero page) are done, LDS reads too
  raw_barrier();

  // add the two K halves, (+ bias), round to the dtype into the LDS tile [BT][LDO]
  float* red = reinterpret_cast<float*>(smem);
  uint16_t* sO = smem + BT * RS * 2;
  if (par == 1) {
#pragma unroll
    for (int tb = 0; tb < NB; ++tb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int tok = tb * 32 + r32;
        const int row = 32 * w + 8 * q + 4 * hh;
        *reinterpret_cast<float4*>(red + tok * RS + row) =
            make_float4(acc[tb][4 * q], acc[tb][4 * q + 1], acc[tb][4 * q + 2], acc[tb][4 * q + 3]);
      }
  }
  __syncthreads();
  if (D != kRowsOut && ks > 1) {
    // fp32 sums of this K part in the MFMA accumulator layout: tile (kq, rt,
    // sp) of BT x 128 floats, (block tb, row group w, quad q) 256 floats at
    // ((tb * 4 + w) * 4 + q) * 256, lane l at 4 l (one KiB per store)
    if (par == 0) {
      float* part = a.partial + ((int64_t)kq * R * splits + rt * splits + sp) * (int64_t)(BT * BN) +
                    w * 1024 + lane * 4;
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) {
        if (tb >= nbe) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int tok = tb * 32 + r32;
          const int row = 32 * w + 8 * q + 4 * hh;
          const float4 o = *reinterpret_cast<const float4*>(red + tok * RS + row);
          *reinterpret_cast<float4*>(part + tb * 4096 + q * 256) =
              make_float4(acc[tb][4 * q] + o.x, acc[tb][4 * q + 1] + o.y,
                          acc[tb][4 * q + 2] + o.z, acc[tb][4 * q + 3] + o.w);
        }
      }
    }
    return;
  }
  if (D == kRowsOut && ks > 1) {
    // fp32 partial sums of this K part: partial[(kq * T + t) * (R * 128) + n]
    if (par == 0) {
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) {
        const int tok = tb * 32 + r32;
        if (t0 + tok >= T) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 32 * w + 8 * q + 4 * hh;
          const float4 o = *reinterpret_cast<const float4*>(red + tok * RS + row);
          *reinterpret_cast<float4*>(a.partial + (kq * T + t0 + tok) * (R * BN) + n0 + row) =
              make_float4(acc[tb][4 * q] + o.x, acc[tb][4 * q + 1] + o.y,
                          acc[tb][4 * q + 2] + o.z, acc[tb][4 * q + 3] + o.w);
        }
      }
    }
    return;
  }
  if (par == 0) {
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      const int tok = tb * 32 + r32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 32 * w + 8 * q + 4 * hh;
        const float4 o = *reinterpret_cast<const float4*>(red + tok * RS + row);
        float v[4] = {acc[tb][4 * q] + o.x, acc[tb][4 * q + 1] + o.y, acc[tb][4 * q + 2] + o.z,
                      acc[tb][4 * q + 3] + o.w};
        if (BIAS) {
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] += E::to_f(a.bias[n0 + row + i]);
        }
        uint2 packed;
        packed.x = E::from_f(v[0]) | (E::from_f(v[1]) << 16);
        packed.y = E::from_f(v[2]) | (E::from_f(v[3]) << 16);
        *reinterpret_cast<uint2*>(sO + tok * LDO + row) = packed;
      }
    }
  }
  __syncthreads();
  if constexpr (D == kRowsOut)
    rows_out_tile<E, BT, LDO, NT, BN>(a, sO, n0, t0, tid);
  else
    scatter_tile<E, D, BT, COMMIT, LDO, NT>(a, sO, n0, t0, tid, COMMIT ? rmap : nullptr);
}

// Second launch of the write's K-split form: workgroup (rt, sp, tb) adds the
// K parts of one 32-token block of its tile in part order (so the sums do not
// depend on timing), adds the bias, rounds to the dtype and runs the epilogue
// of ctx_kv_stream_kernel for those rows (the committed-row map comes from K
// part 0's workgroup of row tile 0).
template <bool FP16, int D, bool BIAS, bool COMMIT, int NB>
__global__ __launch_bounds__(256) void ctx_kv_stream_reduce(const WriteArgs a, int splits) {
  using E = Elem<FP16>;
  constexpr int NT = 256;
  constexpr int BT = 32 * NB;
  constexpr int LDO = BN + 4;
  __shared__ __align__(16) uint16_t sO[32 * LDO];
  __shared__ int smap[32];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;  // 32-row group
  const int r32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t R = a.R;
  const int tb = (int)(blockIdx.x % NB);
  const int64_t sp = (blockIdx.x / NB) % splits;
  const int64_t rt = blockIdx.x / ((int64_t)NB * splits);
  const int ks = a.ksplits;
  if (COMMIT) {
    // the split's rows are compacted: a block whose first slot is empty is empty
    if (a.rowmap[sp * BT + tb * 32] < 0) return;
    if (tid < 32) smap[tid] = a.rowmap[sp * BT + tb * 32 + tid];
  } else if (sp * BT + tb * 32 >= a.T) {
    return;
  }
  const int64_t pstride = R * splits * (int64_t)(BT * BN);  // floats between K parts
  const float* src = a.partial + (rt * splits + sp) * (int64_t)(BT * BN) + tb * 4096 + w * 1024 +
                     lane * 4;
  float4 sum[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) sum[q] = *reinterpret_cast<const float4*>(src + q * 256);
  for (int k0 = 1; k0 < ks; k0 += 4) {  // up to four parts' loads in flight, added in order
    float4 v[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (k0 + u < ks) v[u][q] = *reinterpret_cast<const float4*>(src + (k0 + u) * pstride + q * 256);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (k0 + u < ks) {
          sum[q].x += v[u][q].x;
          sum[q].y += v[u][q].y;
          sum[q].z += v[u][q].z;
          sum[q].w += v[u][q].w;
        }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 32 * w + 8 * q + 4 * hh;
    float v[4] = {sum[q].x, sum[q].y, sum[q].z, sum[q].w};
    if (BIAS) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += E::to_f(a.bias[rt * BN + row + i]);
    }
    uint2 packed;
    packed.x = E::from_f(v[0]) | (E::from_f(v[1]) << 16);
    packed.y = E::from_f(v[2]) | (E::from_f(v[3]) << 16);
    *reinterpret_cast<uint2*>(sO + r32 * LDO + row) = packed;
  }
  __syncthreads();
  scatter_tile<E, D, 32, COMMIT, LDO, NT>(a, sO, rt * BN, sp * BT + tb * 32, tid,
                                          COMMIT ? smap : nullptr);
}

template <bool FP16, int D, bool BIAS, bool COMMIT>
hipError_t launch_tiled(const WriteArgs& a, const WritePlan& p, hipStream_t stream) {
  if (p.grid <= 0 || p.grid > 0x7FFFFFFF || p.splits > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)p.grid), block(512);
  const int t_tiles = (int)p.splits;
  switch (p.bt) {
    case 256:
      hipLaunchKernelGGL((ctx_kv_tiled_kernel<FP16, D, BIAS, COMMIT, 256>), grid, block, 0, stream,
                         a, t_tiles);
      break;
    case 192:
      hipLaunchKernelGGL((ctx_kv_tiled_kernel<FP16, D, BIAS, COMMIT, 192>), grid, block, 0, stream,
                         a, t_tiles);
      break;
    case 128:
      hipLaunchKernelGGL((ctx_kv_tiled_kernel<FP16, D, BIAS, COMMIT, 128>), grid, block, 0, stream,
                         a, t_tiles);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool FP16, int D, bool BIAS, bool COMMIT, int NB>
hipError_t launch_stream_nb(const WriteArgs& a, const WritePlan& p, hipStream_t stream) {
  if (p.grid <= 0 || p.grid > 0x7FFFFFFF || p.reduce_grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  WriteArgs b = a;
  b.ksplits = p.kernel == kKernelStreamKSplit ? p.ksplits : 1;
  if (p.adaptive) {  // compacted, K split unless the written rows need K whole
    if constexpr (COMMIT && NB == 4 && D != kRowsOut) {
      // (the adaptive scan holds two rows per thread)
      if (p.kernel != kKernelStreamKSplit || a.T > 1024) return hipErrorInvalidValue;
      hipLaunchKernelGGL((ctx_kv_stream_kernel<FP16, D, BIAS, COMMIT, NB, true>),
                         dim3((uint32_t)p.grid), dim3(512), 0, stream, b, (int)p.splits);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    hipLaunchKernelGGL((ctx_kv_stream_kernel<FP16, D, BIAS, COMMIT, NB>), dim3((uint32_t)p.grid),
                       dim3(512), 0, stream, b, (int)p.splits);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.kernel != kKernelStreamKSplit) return e;
  if constexpr (D != kRowsOut)
    hipLaunchKernelGGL((ctx_kv_stream_reduce<FP16, D, BIAS, COMMIT, NB>),
                       dim3((uint32_t)p.reduce_grid), dim3(256), 0, stream, b, (int)p.splits);
  return hipGetLastError();
}

// The plan's kernels: the LDS-tiled kernel for large T, else one round of
// streaming workgroups (row tiles x token splits of up to 4 blocks of 32
// tokens), with K also split over workgroups where few weight tiles would
// leave the device idle.
template <bool FP16, int D, bool BIAS, bool COMMIT>
hipError_t launch_plan(const WriteArgs& a, const WritePlan& p, hipStream_t stream) {
  if (p.kernel == kKernelTiled) return launch_tiled<FP16, D, BIAS, COMMIT>(a, p, stream);
  switch (p.nb) {
    case 1: return launch_stream_nb<FP16, D, BIAS, COMMIT, 1>(a, p, stream);
    case 2: return launch_stream_nb<FP16, D, BIAS, COMMIT, 2>(a, p, stream);
    case 3: return launch_stream_nb<FP16, D, BIAS, COMMIT, 3>(a, p, stream);
    case 4: return launch_stream_nb<FP16, D, BIAS, COMMIT, 4>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool FP16, int D, bool BIAS>
hipError_t launch_commit(const WriteArgs& a, const WritePlan& p, bool has_commit,
                         hipStream_t stream) {
  return has_commit ? launch_plan<FP16, D, BIAS, true>(a, p, stream)
                    : launch_plan<FP16, D, BIAS, false>(a, p, stream);
}

template <bool FP16, int D>
hipError_t launch_bias(const WriteArgs& a, const WritePlan& p, bool has_bias, bool has_commit,
                       hipStream_t stream) {
  return has_bias ? launch_commit<FP16, D, true>(a, p, has_commit, stream)
                  : launch_commit<FP16, D, false>(a, p, has_commit, stream);
}

template <bool FP16>
hipError_t launch_dim(const WriteArgs& a, const WritePlan& p, int head_dim, bool has_bias,
                      bool has_commit, hipStream_t stream) {
  if (head_dim == 128) return launch_bias<FP16, 128>(a, p, has_bias, has_commit, stream);
  if (head_dim == 64) return launch_bias<FP16, 64>(a, p, has_bias, has_commit, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rows_out(const WriteArgs& a, bool is_fp16, int num_cus, hipStream_t stream) {
  if (num_cus < 1) num_cus = 1;
  if (a.ksplits > 1) {  // 128-token tiles x K parts (see producer_ksplits)
    const int64_t splits = (a.T + 127) / 128;
    const int64_t grid = a.R * splits * a.ksplits;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (is_fp16)
      hipLaunchKernelGGL((ctx_kv_stream_kernel<true, kRowsOut, false, false, 4>), dim3((uint32_t)grid),
                         dim3(512), 0, stream, a, (int)splits);
    else
      hipLaunchKernelGGL((ctx_kv_stream_kernel<false, kRowsOut, false, false, 4>),
                         dim3((uint32_t)grid), dim3(512), 0, stream, a, (int)splits);
    return hipGetLastError();
  }
  const WritePlan p = plan_write(a.T, a.R, a.H, false, true, num_cus);
  return is_fp16 ? launch_plan<true, kRowsOut, false, false>(a, p, stream)
                 : launch_plan<false, kRowsOut, false, false>(a, p, stream);
}

hipError_t launch_ctx_kv_write(const WriteArgs& a, const WritePlan& plan, int head_dim,
                               bool is_fp16, bool has_bias, bool has_commit, hipStream_t stream) {
  return is_fp16 ? launch_dim<true>(a, plan, head_dim, has_bias, has_commit, stream)
                 : launch_dim<false>(a, plan, head_dim, has_bias, has_commit, stream);
}

}  // namespace dspark
