// Internal declarations of the HIP library (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dspark.h"
#include "host_logic.h"

namespace dspark {

constexpr int kMaxLayers = DSPARK_MAX_LAYERS;

// Everything the fused write kernel reads, passed by value in the kernel
// arguments so that one launch can address every layer's pool.
struct WriteArgs {
  const uint16_t* x;        // ctx_hidden [T, H] (row stride x_stride)
  const uint16_t* w;        // W_stacked in the blocked layout, N_tot = L * 2 * NH * D rows
  const uint16_t* bias;     // [N_tot] or nullptr
  const float* knw;         // [L, D] fp32
  const uint16_t* zeros;    // 16 zero bytes: the source of K-tail lanes past H
  const float* table;       // [P, D] fp32: cos half | sin half
  const int64_t* pos;       // [T]
  const int64_t* locs;      // [T]
  const int64_t* commit;    // [T / W] or nullptr
  unsigned long long* err;  // range error counter or nullptr
  uint16_t* y;              // producer only: [T, R * 128] output rows (row stride y_stride)
  float* partial;           // producer: [R, T] sums of squares per 128-feature group;
                            // write: fp32 K-part sums of the caller's workspace
  int* rowmap;              // write: committed-row map of the caller's workspace
  int64_t y_stride;
  int64_t R;                // 128-row tiles of the blocked weight
  int32_t ksplits;          // K parts over workgroups (<= 1: none); set by the launchers
  int64_t x_stride;
  int64_t T;
  int64_t P;
  int64_t W;                // commit window width (1 when no commit_lens)
  int32_t H;
  int32_t L;
  int32_t NH;
  float eps;
  uint16_t* pk[kMaxLayers];
  uint16_t* pv[kMaxLayers];
  int64_t ks0[kMaxLayers];
  int64_t vs0[kMaxLayers];
  int64_t slots[kMaxLayers];
};

// Arguments of the in-place table QK norm + rotation.
struct QkArgs {
  uint16_t* qkv;            // [T, row_stride]: NHQ query heads, NHK key heads, ...
  const int64_t* pos;       // [T]
  const void* qw;           // [D] query norm weight (dtype patterns or fp32)
  const void* kw;           // [D] key norm weight
  const float* table;       // [P, D] fp32: cos half | sin half
  unsigned long long* err;  // tokens skipped for a position outside the table, or nullptr
  int64_t T;
  int64_t row_stride;
  int64_t P;
  int32_t NHQ;
  int32_t NHT;              // NHQ + NHK
  float eps;
};

// Launches the in-place QK norm + rotation for `a` on `stream` (head_dim 64
// or 128, validated by the caller). Returns the launch status.
hipError_t launch_qk_norm_rope(const QkArgs& a, int head_dim, bool is_fp16, bool weight_fp32,
                               hipStream_t stream);

// Arguments of the verify accept length + bonus token.
struct VerifyArgs {
  const int64_t* draft;     // [B, >= K] drafted tokens
  const int64_t* target;    // [B, >= K + 1] target tokens
  int64_t draft_stride;     // elements between requests
  int64_t target_stride;
  int64_t B;
  int64_t* accept;          // [B]
  int64_t* bonus;           // [B]
  int32_t K;
  int32_t lanes_per_request;  // set by the launcher
};

// Launches the verify accept/bonus kernel for `a` on `stream` (validated by
// the caller). Returns the launch status.
hipError_t launch_verify_accept(const VerifyArgs& a, hipStream_t stream);

// Launches the context producer's GEMM for `a` (x = aux hidden, w = blocked
// projection weight with a.R row tiles, H = input features): rounded outputs
// to a.y and per-(128-feature group, token) sums of squares to a.partial, or,
// with a.ksplits > 1, fp32 partial projections to a.partial.
hipError_t launch_rows_out(const WriteArgs& a, bool is_fp16, int num_cus, hipStream_t stream);

// Launches the row RMSNorm that completes the producer. With ksplits <= 1, y
// holds the rounded projection and `partial` the [groups, T] group sums of
// squares; with ksplits > 1, `partial` holds [ksplits, T, groups * 128] fp32
// partial projections and y is written whole.
hipError_t launch_row_norm(uint16_t* y, int64_t y_stride, const float* partial, int64_t T,
                           int64_t groups, int ksplits, const float* g, float eps, bool is_fp16,
                           hipStream_t stream);

// Arguments of the draft attention (element strides).
struct AttnArgs {
  const uint16_t* q;        // [B * block, nhq, D]
  const uint16_t* k_ext;    // [B * block, nhk, D] (the block's own keys)
  const uint16_t* v_ext;
  const uint16_t* k_pool;   // [num_slots, nhk, D]
  const uint16_t* v_pool;
  const int64_t* kv_indptr;   // [B + 1]
  const int64_t* kv_indices;  // prefix slots
  uint16_t* out;            // [B * block, nhq, D]
  float* part;              // workspace: per split record O [32][D], m [32], l [32]
  unsigned long long* err;  // skipped slots and uncovered prefixes, or nullptr
  int64_t q_stride0, q_stride1;
  int64_t ext_stride0, ext_stride1;
  int64_t pool_stride0, pool_stride1;
  int64_t out_stride0, out_stride1;
  int64_t num_slots;
  int64_t B;
  int64_t split_len;        // prefix keys per split (multiple of 32)
  int64_t max_prefix;       // prefix keys past this are not attended
  int32_t block, nhk, G, M;  // M = block * G rows per (request, KV head)
  int32_t row_tiles;        // ceil(M / 32)
  int32_t n_splits;         // prefix splits; the block's keys are one more
  float sm_scale;
};

// Launches the two draft-attention stages for `a` (validated by the caller).
hipError_t launch_draft_attention(const AttnArgs& a, int head_dim, bool is_fp16,
                                  hipStream_t stream);

// Launches the fused GEMM + norm + rotation + scatter for `a` on `stream`
// following `plan` (plan_write for a.T, a.R, a.H). Shapes and the workspace
// (a.partial, a.rowmap for the K-split plan) have been validated by the
// caller. Returns the launch status.
hipError_t launch_ctx_kv_write(const WriteArgs& a, const WritePlan& plan, int head_dim,
                               bool is_fp16, bool has_bias, bool has_commit, hipStream_t stream);

// Pack helpers.
hipError_t launch_widen_to_f32(const void* src, int dtype, float* dst, int64_t n,
                               hipStream_t stream);
// Rewrites a plain row-major [rows, H] weight (rows % 128 == 0) into the
// blocked layout the write kernels read.
hipError_t launch_block_weight(const uint16_t* plain, int64_t rows, int64_t H, uint16_t* blk,
                               hipStream_t stream);
hipError_t launch_compare_f32(const float* a, const float* b, int64_t n, int* differ,
                              hipStream_t stream);

}  // namespace dspark
