/*
 * dspark.h - C ABI of the DSpark cross-layer context-KV write for MI355X (gfx950).
 *
 * The operation (sglang PR #31986 "stack every DSpark layer's KV projection into
 * one GEMM", key source snippets; sglang PR #31847 "[spec decoding] support
 * inkling dspark", key source snippets): every draft layer's K/V rows of its
 * fused QKV projection are stacked into one weight W_stacked [L*2*kv, H]. The
 * shared ctx_hidden [T, H] goes through one GEMM against it (plus the stacked
 * bias when every layer has one). Per layer and per KV head, K then gets an
 * fp32 RMSNorm with that layer's k_norm weight and the shared eps, and a neox
 * rotation read from a cos/sin table at the row's position. K and the raw V are
 * scattered into each layer's KV pool at the row's slot.
 *
 * Numerics: fp32 accumulation; the GEMM output is rounded to the activation
 * dtype, the normalised K is rounded again, and the rotated K once more
 * (round-to-nearest-even each time), as in the per-layer eager path.
 *
 * Conventions for every call:
 *   - "device" pointers are HIP device memory of the device that is current on
 *     the calling thread; "host" pointers are ordinary host memory.
 *   - Element strides are in elements, not bytes.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *   - Status codes are the DSPARK_* values below. A call that returns anything
 *     but DSPARK_OK has enqueued no device work.
 *   - The calls that enqueue work (the write, the QK op, the verify step, the
 *     producer, the attention) allocate nothing and never synchronise the
 *     stream, so they can be captured in a HIP graph (the write's validate mode
 *     excepted); the pack calls allocate and synchronise.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
enum {
  DSPARK_OK = 0,
  DSPARK_FALLBACK = 1,     /* not eligible: the caller runs its per-layer path */
  DSPARK_E_INVALID = -1,   /* misuse: bad pointer, size or argument pairing */
  DSPARK_E_RANGE = -2,     /* validate mode: a stored row's position or slot is out of range,
                              or two stored rows name one slot (see DSPARK_RANGE_*) */
  DSPARK_E_DEVICE = -3,    /* a HIP runtime call failed */
  DSPARK_E_NOMEM = -4,     /* device allocation failed (pack only) */
  DSPARK_E_TOO_LARGE = -5  /* the static scratch cannot hold the workspace needed */
};

/* Why a pack or a write returned DSPARK_FALLBACK. */
enum {
  DSPARK_FB_NONE = 0,
  DSPARK_FB_NO_LAYERS = 1,       /* zero layers */
  DSPARK_FB_TOO_MANY_LAYERS = 2, /* more than DSPARK_MAX_LAYERS */
  DSPARK_FB_NOT_SLICEABLE = 3,   /* weight quantized, of another dtype, or not row-sliceable */
  DSPARK_FB_EPS_MISMATCH = 4,    /* layers disagree on the k_norm epsilon */
  DSPARK_FB_MIXED_BIAS = 5,      /* some layers have a QKV bias and some do not */
  DSPARK_FB_SHAPE = 6,           /* head_dim / kv_size differ across layers or are unsupported */
  DSPARK_FB_DTYPE = 7,           /* activation or k_norm dtype unsupported */
  DSPARK_FB_KV_SCALE = 8,        /* a K/V quantization scale is attached */
  DSPARK_FB_ROPE = 9,            /* rotary is not neox full-dim over one shared fp32 table */
  DSPARK_FB_POOL_LAYOUT = 10     /* pool dtype, head layout or alignment unsupported */
};

/* What a DSPARK_E_RANGE return of the write's validate mode found. */
enum {
  DSPARK_RANGE_NONE = 0,
  DSPARK_RANGE_POSITION = 1,   /* a stored row's position is outside [0, rope_max_pos) */
  DSPARK_RANGE_SLOT = 2,       /* a stored row's loc is >= a layer's num_slots */
  DSPARK_RANGE_DUPLICATE = 3   /* two stored rows name the same slot */
};

/* Flags of dspark_ctx_kv_write. */
enum {
  /* Before enqueueing, copy positions, locs and commit_lens to the host
   * (synchronising `stream`) and check the rows that would be stored; any
   * DSPARK_RANGE_* finding returns DSPARK_E_RANGE with nothing enqueued. Not
   * usable under stream capture. Without it the write trusts these
   * preconditions and only guards memory (see dspark_ctx_kv_write). */
  DSPARK_WRITE_VALIDATE = 1
};

/* Kernels a write can run (dspark_ctx_kv_plan). */
enum {
  DSPARK_KERNEL_STREAM = 0,         /* weight-streaming kernel, one launch */
  DSPARK_KERNEL_STREAM_KSPLIT = 1,  /* streaming kernel over K parts + a reduce launch */
  DSPARK_KERNEL_TILED = 2           /* LDS-tiled MFMA kernel, one launch */
};

/* Element types. */
enum { DSPARK_BF16 = 0, DSPARK_FP16 = 1, DSPARK_FP32 = 2, DSPARK_QUANTIZED = 99 };

#define DSPARK_MAX_LAYERS 32

/* One draft layer's attention parameters, as the layer holds them.
 * qkv_weight: device, w_rows x hidden, element (r, c) at r*w_row_stride +
 *   c*w_col_stride; rows are [Q: q_size | K: kv_size | V: kv_size | ...].
 *   The K/V slice is rows [q_size, q_size + 2*kv_size) (sglang PR #31986,
 *   "_stacked_ctx_kv_params"). Sliceable means w_dtype equals the activation
 *   dtype, w_col_stride == 1 and w_rows >= q_size + 2*kv_size.
 * qkv_bias: device [w_rows] contiguous, same dtype, or NULL.
 * k_norm_weight: device [head_dim] contiguous, dtype bf16, fp16 or fp32.
 * rope_cos_sin: device [rope_max_pos, rope_dim] fp32, row p = cos half | sin half.
 */
typedef struct {
  const void* qkv_weight;
  int64_t w_rows;
  int64_t w_row_stride;
  int64_t w_col_stride;
  int32_t w_dtype;
  const void* qkv_bias;
  const void* k_norm_weight;
  int32_t k_norm_dtype;
  double k_norm_eps;
  int64_t q_size;
  int64_t kv_size;
  int64_t head_dim;
  int32_t has_kv_scale;
  const void* rope_cos_sin;
  int32_t rope_dtype;
  int64_t rope_max_pos;
  int64_t rope_dim;
  int32_t rope_is_neox;
} dspark_layer_desc;

/* One layer's KV pool: device buffers [num_slots, num_kv_heads, head_dim].
 * Supported layout (else DSPARK_FALLBACK / DSPARK_FB_POOL_LAYOUT, as the
 * reference's bundle builder requires in sglang PR #31847): dtype equal to the
 * activation dtype, stride1 == head_dim, stride2 == 1, stride0 >= num_kv_heads *
 * head_dim, base pointers 16-byte aligned and stride0 a multiple of 8. */
typedef struct {
  void* k;
  void* v;
  int64_t num_slots;
  int64_t k_stride0, k_stride1, k_stride2;
  int64_t v_stride0, v_stride1, v_stride2;
  int32_t dtype;
} dspark_pool_desc;

typedef struct dspark_ctx_kv_pack dspark_ctx_kv_pack; /* opaque */

/* Eligibility of a set of layers for the stacked write, host-only: reads the
 * descriptors, never dereferences a device pointer. Checks (sglang PR #31986
 * "_stacked_ctx_kv_params" and PR #31847 "_build_fused_kv_write_bundle"):
 * at least one and at most DSPARK_MAX_LAYERS layers; every weight sliceable;
 * equal k_norm eps; bias present in all layers or none; equal head_dim and
 * kv_size with kv_size % head_dim == 0, head_dim in {64, 128}, hidden % 8 == 0;
 * act_dtype bf16 or fp16; no K/V scale; neox rotary with rope_dim == head_dim
 * over an fp32 table of the same shape in every layer.
 * Returns DSPARK_OK, or DSPARK_FALLBACK with *fallback_reason set (may be NULL),
 * or DSPARK_E_INVALID for a NULL `layers` with num_layers > 0 or hidden <= 0.
 * When two layers' table pointers differ, only dspark_pack_ctx_kv can compare
 * their contents; this call then assumes they are equal. */
int dspark_check_eligibility(const dspark_layer_desc* layers, int32_t num_layers,
                             int64_t hidden, int32_t act_dtype, int32_t* fallback_reason);

/* Builds the stacked parameters once (sglang PR #31986: cached stack of weight,
 * bias and fp32 k_norm weights). Runs dspark_check_eligibility, compares rotary
 * tables whose pointers differ, then allocates and fills on `stream`:
 * W_stacked [L*2*kv, hidden] (layer-major, K rows then V rows), the stacked bias
 * [L*2*kv] when present, k_norm [L, head_dim] widened to fp32. The rotary table
 * of layer 0 is referenced, not copied: it must outlive the pack. Synchronises
 * `stream` before returning, so the source weights may change afterwards; the
 * pack then still holds the old values (re-pack after a weight update). After
 * this call the pack is never written again: any number of writes may use it
 * at once, on any streams.
 * With the environment variable DSPARK_LOG set to a non-empty value other than
 * "0", every FALLBACK of this call and the first write FALLBACK of each pack
 * print their reason on stderr.
 * Returns DSPARK_OK with *out set, DSPARK_FALLBACK with *fallback_reason set
 * (*out = NULL), DSPARK_E_INVALID (NULL out), DSPARK_E_NOMEM or DSPARK_E_DEVICE. */
int dspark_pack_ctx_kv(const dspark_layer_desc* layers, int32_t num_layers, int64_t hidden,
                       int32_t act_dtype, void* stream, dspark_ctx_kv_pack** out,
                       int32_t* fallback_reason);

/* Launch plan of a write of num_tokens rows through `pack` on the current
 * device (host-only; what dspark_ctx_kv_write would enqueue). */
typedef struct {
  int32_t kernel;          /* DSPARK_KERNEL_* */
  int32_t token_tile;      /* tokens per workgroup (tiled: 128/192/256; streaming: 32..128) */
  int64_t workgroups;      /* of the main launch */
  int64_t reduce_workgroups; /* of the K-part reduce launch (0: none) */
  int32_t k_parts;         /* K split over workgroups (1: none) */
  int32_t compacts;        /* 1: only the rows that are stored are projected */
  int64_t workspace_bytes; /* device workspace the write needs (0: none) */
  int64_t token_splits;    /* streaming: token splits per weight tile; tiled: token tiles */
  int64_t adaptive;        /* 1: K parts only when the stored rows fit token_splits splits,
                              else K whole over token_splits x k_parts splits (decided on
                              the device from the committed rows) */
} dspark_write_plan;

/* Fills *plan for a write of num_tokens rows (has_commit: commit_lens given).
 * Returns DSPARK_OK, DSPARK_E_INVALID (NULL arguments, num_tokens < 0) or
 * DSPARK_E_DEVICE. */
int dspark_ctx_kv_plan(const dspark_ctx_kv_pack* pack, int64_t num_tokens, int32_t has_commit,
                       dspark_write_plan* plan);

/* Device workspace bytes dspark_ctx_kv_write needs for num_tokens rows
 * (has_commit: commit_lens given): fp32 sums of K parts when the write splits
 * K over workgroups (few weight tiles for the device, at most 128 x 128 floats
 * per compute unit plus an 8 KiB row map), else 0. Host-only. */
int dspark_ctx_kv_workspace_bytes(const dspark_ctx_kv_pack* pack, int64_t num_tokens,
                                  int32_t has_commit, int64_t* bytes);

/* The write: one GEMM of ctx_hidden against W_stacked, then per layer and K head
 * RMSNorm + neox rotation, and the scatter of K and raw V into the pools.
 *   ctx_hidden: device [num_tokens, hidden] in the activation dtype, row stride
 *     hidden_row_stride (>= hidden, multiple of 8), 16-byte aligned.
 *   positions: device int64 [num_tokens], each in [0, rope_max_pos).
 *   locs: device int64 [num_tokens]; a row with loc < 0 is not written
 *     (sglang PR #31847, "fused_kv_norm_rope_write").
 *   commit_lens: device int64 [num_requests] or NULL. When given, locs is a
 *     flattened [num_requests, locs_row_width] window and only columns
 *     c < commit_lens[b] of request b are written; other slots stay untouched.
 *     commit_lens and locs_row_width > 0 must come together, and
 *     num_requests * locs_row_width == num_tokens (else DSPARK_E_INVALID).
 *     Without commit_lens, locs_row_width and num_requests must be 0.
 *   pools: host array of num_pools == L descriptors, layer order of the pack.
 *   workspace: device, 16-byte aligned, at least dspark_ctx_kv_workspace_bytes
 *     bytes (may be NULL when that is 0). Scratch, owned by the caller: no
 *     need to clear it; writes that overlap in time must use different
 *     workspaces.
 *   range_errors: device counter or NULL. A stored row whose position is
 *     outside [0, rope_max_pos) or whose loc is >= that layer's num_slots is
 *     not written and adds 1 per (row, layer) here (atomically, never cleared);
 *     no memory outside the given buffers is ever accessed.
 *   flags: 0 or DSPARK_WRITE_VALIDATE (see there).
 * The rows that are stored must name distinct slots (the scatter is not
 * ordered between rows); validate mode reports a violation.
 * num_tokens == 0 returns DSPARK_OK with nothing enqueued. Without
 * DSPARK_WRITE_VALIDATE the call never synchronises the stream and allocates
 * nothing, so it can be captured in a HIP graph.
 * Returns DSPARK_OK (enqueued on `stream`); DSPARK_FALLBACK with *detail (may
 * be NULL) = DSPARK_FB_POOL_LAYOUT; DSPARK_E_RANGE (validate mode) with
 * *detail = DSPARK_RANGE_*; DSPARK_E_INVALID; or DSPARK_E_DEVICE. */
int dspark_ctx_kv_write(const dspark_ctx_kv_pack* pack, const void* ctx_hidden,
                        int64_t num_tokens, int64_t hidden_row_stride,
                        const int64_t* positions, const int64_t* locs,
                        const int64_t* commit_lens, int64_t locs_row_width,
                        int64_t num_requests, const dspark_pool_desc* pools,
                        int32_t num_pools, void* workspace, int64_t workspace_bytes,
                        unsigned long long* range_errors, uint32_t flags, void* stream,
                        int32_t* detail);

/* The write for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same operation, arguments and kernels as dspark_ctx_kv_write, without the
 * workspace arguments. Its scratch (the K-split part sums and row map, when
 * the write splits K) is a file-scope device array of
 * DSPARK_STATIC_SCRATCH_BYTES bytes, enough for any write on a device of up
 * to DSPARK_STATIC_SCRATCH_CUS compute units; each device the library runs
 * on holds its own copy until the process ends. The call allocates nothing,
 * never synchronises and keeps nothing between calls that must start at
 * zero. Every call on one device shares that device's scratch: calls that
 * overlap in time on one device (different streams) race.
 * flags must be 0 (validate mode synchronises; use dspark_ctx_kv_write).
 * Returns as dspark_ctx_kv_write, and DSPARK_E_TOO_LARGE when the write
 * would need more workspace than the scratch holds (nothing enqueued). */
#define DSPARK_STATIC_SCRATCH_CUS 256
#define DSPARK_STATIC_SCRATCH_BYTES (256LL * 128 * 128 * 4 + 2048 * 4)
int dspark_ctx_kv_write_static(const dspark_ctx_kv_pack* pack, const void* ctx_hidden,
                               int64_t num_tokens, int64_t hidden_row_stride,
                               const int64_t* positions, const int64_t* locs,
                               const int64_t* commit_lens, int64_t locs_row_width,
                               int64_t num_requests, const dspark_pool_desc* pools,
                               int32_t num_pools, unsigned long long* range_errors,
                               uint32_t flags, void* stream, int32_t* detail);

/* In-place table QK RMSNorm + neox RoPE on a fused QKV tensor (sglang PR
 * #31847, key source snippets: table_qk_norm_rope_ and
 * _table_qk_norm_rope_kernel in dflash_utils.py). No pack is involved.
 *   qkv: device [num_tokens, row_stride] in act_dtype (bf16 or fp16), 16-byte
 *     aligned, row_stride a multiple of 8 and >= (num_q_heads + num_k_heads) *
 *     head_dim. A row is [num_q_heads query heads | num_k_heads key heads |
 *     anything else], each head head_dim (64 or 128) wide: query head h and key
 *     head j start at columns h * head_dim and (num_q_heads + j) * head_dim.
 *   positions: device int64 [num_tokens].
 *   q_norm_weight, k_norm_weight: device [head_dim], 16-byte aligned, in
 *     act_dtype or fp32 (norm_weight_dtype).
 *   cos_sin: device fp32 [rope_max_pos, head_dim], row p = cos half | sin half,
 *     16-byte aligned.
 *   range_errors: device counter or NULL; see below.
 * For every token and every query and key head, the head is replaced by
 * round(round(x * inv * w) rotated), inv = 1 / sqrt(mean(x^2) + eps) in fp32, w
 * the query or key norm weight, the neox rotation over the pairs (i, i +
 * head_dim/2) with the cos/sin of the token's position; each rounding is
 * round-to-nearest-even into act_dtype. Every other column is left untouched.
 * A token whose position is outside [0, rope_max_pos) is left untouched and, if
 * range_errors is not NULL, counted there (atomically added, never cleared).
 * num_tokens == 0 returns DSPARK_OK with nothing enqueued. Enqueued on `stream`;
 * allocates nothing and does not synchronise.
 * Returns DSPARK_OK; DSPARK_FALLBACK with *fallback_reason (may be NULL) =
 * DSPARK_FB_DTYPE (act_dtype not bf16/fp16, or a weight dtype other than
 * act_dtype/fp32) or DSPARK_FB_SHAPE (head_dim not 64 or 128); DSPARK_E_INVALID
 * (negative sizes, non-positive head counts, short or unaligned row stride,
 * NULL or misaligned pointers with num_tokens > 0, rope_max_pos <= 0, eps
 * negative or not finite); DSPARK_E_DEVICE. */
int dspark_table_qk_norm_rope(void* qkv, int64_t num_tokens, int64_t row_stride,
                              const int64_t* positions, int32_t num_q_heads, int32_t num_k_heads,
                              int32_t head_dim, int32_t act_dtype, const void* q_norm_weight,
                              const void* k_norm_weight, int32_t norm_weight_dtype, double eps,
                              const float* cos_sin, int64_t rope_max_pos,
                              unsigned long long* range_errors, void* stream,
                              int32_t* fallback_reason);

/* Accept length and bonus token of the verify step (sglang PR #31847,
 * implementation breakdown step 2: compute_dflash_correct_drafts_and_bonus).
 *   draft_tokens: device int64 [num_requests, num_drafts], row stride
 *     draft_row_stride (>= num_drafts); may be NULL when num_drafts == 0.
 *   target_tokens: device int64 [num_requests, num_drafts + 1], row stride
 *     target_row_stride (>= num_drafts + 1): the target model's token at each
 *     verified position.
 *   accept_lens, bonus_tokens: device int64 [num_requests], written.
 * accept_lens[b] = length of the longest prefix of request b's drafts equal to
 * its target tokens (the first mismatching position, num_drafts when none);
 * bonus_tokens[b] = target_tokens[b][accept_lens[b]]. Exact integer compares.
 * num_requests == 0 returns DSPARK_OK with nothing enqueued. Enqueued on
 * `stream`; allocates nothing and does not synchronise.
 * Returns DSPARK_OK, DSPARK_E_INVALID (negative sizes, short strides, NULL
 * pointers with work to do) or DSPARK_E_DEVICE. */
int dspark_verify_accept(const int64_t* draft_tokens, int64_t draft_row_stride,
                         const int64_t* target_tokens, int64_t target_row_stride,
                         int64_t num_requests, int32_t num_drafts, int64_t* accept_lens,
                         int64_t* bonus_tokens, void* stream);

/* ---------------------------------------------------------- context producer
 * ctx_hidden = main_norm(main_proj(aux)) (vLLM PR #46995, key source snippets:
 * DSparkDeepseekV4Model.combine_hidden_states): the target's auxiliary hidden
 * states of n layers, concatenated to aux [T, n*H], go through a bias-free
 * linear main_proj (weight [H, n*H]) and an RMSNorm main_norm over the H
 * features: y = round(aux @ W^T), ctx = round(y * inv * g) with
 * inv = 1 / sqrt(mean(y^2) + eps) in fp32 and g the norm weight widened to
 * fp32; both roundings are round-to-nearest-even into the activation dtype. */
typedef struct dspark_main_proj_pack dspark_main_proj_pack; /* opaque */

/* Packs the projection once. weight: device [out_features, in_features] in
 * w_dtype, row stride w_row_stride (elements, >= in_features), 16-byte
 * aligned. norm_weight: device [out_features] in act_dtype or fp32. Copies
 * both (the weight into the library's blocked layout, see dspark_pack_buffers;
 * the norm weight widened to fp32), synchronises `stream`, and keeps no
 * reference to the sources.
 * Returns DSPARK_OK with *out set; DSPARK_FALLBACK with *fallback_reason
 * (may be NULL) = DSPARK_FB_DTYPE (act_dtype not bf16/fp16, norm weight dtype
 * not act_dtype/fp32), DSPARK_FB_NOT_SLICEABLE (w_dtype != act_dtype) or
 * DSPARK_FB_SHAPE (out_features % 128, in_features % 8, w_row_stride % 8 or
 * weight alignment); DSPARK_E_INVALID (NULL pointers or out, non-positive
 * sizes, short row stride, eps negative or not finite); DSPARK_E_NOMEM;
 * DSPARK_E_DEVICE. */
int dspark_pack_main_proj(const void* weight, int64_t out_features, int64_t in_features,
                          int64_t w_row_stride, int32_t w_dtype, const void* norm_weight,
                          int32_t norm_weight_dtype, double eps, int32_t act_dtype, void* stream,
                          dspark_main_proj_pack** out, int32_t* fallback_reason);

/* Device workspace bytes dspark_main_proj_norm needs for num_tokens tokens
 * (one fp32 per token and 128-feature group). Host-only. */
int dspark_main_proj_workspace_bytes(const dspark_main_proj_pack* pack, int64_t num_tokens,
                                     int64_t* bytes);

/* The producer for num_tokens tokens: aux_hidden device [num_tokens,
 * in_features] (row stride aux_row_stride >= in_features, a multiple of 8,
 * 16-byte aligned) -> ctx_hidden device [num_tokens, out_features] (row stride
 * ctx_row_stride, same rules), written whole. workspace: device, 16-byte
 * aligned, at least dspark_main_proj_workspace_bytes; its contents are
 * scratch (no need to clear; calls sharing a workspace on different streams
 * race). Two launches on `stream` (the projection, then the row norm in place
 * on ctx_hidden); allocates nothing and does not synchronise.
 * num_tokens == 0 returns DSPARK_OK with nothing enqueued.
 * Returns DSPARK_OK, DSPARK_E_INVALID (NULL pointers with work to do, strides,
 * alignment, workspace too small, pack of another device) or DSPARK_E_DEVICE. */
int dspark_main_proj_norm(const dspark_main_proj_pack* pack, const void* aux_hidden,
                          int64_t num_tokens, int64_t aux_row_stride, void* ctx_hidden,
                          int64_t ctx_row_stride, void* workspace, int64_t workspace_bytes,
                          void* stream);

/* Frees the producer pack (waits for the device first). NULL is a no-op. */
void dspark_main_proj_free(dspark_main_proj_pack* pack);

/* ------------------------------------------------------------ draft attention
 * Bidirectional grouped-query attention of the draft over a layer's KV pool
 * (sglang PR #35499, implementation breakdown and key source snippets: the
 * shared-KV split-KV stage and the combine stage, query head h reading KV
 * head h // (num_q_heads / num_kv_heads), the causal mask off for the draft).
 * Every request b has `block` query tokens (rows b * block + j); its keys and
 * values are its prefix, the pool slots kv_indices[kv_indptr[b] ..
 * kv_indptr[b + 1]), followed by the block's own rows of k_ext / v_ext; every
 * query sees every key of its request:
 *   o = softmax(q . K^T * sm_scale) V, fp32 accumulation and softmax, the
 *   probabilities rounded to the dtype for the value product, o rounded once.
 * All tensors are device memory in the activation dtype with element strides;
 * the last (head_dim) stride is 1 and rows are 16-byte aligned. */
typedef struct {
  const void* q;            /* [num_requests * block, num_q_heads, head_dim] */
  int64_t q_token_stride, q_head_stride;
  const void* k_ext;        /* [num_requests * block, num_kv_heads, head_dim] */
  const void* v_ext;        /* same layout as k_ext */
  int64_t ext_token_stride, ext_head_stride;
  const void* k_pool;       /* [num_slots, num_kv_heads, head_dim] */
  const void* v_pool;       /* same layout as k_pool */
  int64_t pool_slot_stride, pool_head_stride;
  int64_t num_slots;
  const int64_t* kv_indptr;   /* device [num_requests + 1], non-decreasing */
  const int64_t* kv_indices;  /* device, the prefix slots */
  void* out;                /* [num_requests * block, num_q_heads, head_dim], written */
  int64_t out_token_stride, out_head_stride;
} dspark_attn_desc;

/* Device workspace bytes of dspark_draft_attention for these sizes (one fp32
 * record of 32 rows x (head_dim + 2) per request, KV head, 32-row tile and
 * key split). Host-only. Returns DSPARK_OK or DSPARK_E_INVALID. */
int dspark_draft_attention_workspace_bytes(int64_t num_requests, int32_t block,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int64_t max_prefix, int64_t* bytes);

/* The attention. max_prefix (host) must be >= every request's prefix length:
 * it sizes the key splits; keys of a prefix past max_prefix are not attended,
 * and each such request is counted in range_errors. A slot outside [0, num_slots) is skipped and
 * counted. range_errors: device counter or NULL (atomically added, never
 * cleared). workspace: device, 16-byte aligned, at least
 * dspark_draft_attention_workspace_bytes (scratch; calls sharing it on
 * different streams race). Two launches on `stream`; allocates nothing and
 * does not synchronise. num_requests == 0 returns DSPARK_OK, nothing enqueued.
 * Returns DSPARK_OK; DSPARK_FALLBACK with *fallback_reason (may be NULL) =
 * DSPARK_FB_SHAPE (head_dim not 64 or 128) or DSPARK_FB_DTYPE (not bf16/fp16);
 * DSPARK_E_INVALID (NULL desc or pointers with work to do, num_q_heads not a
 * multiple of num_kv_heads, block < 1, strides not multiples of 8 or
 * misaligned bases, num_slots < 1, workspace too small); DSPARK_E_DEVICE. */
int dspark_draft_attention(const dspark_attn_desc* desc, int64_t num_requests, int32_t block,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t act_dtype, double sm_scale, int64_t max_prefix,
                           void* workspace, int64_t workspace_bytes,
                           unsigned long long* range_errors, void* stream,
                           int32_t* fallback_reason);

/* Shape of a pack (host-only). Any output pointer may be NULL. */
int dspark_pack_info(const dspark_ctx_kv_pack* pack, int32_t* num_layers, int64_t* hidden,
                     int64_t* kv_size, int64_t* head_dim, int32_t* act_dtype,
                     int32_t* has_bias);

/* Device pointers of the pack's stacked weight, bias (NULL if none) and fp32
 * k_norm [L, head_dim], for inspection. Owned by the pack.
 * The bias is [L*2*kv] in stacking order. The stacked weight [L*2*kv, hidden]
 * (layer-major, K rows then V rows) is stored in the library's blocked
 * layout: with nk = ceil(hidden / 64), block (rt, c) for row tile rt (rows
 * [128 rt, 128 rt + 128)) and column chunk c (columns [64 c, 64 c + 64)) is
 * 1024 pieces of 8 elements starting at element ((rt * nk + c) * 1024) * 8;
 * piece q = (g * 4 + s) * 64 + l holds row 128 rt + 32 g + (l % 32), columns
 * 64 c + 32 (l / 32) + 8 s + [0, 8). Columns at or past `hidden` are zero. */
int dspark_pack_buffers(const dspark_ctx_kv_pack* pack, const void** w_stacked,
                        const void** bias, const float** k_norm);

/* Frees the pack's device buffers (waits for the device first). NULL is a no-op. */
void dspark_pack_free(dspark_ctx_kv_pack* pack);

/* Static strings for a status code, a fallback reason and a range cause. */
const char* dspark_status_str(int status);
const char* dspark_fallback_str(int reason);
const char* dspark_range_str(int cause);

#ifdef __cplusplus
}
#endif
#endif /* DSPARK_H */
