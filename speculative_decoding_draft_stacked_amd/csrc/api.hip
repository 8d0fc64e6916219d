// C ABI of the context-KV write library: eligibility, pack, plan, write, strings.
//
// Eligibility follows the fast-path-or-fallback pattern of sglang PR #31986
// ("_stacked_ctx_kv_params": sliceable weights, equal eps, consistent bias) and
// sglang PR #31847 ("_build_fused_kv_write_bundle": no K/V scale, equal head
// shape, neox full-dim rotary over one shared table, pool dtype and head-major
// layout). Every reason is reported instead of falling back silently, and with
// DSPARK_LOG set it is also printed.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <new>
#include <vector>

#include "internal.h"

// Scratch of dspark_ctx_kv_write_static: the K-split part sums and row map of
// one write for up to DSPARK_STATIC_SCRATCH_CUS compute units, in a
// file-scope device array (each device holds its own copy for the life of the
// process). Host code uses only the device address that hipGetSymbolAddress
// returns for it, taken once per device with that device current; the name
// itself is a host-side stand-in.
constexpr int64_t kStaticScratchBytes =
    (int64_t)DSPARK_STATIC_SCRATCH_CUS * 128 * 128 * 4 + dspark::kRowMapInts * 4;
static_assert(kStaticScratchBytes == DSPARK_STATIC_SCRATCH_BYTES, "header constant");
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

struct dspark_ctx_kv_pack {
  int device;
  int num_cus;               // compute units of `device`
  int32_t num_layers;
  int64_t hidden;
  int64_t kv_size;
  int64_t head_dim;
  int32_t dtype;
  int32_t has_bias;
  float eps;
  uint16_t* w;               // [L * 2 * kv, hidden] in the blocked layout
  uint16_t* bias;            // [L * 2 * kv] or nullptr
  float* knw;                // [L, head_dim]
  const float* table;        // [P, head_dim], caller-owned
  int64_t table_rows;
  uint16_t* zeros;           // 256 zero bytes read by out-of-range K lanes
  mutable std::atomic<bool> logged_fallback{false};  // DSPARK_LOG: first write fallback printed
};

namespace {

void set_reason(int32_t* out, int32_t r) {
  if (out) *out = r;
}

int fallback(int32_t* out, int32_t r) {
  set_reason(out, r);
  return DSPARK_FALLBACK;
}

// DSPARK_LOG set to a non-empty value other than "0" (read on fallback and
// error paths only).
bool log_enabled() {
  const char* v = std::getenv("DSPARK_LOG");
  return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

void free_pack(dspark_ctx_kv_pack* p) {
  if (!p) return;
  if (p->w) (void)hipFree(p->w);
  if (p->bias) (void)hipFree(p->bias);
  if (p->knw) (void)hipFree(p->knw);
  if (p->zeros) (void)hipFree(p->zeros);
  delete p;
}

int pack_fallback(int32_t* out, int32_t r) {
  if (log_enabled())
    std::fprintf(stderr, "dspark: dspark_pack_ctx_kv fell back: %s\n", dspark_fallback_str(r));
  return fallback(out, r);
}

dspark::WritePlan plan_for(const dspark_ctx_kv_pack* p, int64_t T, bool has_commit) {
  const int64_t R = (int64_t)p->num_layers * 2 * p->kv_size / 128;
  return dspark::plan_write(T, R, p->hidden, has_commit, false, p->num_cus);
}

}  // namespace

extern "C" {

int dspark_check_eligibility(const dspark_layer_desc* layers, int32_t num_layers, int64_t hidden,
                             int32_t act_dtype, int32_t* fallback_reason) {
  return dspark::check_layers(layers, num_layers, hidden, act_dtype, fallback_reason);
}

int dspark_pack_ctx_kv(const dspark_layer_desc* layers, int32_t num_layers, int64_t hidden,
                       int32_t act_dtype, void* stream_ptr, dspark_ctx_kv_pack** out,
                       int32_t* fallback_reason) {
  if (!out) return DSPARK_E_INVALID;
  *out = nullptr;
  int32_t reason = DSPARK_FB_NONE;
  const int st = dspark::check_layers(layers, num_layers, hidden, act_dtype, &reason);
  set_reason(fallback_reason, reason);
  if (st == DSPARK_FALLBACK) return pack_fallback(fallback_reason, reason);
  if (st != DSPARK_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  for (int32_t i = 0; i < num_layers; ++i) {
    // 16-byte vector reads of every weight row need an aligned base
    if (reinterpret_cast<uintptr_t>(layers[i].qkv_weight) % 16 != 0)
      return pack_fallback(fallback_reason, DSPARK_FB_NOT_SLICEABLE);
  }

  dspark_ctx_kv_pack* p = new (std::nothrow) dspark_ctx_kv_pack();
  if (!p) return DSPARK_E_NOMEM;
  const dspark_layer_desc& l0 = layers[0];
  if (hipGetDevice(&p->device) != hipSuccess ||
      hipDeviceGetAttribute(&p->num_cus, hipDeviceAttributeMultiprocessorCount, p->device) !=
          hipSuccess) {
    delete p;
    return DSPARK_E_DEVICE;
  }
  p->num_layers = num_layers;
  p->hidden = hidden;
  p->kv_size = l0.kv_size;
  p->head_dim = l0.head_dim;
  p->dtype = act_dtype;
  p->has_bias = l0.qkv_bias != nullptr;
  p->eps = (float)l0.k_norm_eps;
  p->table = static_cast<const float*>(l0.rope_cos_sin);
  p->table_rows = l0.rope_max_pos;

  const int64_t kv2 = 2 * l0.kv_size;
  const int64_t n_tot = num_layers * kv2;
  const int64_t nk = (hidden + 63) / 64;
  int* differ = nullptr;
  uint16_t* plain = nullptr;
  auto fail = [&](int s) {
    if (differ) (void)hipFree(differ);
    if (plain) (void)hipFree(plain);
    free_pack(p);
    return s;
  };
  if (hipMalloc(&p->w, (size_t)(n_tot * nk * 64 * 2)) != hipSuccess) return fail(DSPARK_E_NOMEM);
  if (hipMalloc(&plain, (size_t)(n_tot * hidden * 2)) != hipSuccess) return fail(DSPARK_E_NOMEM);
  if (p->has_bias && hipMalloc(&p->bias, (size_t)(n_tot * 2)) != hipSuccess)
    return fail(DSPARK_E_NOMEM);
  if (hipMalloc(&p->knw, (size_t)(num_layers * l0.head_dim * 4)) != hipSuccess)
    return fail(DSPARK_E_NOMEM);
  if (hipMalloc(&p->zeros, 256) != hipSuccess) return fail(DSPARK_E_NOMEM);
  if (hipMalloc(&differ, sizeof(int)) != hipSuccess) return fail(DSPARK_E_NOMEM);

  bool ok = true;
  for (int32_t l = 0; l < num_layers && ok; ++l) {
    const dspark_layer_desc& d = layers[l];
    const uint16_t* src = static_cast<const uint16_t*>(d.qkv_weight) + d.q_size * d.w_row_stride;
    ok &= hipMemcpy2DAsync(plain + l * kv2 * hidden, (size_t)(hidden * 2), src,
                           (size_t)(d.w_row_stride * 2), (size_t)(hidden * 2), (size_t)kv2,
                           hipMemcpyDeviceToDevice, stream) == hipSuccess;
    if (p->has_bias)
      ok &= hipMemcpyAsync(p->bias + l * kv2, static_cast<const uint16_t*>(d.qkv_bias) + d.q_size,
                           (size_t)(kv2 * 2), hipMemcpyDeviceToDevice, stream) == hipSuccess;
    ok &= dspark::launch_widen_to_f32(d.k_norm_weight, d.k_norm_dtype, p->knw + l * l0.head_dim,
                                      l0.head_dim, stream) == hipSuccess;
  }
  ok = ok && dspark::launch_block_weight(plain, n_tot, hidden, p->w, stream) == hipSuccess;
  ok = ok && hipMemsetAsync(p->zeros, 0, 256, stream) == hipSuccess;
  ok = ok && hipMemsetAsync(differ, 0, sizeof(int), stream) == hipSuccess;
  for (int32_t l = 1; l < num_layers && ok; ++l) {
    if (layers[l].rope_cos_sin != l0.rope_cos_sin)
      ok &= dspark::launch_compare_f32(p->table, static_cast<const float*>(layers[l].rope_cos_sin),
                                       l0.rope_max_pos * l0.rope_dim, differ, stream) == hipSuccess;
  }
  int h_differ = 0;
  ok = ok && hipMemcpyAsync(&h_differ, differ, sizeof(int), hipMemcpyDeviceToHost, stream) ==
                 hipSuccess;
  ok = ok && hipStreamSynchronize(stream) == hipSuccess;
  if (!ok) return fail(DSPARK_E_DEVICE);
  if (h_differ) {
    fail(DSPARK_FALLBACK);
    return pack_fallback(fallback_reason, DSPARK_FB_ROPE);
  }
  (void)hipFree(differ);
  (void)hipFree(plain);
  *out = p;
  return DSPARK_OK;
}

int dspark_ctx_kv_plan(const dspark_ctx_kv_pack* p, int64_t num_tokens, int32_t has_commit,
                       dspark_write_plan* plan) {
  if (!p || !plan || num_tokens < 0) return DSPARK_E_INVALID;
  const dspark::WritePlan w = plan_for(p, num_tokens, has_commit != 0);
  plan->kernel = w.kernel;
  plan->token_tile = w.kernel == dspark::kKernelTiled ? w.bt : 32 * w.nb;
  plan->workgroups = w.grid;
  plan->reduce_workgroups = w.reduce_grid;
  plan->k_parts = w.ksplits;
  plan->compacts = w.compacts ? 1 : 0;
  plan->workspace_bytes = dspark::plan_workspace_bytes(w);
  plan->token_splits = w.splits;
  plan->adaptive = w.adaptive ? 1 : 0;
  return DSPARK_OK;
}

int dspark_ctx_kv_workspace_bytes(const dspark_ctx_kv_pack* p, int64_t num_tokens,
                                  int32_t has_commit, int64_t* bytes) {
  if (!p || !bytes || num_tokens < 0) return DSPARK_E_INVALID;
  *bytes = dspark::plan_workspace_bytes(plan_for(p, num_tokens, has_commit != 0));
  return DSPARK_OK;
}

}  // extern "C"

namespace {

// Validate mode: the index arrays to the host (synchronising `stream`) and the
// row checks. DSPARK_OK, DSPARK_E_RANGE (cause in *detail) or DSPARK_E_DEVICE.
int validate_rows(const dspark_ctx_kv_pack* p, const dspark::WriteArgs& a, int64_t num_requests,
                  hipStream_t stream, int32_t* detail) {
  const int64_t T = a.T;
  std::vector<int64_t> pos((size_t)T), locs((size_t)T), commit((size_t)num_requests);
  bool ok = hipMemcpyAsync(pos.data(), a.pos, (size_t)T * 8, hipMemcpyDeviceToHost, stream) ==
                hipSuccess &&
            hipMemcpyAsync(locs.data(), a.locs, (size_t)T * 8, hipMemcpyDeviceToHost, stream) ==
                hipSuccess;
  if (ok && a.commit)
    ok = hipMemcpyAsync(commit.data(), a.commit, (size_t)num_requests * 8, hipMemcpyDeviceToHost,
                        stream) == hipSuccess;
  ok = ok && hipStreamSynchronize(stream) == hipSuccess;
  if (!ok) return DSPARK_E_DEVICE;
  int32_t cause = DSPARK_RANGE_NONE;
  int64_t row = -1;
  const int st = dspark::check_rows(pos.data(), locs.data(), a.commit ? commit.data() : nullptr,
                                    T, a.W, a.P, a.slots, p->num_layers, &cause, &row);
  if (st == DSPARK_E_RANGE) {
    set_reason(detail, cause);
    if (log_enabled())
      std::fprintf(stderr, "dspark: dspark_ctx_kv_write validate: row %lld: %s\n",
                   (long long)row, dspark_range_str(cause));
  }
  return st;
}

// Shared body of the write entry points: checks, the args, the plan, launch.
int write_impl(const dspark_ctx_kv_pack* p, const void* ctx_hidden, int64_t num_tokens,
               int64_t hidden_row_stride, const int64_t* positions, const int64_t* locs,
               const int64_t* commit_lens, int64_t locs_row_width, int64_t num_requests,
               const dspark_pool_desc* pools, int32_t num_pools, void* workspace,
               int64_t workspace_bytes, unsigned long long* range_errors, uint32_t flags,
               void* stream_ptr, int32_t* detail) {
  set_reason(detail, DSPARK_FB_NONE);
  if (!p || num_tokens < 0) return DSPARK_E_INVALID;
  // commit_lens and the window width come together (sglang PR #31847,
  // "fused_kv_norm_rope_write": ValueError otherwise)
  const bool has_commit = commit_lens != nullptr;
  if (!dspark::write_window_ok(has_commit, num_tokens, locs_row_width, num_requests))
    return DSPARK_E_INVALID;
  if (flags & ~(uint32_t)DSPARK_WRITE_VALIDATE) return DSPARK_E_INVALID;
  if (!pools || num_pools != p->num_layers) return DSPARK_E_INVALID;
  if (num_tokens == 0) return DSPARK_OK;
  if (!ctx_hidden || !positions || !locs) return DSPARK_E_INVALID;
  if (hidden_row_stride < p->hidden || hidden_row_stride % 8 != 0 ||
      reinterpret_cast<uintptr_t>(ctx_hidden) % 16 != 0)
    return DSPARK_E_INVALID;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DSPARK_E_DEVICE;
  if (dev != p->device) return DSPARK_E_INVALID;

  const int64_t D = p->head_dim;
  const int64_t NH = p->kv_size / D;
  dspark::WriteArgs a = {};
  for (int32_t l = 0; l < p->num_layers; ++l) {
    const dspark_pool_desc& q = pools[l];
    if (!q.k || !q.v || q.num_slots < 0) return DSPARK_E_INVALID;
    if (!dspark::pool_layout_ok(q, p->dtype, NH, D)) {
      if (log_enabled() && !p->logged_fallback.exchange(true))
        std::fprintf(stderr, "dspark: dspark_ctx_kv_write fell back (layer %d): %s\n", (int)l,
                     dspark_fallback_str(DSPARK_FB_POOL_LAYOUT));
      return fallback(detail, DSPARK_FB_POOL_LAYOUT);
    }
    a.pk[l] = static_cast<uint16_t*>(q.k);
    a.pv[l] = static_cast<uint16_t*>(q.v);
    a.ks0[l] = q.k_stride0;
    a.vs0[l] = q.v_stride0;
    a.slots[l] = q.num_slots;
  }
  const dspark::WritePlan plan = plan_for(p, num_tokens, has_commit);
  const int64_t need = dspark::plan_workspace_bytes(plan);
  if (need > 0) {
    if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
      return DSPARK_E_INVALID;
    a.partial = static_cast<float*>(workspace);
    a.rowmap = reinterpret_cast<int*>(static_cast<char*>(workspace) + plan.part_floats * 4);
  }
  a.x = static_cast<const uint16_t*>(ctx_hidden);
  a.w = p->w;
  a.bias = p->bias;
  a.knw = p->knw;
  a.zeros = p->zeros;
  a.table = p->table;
  a.pos = positions;
  a.locs = locs;
  a.commit = commit_lens;
  a.err = range_errors;
  a.x_stride = hidden_row_stride;
  a.T = num_tokens;
  a.P = p->table_rows;
  a.W = has_commit ? locs_row_width : 1;
  a.H = (int32_t)p->hidden;
  a.L = p->num_layers;
  a.NH = (int32_t)NH;
  a.R = (int64_t)p->num_layers * 2 * p->kv_size / 128;
  a.eps = p->eps;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  if (flags & DSPARK_WRITE_VALIDATE) {
    const int st = validate_rows(p, a, num_requests, stream, detail);
    if (st != DSPARK_OK) return st;
  }
  const hipError_t e = dspark::launch_ctx_kv_write(a, plan, (int)D, p->dtype == DSPARK_FP16,
                                                   p->has_bias != 0, has_commit, stream);
  return e == hipSuccess ? DSPARK_OK : DSPARK_E_DEVICE;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the
// first call on that device).
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSPARK_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return DSPARK_E_DEVICE;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSPARK_OK;
}

}  // namespace

extern "C" {

int dspark_ctx_kv_write_static(const dspark_ctx_kv_pack* p, const void* ctx_hidden,
                               int64_t num_tokens, int64_t hidden_row_stride,
                               const int64_t* positions, const int64_t* locs,
                               const int64_t* commit_lens, int64_t locs_row_width,
                               int64_t num_requests, const dspark_pool_desc* pools,
                               int32_t num_pools, unsigned long long* range_errors,
                               uint32_t flags, void* stream_ptr, int32_t* detail) {
  set_reason(detail, DSPARK_FB_NONE);
  if (!p || num_tokens < 0 || flags != 0) return DSPARK_E_INVALID;
  void* ws = nullptr;
  const int64_t need =
      dspark::plan_workspace_bytes(plan_for(p, num_tokens, commit_lens != nullptr));
  if (need > kStaticScratchBytes) {
    if (log_enabled())
      std::fprintf(stderr,
                   "dspark: dspark_ctx_kv_write_static: %lld workspace bytes needed, the static "
                   "scratch holds %lld\n",
                   (long long)need, (long long)kStaticScratchBytes);
    return DSPARK_E_TOO_LARGE;
  }
  if (need > 0 && num_tokens > 0) {
    const int st = scratch_on_current_device(&ws);
    if (st != DSPARK_OK) return st;
  }
  return write_impl(p, ctx_hidden, num_tokens, hidden_row_stride, positions, locs, commit_lens,
                    locs_row_width, num_requests, pools, num_pools, ws,
                    ws ? kStaticScratchBytes : 0, range_errors, flags, stream_ptr, detail);
}

int dspark_ctx_kv_write(const dspark_ctx_kv_pack* p, const void* ctx_hidden, int64_t num_tokens,
                        int64_t hidden_row_stride, const int64_t* positions, const int64_t* locs,
                        const int64_t* commit_lens, int64_t locs_row_width, int64_t num_requests,
                        const dspark_pool_desc* pools, int32_t num_pools, void* workspace,
                        int64_t workspace_bytes, unsigned long long* range_errors, uint32_t flags,
                        void* stream_ptr, int32_t* detail) {
  return write_impl(p, ctx_hidden, num_tokens, hidden_row_stride, positions, locs, commit_lens,
                    locs_row_width, num_requests, pools, num_pools, workspace, workspace_bytes,
                    range_errors, flags, stream_ptr, detail);
}

int dspark_table_qk_norm_rope(void* qkv, int64_t num_tokens, int64_t row_stride,
                              const int64_t* positions, int32_t num_q_heads, int32_t num_k_heads,
                              int32_t head_dim, int32_t act_dtype, const void* q_norm_weight,
                              const void* k_norm_weight, int32_t norm_weight_dtype, double eps,
                              const float* cos_sin, int64_t rope_max_pos,
                              unsigned long long* range_errors, void* stream_ptr,
                              int32_t* fallback_reason) {
  set_reason(fallback_reason, DSPARK_FB_NONE);
  if (num_tokens < 0 || num_q_heads <= 0 || num_k_heads <= 0 || head_dim <= 0)
    return DSPARK_E_INVALID;
  if (act_dtype != DSPARK_BF16 && act_dtype != DSPARK_FP16)
    return fallback(fallback_reason, DSPARK_FB_DTYPE);
  if (norm_weight_dtype != act_dtype && norm_weight_dtype != DSPARK_FP32)
    return fallback(fallback_reason, DSPARK_FB_DTYPE);
  if (head_dim != 64 && head_dim != 128) return fallback(fallback_reason, DSPARK_FB_SHAPE);
  const int64_t heads = (int64_t)num_q_heads + num_k_heads;
  if (row_stride < heads * head_dim || row_stride % 8 != 0) return DSPARK_E_INVALID;
  if (!(eps >= 0.0) || eps > 3.0e38) return DSPARK_E_INVALID;
  if (rope_max_pos <= 0) return DSPARK_E_INVALID;
  if (num_tokens == 0) return DSPARK_OK;
  if (!qkv || !positions || !q_norm_weight || !k_norm_weight || !cos_sin) return DSPARK_E_INVALID;
  const uintptr_t walign = 16;  // 8 weight entries (fp32: 2 x 16 bytes) per vector load
  if (reinterpret_cast<uintptr_t>(qkv) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(q_norm_weight) % walign != 0 ||
      reinterpret_cast<uintptr_t>(k_norm_weight) % walign != 0 ||
      reinterpret_cast<uintptr_t>(cos_sin) % 16 != 0)
    return DSPARK_E_INVALID;
  dspark::QkArgs a = {};
  a.qkv = static_cast<uint16_t*>(qkv);
  a.pos = positions;
  a.qw = q_norm_weight;
  a.kw = k_norm_weight;
  a.table = cos_sin;
  a.err = range_errors;
  a.T = num_tokens;
  a.row_stride = row_stride;
  a.P = rope_max_pos;
  a.NHQ = num_q_heads;
  a.NHT = (int32_t)heads;
  a.eps = (float)eps;
  const hipError_t e = dspark::launch_qk_norm_rope(a, head_dim, act_dtype == DSPARK_FP16,
                                                   norm_weight_dtype == DSPARK_FP32,
                                                   static_cast<hipStream_t>(stream_ptr));
  return e == hipSuccess ? DSPARK_OK : DSPARK_E_DEVICE;
}

int dspark_verify_accept(const int64_t* draft_tokens, int64_t draft_row_stride,
                         const int64_t* target_tokens, int64_t target_row_stride,
                         int64_t num_requests, int32_t num_drafts, int64_t* accept_lens,
                         int64_t* bonus_tokens, void* stream_ptr) {
  if (num_requests < 0 || num_drafts < 0) return DSPARK_E_INVALID;
  if (draft_row_stride < num_drafts || target_row_stride < (int64_t)num_drafts + 1)
    return DSPARK_E_INVALID;
  if (num_requests == 0) return DSPARK_OK;
  if ((num_drafts > 0 && !draft_tokens) || !target_tokens || !accept_lens || !bonus_tokens)
    return DSPARK_E_INVALID;
  dspark::VerifyArgs a = {};
  a.draft = draft_tokens;
  a.target = target_tokens;
  a.draft_stride = draft_row_stride;
  a.target_stride = target_row_stride;
  a.B = num_requests;
  a.accept = accept_lens;
  a.bonus = bonus_tokens;
  a.K = num_drafts;
  const hipError_t e =
      dspark::launch_verify_accept(a, static_cast<hipStream_t>(stream_ptr));
  return e == hipSuccess ? DSPARK_OK : DSPARK_E_DEVICE;
}

int dspark_pack_info(const dspark_ctx_kv_pack* p, int32_t* num_layers, int64_t* hidden,
                     int64_t* kv_size, int64_t* head_dim, int32_t* act_dtype, int32_t* has_bias) {
  if (!p) return DSPARK_E_INVALID;
  if (num_layers) *num_layers = p->num_layers;
  if (hidden) *hidden = p->hidden;
  if (kv_size) *kv_size = p->kv_size;
  if (head_dim) *head_dim = p->head_dim;
  if (act_dtype) *act_dtype = p->dtype;
  if (has_bias) *has_bias = p->has_bias;
  return DSPARK_OK;
}

int dspark_pack_buffers(const dspark_ctx_kv_pack* p, const void** w_stacked, const void** bias,
                        const float** k_norm) {
  if (!p) return DSPARK_E_INVALID;
  if (w_stacked) *w_stacked = p->w;
  if (bias) *bias = p->bias;
  if (k_norm) *k_norm = p->knw;
  return DSPARK_OK;
}

void dspark_pack_free(dspark_ctx_kv_pack* p) {
  if (!p) return;
  int cur = -1;
  (void)hipGetDevice(&cur);
  if (cur != p->device) (void)hipSetDevice(p->device);
  (void)hipDeviceSynchronize();
  free_pack(p);
  if (cur >= 0 && cur != p->device) (void)hipSetDevice(cur);
}

const char* dspark_status_str(int status) {
  switch (status) {
    case DSPARK_OK: return "ok";
    case DSPARK_FALLBACK: return "fallback: not eligible for the stacked write";
    case DSPARK_E_INVALID: return "invalid argument";
    case DSPARK_E_RANGE: return "position or slot out of range, or a slot written twice";
    case DSPARK_E_DEVICE: return "HIP runtime error";
    case DSPARK_E_NOMEM: return "device allocation failed";
    case DSPARK_E_TOO_LARGE: return "workspace needed exceeds the static scratch";
    default: return "unknown status";
  }
}

const char* dspark_fallback_str(int reason) {
  switch (reason) {
    case DSPARK_FB_NONE: return "none";
    case DSPARK_FB_NO_LAYERS: return "no layers";
    case DSPARK_FB_TOO_MANY_LAYERS: return "more layers than DSPARK_MAX_LAYERS";
    case DSPARK_FB_NOT_SLICEABLE: return "QKV weight cannot be sliced (quantized, other dtype or layout)";
    case DSPARK_FB_EPS_MISMATCH: return "layers disagree on the k_norm epsilon";
    case DSPARK_FB_MIXED_BIAS: return "QKV bias present in some layers only";
    case DSPARK_FB_SHAPE: return "head_dim / kv_size differ or are unsupported";
    case DSPARK_FB_DTYPE: return "unsupported activation or k_norm dtype";
    case DSPARK_FB_KV_SCALE: return "K/V quantization scale attached";
    case DSPARK_FB_ROPE: return "rotary is not neox full-dim over one shared fp32 table";
    case DSPARK_FB_POOL_LAYOUT: return "KV pool dtype, layout or alignment unsupported";
    default: return "unknown reason";
  }
}

const char* dspark_range_str(int cause) {
  switch (cause) {
    case DSPARK_RANGE_NONE: return "none";
    case DSPARK_RANGE_POSITION: return "a stored row's position is outside the rotary table";
    case DSPARK_RANGE_SLOT: return "a stored row's slot is past a layer's pool";
    case DSPARK_RANGE_DUPLICATE: return "two stored rows name the same slot";
    default: return "unknown cause";
  }
}

}  // extern "C"

// ------------------------------------------------------------ context producer

struct dspark_main_proj_pack {
  int device = -1;
  int num_cus = 0;
  int64_t out_features = 0;  // H
  int64_t in_features = 0;   // n * H
  int32_t dtype = DSPARK_BF16;
  float eps = 0.0f;
  uint16_t* w = nullptr;     // blocked projection weight
  float* g = nullptr;        // [H] fp32 norm weight
  uint16_t* zeros = nullptr;  // 256 zero bytes read by out-of-range K lanes
};

namespace {
void free_proj(dspark_main_proj_pack* p) {
  if (!p) return;
  (void)hipDeviceSynchronize();
  if (p->w) (void)hipFree(p->w);
  if (p->g) (void)hipFree(p->g);
  if (p->zeros) (void)hipFree(p->zeros);
  delete p;
}
}  // namespace

int dspark_pack_main_proj(const void* weight, int64_t out_features, int64_t in_features,
                          int64_t w_row_stride, int32_t w_dtype, const void* norm_weight,
                          int32_t norm_weight_dtype, double eps, int32_t act_dtype,
                          void* stream_ptr, dspark_main_proj_pack** out,
                          int32_t* fallback_reason) {
  set_reason(fallback_reason, DSPARK_FB_NONE);
  if (!out) return DSPARK_E_INVALID;
  *out = nullptr;
  if (!weight || !norm_weight || out_features <= 0 || in_features <= 0 ||
      w_row_stride < in_features || !(eps >= 0.0) || eps > 3.0e38)
    return DSPARK_E_INVALID;
  if (act_dtype != DSPARK_BF16 && act_dtype != DSPARK_FP16)
    return fallback(fallback_reason, DSPARK_FB_DTYPE);
  if (w_dtype != act_dtype) return fallback(fallback_reason, DSPARK_FB_NOT_SLICEABLE);
  if (norm_weight_dtype != act_dtype && norm_weight_dtype != DSPARK_FP32)
    return fallback(fallback_reason, DSPARK_FB_DTYPE);
  if (out_features % 128 != 0 || in_features % 8 != 0 || w_row_stride % 8 != 0 ||
      reinterpret_cast<uintptr_t>(weight) % 16 != 0)
    return fallback(fallback_reason, DSPARK_FB_SHAPE);
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  dspark_main_proj_pack* p = new (std::nothrow) dspark_main_proj_pack();
  if (!p) return DSPARK_E_NOMEM;
  if (hipGetDevice(&p->device) != hipSuccess ||
      hipDeviceGetAttribute(&p->num_cus, hipDeviceAttributeMultiprocessorCount, p->device) !=
          hipSuccess) {
    delete p;
    return DSPARK_E_DEVICE;
  }
  p->out_features = out_features;
  p->in_features = in_features;
  p->dtype = act_dtype;
  p->eps = (float)eps;
  const int64_t nk = (in_features + 63) / 64;
  uint16_t* plain = nullptr;
  auto fail = [&](int s) {
    if (plain) (void)hipFree(plain);
    free_proj(p);
    return s;
  };
  if (hipMalloc(&p->w, (size_t)(out_features * nk * 64 * 2)) != hipSuccess ||
      hipMalloc(&plain, (size_t)(out_features * in_features * 2)) != hipSuccess ||
      hipMalloc(&p->g, (size_t)(out_features * 4)) != hipSuccess ||
      hipMalloc(&p->zeros, 256) != hipSuccess)
    return fail(DSPARK_E_NOMEM);
  bool ok = hipMemcpy2DAsync(plain, (size_t)(in_features * 2), weight, (size_t)(w_row_stride * 2),
                             (size_t)(in_features * 2), (size_t)out_features,
                             hipMemcpyDeviceToDevice, stream) == hipSuccess;
  ok = ok && dspark::launch_block_weight(plain, out_features, in_features, p->w, stream) ==
                 hipSuccess;
  ok = ok && dspark::launch_widen_to_f32(norm_weight, norm_weight_dtype, p->g, out_features,
                                         stream) == hipSuccess;
  ok = ok && hipMemsetAsync(p->zeros, 0, 256, stream) == hipSuccess;
  ok = ok && hipStreamSynchronize(stream) == hipSuccess;
  if (!ok) return fail(DSPARK_E_DEVICE);
  (void)hipFree(plain);
  *out = p;
  return DSPARK_OK;
}

namespace {
// Workspace of one producer call: fp32 partial projections when the
// projection is split over K, else one fp32 sum of squares per 128-feature
// group and token.
int64_t proj_workspace_bytes(const dspark_main_proj_pack* p, int64_t T) {
  const int64_t groups = p->out_features / 128;
  const int ks = dspark::producer_ksplits(T, groups, p->in_features, p->out_features, p->num_cus);
  return (ks > 1 ? ks * p->out_features : groups) * T * (int64_t)sizeof(float);
}
}  // namespace

int dspark_main_proj_workspace_bytes(const dspark_main_proj_pack* p, int64_t num_tokens,
                                     int64_t* bytes) {
  if (!p || !bytes || num_tokens < 0) return DSPARK_E_INVALID;
  *bytes = proj_workspace_bytes(p, num_tokens);
  return DSPARK_OK;
}

int dspark_main_proj_norm(const dspark_main_proj_pack* p, const void* aux_hidden,
                          int64_t num_tokens, int64_t aux_row_stride, void* ctx_hidden,
                          int64_t ctx_row_stride, void* workspace, int64_t workspace_bytes,
                          void* stream_ptr) {
  if (!p || num_tokens < 0) return DSPARK_E_INVALID;
  if (num_tokens == 0) return DSPARK_OK;
  if (!aux_hidden || !ctx_hidden || !workspace) return DSPARK_E_INVALID;
  if (aux_row_stride < p->in_features || aux_row_stride % 8 != 0 ||
      ctx_row_stride < p->out_features || ctx_row_stride % 8 != 0 ||
      reinterpret_cast<uintptr_t>(aux_hidden) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(ctx_hidden) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return DSPARK_E_INVALID;
  const int64_t groups = p->out_features / 128;
  if (workspace_bytes < proj_workspace_bytes(p, num_tokens)) return DSPARK_E_INVALID;
  const int ks = dspark::producer_ksplits(num_tokens, groups, p->in_features, p->out_features,
                                          p->num_cus);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DSPARK_E_DEVICE;
  if (dev != p->device) return DSPARK_E_INVALID;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  dspark::WriteArgs a = {};
  a.x = static_cast<const uint16_t*>(aux_hidden);
  a.w = p->w;
  a.zeros = p->zeros;
  a.x_stride = aux_row_stride;
  a.T = num_tokens;
  a.H = (int32_t)p->in_features;
  a.R = groups;
  a.y = static_cast<uint16_t*>(ctx_hidden);
  a.y_stride = ctx_row_stride;
  a.partial = static_cast<float*>(workspace);
  a.ksplits = ks;
  const bool fp16 = p->dtype == DSPARK_FP16;
  if (dspark::launch_rows_out(a, fp16, p->num_cus, stream) != hipSuccess) return DSPARK_E_DEVICE;
  if (dspark::launch_row_norm(a.y, ctx_row_stride, a.partial, num_tokens, groups, ks, p->g,
                              p->eps, fp16, stream) != hipSuccess)
    return DSPARK_E_DEVICE;
  return DSPARK_OK;
}

void dspark_main_proj_free(dspark_main_proj_pack* p) { free_proj(p); }

// ------------------------------------------------------------ draft attention

namespace {
// Compute units of the current device, queried once per device.
int current_device_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cached[dev] = n;
  return n;
}

struct AttnPlan {
  int32_t row_tiles = 0;
  int32_t n_splits = 0;
  int64_t split_len = 32;
  int64_t bytes = 0;
};

// Key splits: enough waves for about 4 per compute unit at head_dim 128 and 8
// at 64 (a step of a 64-wide head requests half the lines), each split a
// multiple of 32 keys and at least 256 (fewer, longer splits when the batch
// alone fills the device). That keeps a CU's L1 request queue about full;
// more, shorter splits only add records to merge.
AttnPlan attn_plan(int64_t B, int32_t block, int32_t nhq, int32_t nhk, int32_t D,
                   int64_t max_prefix, int num_cus) {
  AttnPlan pl;
  const int64_t M = (int64_t)block * (nhq / nhk);
  pl.row_tiles = (int32_t)((M + 31) / 32);
  const int64_t base = B * nhk * pl.row_tiles;
  if (max_prefix > 0) {
    const int64_t target = (D <= 64 ? 8LL : 4LL) * (num_cus > 0 ? num_cus : 1);
    int64_t ns = base > 0 ? (target + base - 1) / base : 1;
    if (ns < 1) ns = 1;
    int64_t len = (max_prefix + ns - 1) / ns;
    len = (len + 31) / 32 * 32;
    if (len < 256) len = 256;
    pl.split_len = len;
    pl.n_splits = (int32_t)((max_prefix + len - 1) / len);
  }
  pl.bytes = base * (pl.n_splits + 1) * 32 * (int64_t)(D + 2) * (int64_t)sizeof(float);
  return pl;
}
}  // namespace

int dspark_draft_attention_workspace_bytes(int64_t num_requests, int32_t block,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int64_t max_prefix, int64_t* bytes) {
  if (!bytes || num_requests < 0 || block < 1 || num_q_heads < 1 || num_kv_heads < 1 ||
      num_q_heads % num_kv_heads != 0 || head_dim < 1 || max_prefix < 0)
    return DSPARK_E_INVALID;
  *bytes = attn_plan(num_requests, block, num_q_heads, num_kv_heads, head_dim, max_prefix,
                     current_device_cus())
               .bytes;
  return DSPARK_OK;
}

int dspark_draft_attention(const dspark_attn_desc* d, int64_t num_requests, int32_t block,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t act_dtype, double sm_scale, int64_t max_prefix,
                           void* workspace, int64_t workspace_bytes,
                           unsigned long long* range_errors, void* stream_ptr,
                           int32_t* fallback_reason) {
  set_reason(fallback_reason, DSPARK_FB_NONE);
  if (!d || num_requests < 0 || block < 1 || num_q_heads < 1 || num_kv_heads < 1 ||
      num_q_heads % num_kv_heads != 0 || max_prefix < 0 || !(sm_scale == sm_scale))
    return DSPARK_E_INVALID;
  if (act_dtype != DSPARK_BF16 && act_dtype != DSPARK_FP16)
    return fallback(fallback_reason, DSPARK_FB_DTYPE);
  if (head_dim != 64 && head_dim != 128) return fallback(fallback_reason, DSPARK_FB_SHAPE);
  if (num_requests == 0) return DSPARK_OK;
  auto al16 = [](const void* ptr) { return reinterpret_cast<uintptr_t>(ptr) % 16 == 0; };
  if (!d->q || !d->k_ext || !d->v_ext || !d->k_pool || !d->v_pool || !d->kv_indptr ||
      !d->kv_indices || !d->out || !workspace || d->num_slots < 1)
    return DSPARK_E_INVALID;
  const int64_t strides[] = {d->q_token_stride, d->q_head_stride, d->ext_token_stride,
                             d->ext_head_stride, d->pool_slot_stride, d->pool_head_stride,
                             d->out_token_stride, d->out_head_stride};
  for (int64_t st : strides)
    if (st < head_dim || st % 8 != 0) return DSPARK_E_INVALID;
  if (!al16(d->q) || !al16(d->k_ext) || !al16(d->v_ext) || !al16(d->k_pool) ||
      !al16(d->v_pool) || !al16(d->out) || !al16(workspace))
    return DSPARK_E_INVALID;
  const int cus = current_device_cus();
  if (cus <= 0) return DSPARK_E_DEVICE;
  const AttnPlan pl = attn_plan(num_requests, block, num_q_heads, num_kv_heads, head_dim,
                                max_prefix, cus);
  if (workspace_bytes < pl.bytes) return DSPARK_E_INVALID;
  dspark::AttnArgs a = {};
  a.q = static_cast<const uint16_t*>(d->q);
  a.k_ext = static_cast<const uint16_t*>(d->k_ext);
  a.v_ext = static_cast<const uint16_t*>(d->v_ext);
  a.k_pool = static_cast<const uint16_t*>(d->k_pool);
  a.v_pool = static_cast<const uint16_t*>(d->v_pool);
  a.kv_indptr = d->kv_indptr;
  a.kv_indices = d->kv_indices;
  a.out = static_cast<uint16_t*>(d->out);
  a.part = static_cast<float*>(workspace);
  a.err = range_errors;
  a.q_stride0 = d->q_token_stride;
  a.q_stride1 = d->q_head_stride;
  a.ext_stride0 = d->ext_token_stride;
  a.ext_stride1 = d->ext_head_stride;
  a.pool_stride0 = d->pool_slot_stride;
  a.pool_stride1 = d->pool_head_stride;
  a.out_stride0 = d->out_token_stride;
  a.out_stride1 = d->out_head_stride;
  a.num_slots = d->num_slots;
  a.B = num_requests;
  a.split_len = pl.split_len;
  a.max_prefix = max_prefix;
  a.block = block;
  a.nhk = num_kv_heads;
  a.G = num_q_heads / num_kv_heads;
  a.M = block * a.G;
  a.row_tiles = pl.row_tiles;
  a.n_splits = pl.n_splits;
  a.sm_scale = (float)sm_scale;
  const hipError_t e = dspark::launch_draft_attention(a, head_dim, act_dtype == DSPARK_FP16,
                                                      static_cast<hipStream_t>(stream_ptr));
  return e == hipSuccess ? DSPARK_OK : DSPARK_E_DEVICE;
}
