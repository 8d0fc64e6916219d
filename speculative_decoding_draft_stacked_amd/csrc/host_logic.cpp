// Host-side logic of the context-KV write library (no device access).
//
// Eligibility follows the fast-path-or-fallback pattern of sglang PR #31986
// ("_stacked_ctx_kv_params": sliceable weights, equal eps, consistent bias) and
// sglang PR #31847 ("_build_fused_kv_write_bundle": no K/V scale, equal head
// shape, neox full-dim rotary over one shared table, pool dtype and head-major
// layout). The window checks restate the argument checks of PR #31847's
// "fused_kv_norm_rope_write" (commit_lens and the window width come together;
// the window covers every row).
#include "host_logic.h"

#include <algorithm>
#include <vector>

namespace dspark {

namespace {

int fallback(int32_t* out, int32_t r) {
  if (out) *out = r;
  return DSPARK_FALLBACK;
}

bool is_act_dtype(int32_t d) { return d == DSPARK_BF16 || d == DSPARK_FP16; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kBN = 128;  // weight rows per row tile
constexpr int64_t kBK = 64;   // K columns per chunk

// K parts of the write's streaming kernel for `splits` token splits of `nb`
// 32-token blocks: only where row tiles x token splits leave at least half of
// the device idle (few weight tiles), with at least 8 chunks of 64 per part.
int write_ksplits(int64_t T, int64_t R, int64_t H, int64_t splits, int64_t nb, int num_cus) {
  if (T > kCompactMaxRows) return 1;
  if (R * splits * 2 > num_cus) return 1;
  const int64_t nk_all = ceil_div(H, kBK);
  int64_t ks = num_cus / (R * splits);
  if (ks > nk_all / 8) ks = nk_all / 8;
  if (ks > 16) ks = 16;
  if (ks < 2 || splits * 32 * nb > kRowMapInts) return 1;
  return (int)ks;
}

// A commit window whose rows need more token splits than one round of
// two-K-part workgroups holds: as many token splits of 128 slots as that
// round holds, when they take 3/4 of the window. The workgroups count the
// window's written rows first; when those do not fit the splits, the same
// workgroups keep K whole as splits x 2 token splits, which must hold every
// row. Returns the token splits, or 0 when this plan does not apply.
int64_t adaptive_splits(int64_t T, int64_t R, int64_t H, int num_cus) {
  constexpr int64_t kParts = 2, kSlots = 128;
  if (T > 2 * 512) return 0;  // the adaptive scan holds two rows per thread
  if (ceil_div(H, kBK) / 8 < kParts) return 0;
  const int64_t splits = num_cus / (R * kParts);
  if (splits < 1 || splits * kSlots >= T) return 0;
  if (splits * kSlots * 4 < 3 * T || splits * kParts * kSlots < T) return 0;
  if (splits * kSlots > kRowMapInts) return 0;
  return splits;
}

}  // namespace

int check_layers(const dspark_layer_desc* layers, int32_t num_layers, int64_t hidden,
                 int32_t act_dtype, int32_t* reason) {
  if (reason) *reason = DSPARK_FB_NONE;
  if (num_layers < 0 || hidden <= 0 || (num_layers > 0 && !layers)) return DSPARK_E_INVALID;
  if (num_layers == 0) return fallback(reason, DSPARK_FB_NO_LAYERS);
  if (num_layers > DSPARK_MAX_LAYERS) return fallback(reason, DSPARK_FB_TOO_MANY_LAYERS);
  if (!is_act_dtype(act_dtype)) return fallback(reason, DSPARK_FB_DTYPE);
  const dspark_layer_desc& l0 = layers[0];
  for (int32_t i = 0; i < num_layers; ++i) {
    const dspark_layer_desc& d = layers[i];
    if (!d.qkv_weight || !d.k_norm_weight) return DSPARK_E_INVALID;
    const bool sliceable = d.w_dtype == act_dtype && d.w_col_stride == 1 && d.q_size >= 0 &&
                           d.kv_size > 0 && d.w_rows >= d.q_size + 2 * d.kv_size &&
                           d.w_row_stride >= hidden;
    if (!sliceable) return fallback(reason, DSPARK_FB_NOT_SLICEABLE);
    if (d.k_norm_eps != l0.k_norm_eps) return fallback(reason, DSPARK_FB_EPS_MISMATCH);
    if (d.has_kv_scale) return fallback(reason, DSPARK_FB_KV_SCALE);
    if (d.head_dim != l0.head_dim || d.kv_size != l0.kv_size)
      return fallback(reason, DSPARK_FB_SHAPE);
    if (!d.rope_is_neox || d.rope_dim != d.head_dim || d.rope_dtype != DSPARK_FP32 ||
        !d.rope_cos_sin || d.rope_max_pos <= 0 || d.rope_max_pos != l0.rope_max_pos)
      return fallback(reason, DSPARK_FB_ROPE);
    if (d.k_norm_dtype != DSPARK_BF16 && d.k_norm_dtype != DSPARK_FP16 &&
        d.k_norm_dtype != DSPARK_FP32)
      return fallback(reason, DSPARK_FB_DTYPE);
  }
  for (int32_t i = 0; i < num_layers; ++i)
    if ((layers[i].qkv_bias != nullptr) != (l0.qkv_bias != nullptr))
      return fallback(reason, DSPARK_FB_MIXED_BIAS);
  const int64_t D = l0.head_dim;
  if ((D != 64 && D != 128) || l0.kv_size % D != 0 || hidden % 8 != 0 ||
      l0.w_row_stride % 8 != 0)
    return fallback(reason, DSPARK_FB_SHAPE);
  return DSPARK_OK;
}

bool write_window_ok(bool has_commit, int64_t num_tokens, int64_t locs_row_width,
                     int64_t num_requests) {
  if (num_tokens < 0) return false;
  if (has_commit != (locs_row_width > 0)) return false;
  if (has_commit) {
    if (num_requests < 0) return false;
    // num_requests * locs_row_width == num_tokens, without overflow
    if (num_requests != 0 && locs_row_width > num_tokens / num_requests) return false;
    return num_requests * locs_row_width == num_tokens;
  }
  return locs_row_width == 0 && num_requests == 0;
}

bool pool_layout_ok(const dspark_pool_desc& q, int32_t act_dtype, int64_t num_kv_heads,
                    int64_t head_dim) {
  const int64_t row = num_kv_heads * head_dim;
  return q.dtype == act_dtype && q.k_stride1 == head_dim && q.k_stride2 == 1 &&
         q.v_stride1 == head_dim && q.v_stride2 == 1 && q.k_stride0 >= row &&
         q.v_stride0 >= row && q.k_stride0 % 8 == 0 && q.v_stride0 % 8 == 0 &&
         reinterpret_cast<uintptr_t>(q.k) % 16 == 0 && reinterpret_cast<uintptr_t>(q.v) % 16 == 0;
}

WritePlan plan_write(int64_t T, int64_t R, int64_t H, bool has_commit, bool rows_out,
                     int num_cus) {
  WritePlan p;
  if (num_cus < 1) num_cus = 1;
  if (T <= 0 || R <= 0 || H <= 0) return p;
  const int64_t blocks = ceil_div(T, 32);
  const int64_t cap = R >= num_cus ? 1 : num_cus / R;
  if (blocks > 4 * cap) {
    // LDS-tiled kernel: 256 weight rows x bt tokens per workgroup; the token
    // tile with the fewest (rounds of workgroups over the device) x (tile
    // width), ties to the larger tile (fewer line requests per MFMA)
    const int64_t rp = ceil_div(R, 2);
    int64_t best_cost = -1;
    for (int bt : {256, 192, 128}) {
      const int64_t grid = rp * ceil_div(T, bt);
      const int64_t cost = ceil_div(grid, num_cus) * bt;
      if (best_cost < 0 || cost < best_cost) best_cost = cost, p.bt = bt;
    }
    p.kernel = kKernelTiled;
    p.splits = ceil_div(T, p.bt);
    p.grid = rp * p.splits;
    return p;
  }
  // Streaming kernel: row tiles x token splits of up to 4 blocks of 32 tokens,
  // one round of workgroups.
  int64_t splits = blocks < cap ? blocks : cap;
  int64_t nb = ceil_div(blocks, splits);
  splits = ceil_div(blocks, nb);
  int ks = 1;
  if (!rows_out) {
    // With K split over workgroups as well, fewer token splits (each weight
    // line requested by fewer workgroups) and more K parts cost less: the
    // K-split plan takes at most kKSplitTokenSplits splits of up to 4 blocks
    // and is used where that plan leaves at least half of the device idle.
    int64_t s2 = splits < kKSplitTokenSplits ? splits : kKSplitTokenSplits;
    if (ceil_div(blocks, 4) > s2) s2 = ceil_div(blocks, 4);
    const int64_t nb2 = ceil_div(blocks, s2);
    s2 = ceil_div(blocks, nb2);
    if (write_ksplits(T, R, H, s2, nb2, num_cus) > 1) {
      splits = s2;
      nb = nb2;
    }
    ks = write_ksplits(T, R, H, splits, nb, num_cus);
    if (ks == 1 && has_commit && T <= kCompactMaxRows) {
      const int64_t s3 = adaptive_splits(T, R, H, num_cus);
      if (s3 > 0) {
        splits = s3;
        nb = 4;
        ks = 2;
        p.adaptive = true;
      }
    }
  }
  p.nb = (int32_t)nb;
  p.splits = splits;
  p.compacts = has_commit && !rows_out && T <= kCompactMaxRows;
  if (ks > 1) {
    p.kernel = kKernelStreamKSplit;
    p.ksplits = ks;
    // the token splits of one (row tile, K part) slice run 8 workgroups
    // apart (one XCD); the grid is padded to whole groups of 8 slices
    p.grid = ceil_div(R * ks, 8) * 8 * splits;
    p.reduce_grid = R * splits * nb;
    p.part_floats = (int64_t)ks * R * splits * 32 * nb * kBN;
    p.rowmap_ints = kRowMapInts;
  } else {
    p.kernel = kKernelStream;
    p.grid = R * splits;
  }
  return p;
}

int64_t plan_workspace_bytes(const WritePlan& p) {
  if (p.kernel != kKernelStreamKSplit) return 0;
  return p.part_floats * 4 + p.rowmap_ints * 4;
}

int64_t max_write_workspace_bytes(int num_cus) {
  if (num_cus < 1) num_cus = 1;
  return (int64_t)num_cus * kBN * kBN * 4 + kRowMapInts * 4;
}

int producer_ksplits(int64_t T, int64_t R, int64_t in_features, int64_t out_features,
                     int num_cus) {
  // Split K only where the small-T path would run (so that the grid is one
  // round) and 128-token tiles alone leave the device under-filled; the row
  // norm then holds a row in registers (<= 8192 features, a multiple of 512:
  // four waves of whole 128-feature passes).
  if (num_cus < 1) num_cus = 1;
  const int64_t cap = R >= num_cus ? 1 : num_cus / R;
  const int64_t blocks32 = ceil_div(T, 32);
  if (blocks32 > 4 * cap || out_features > 8192 || out_features % 512 != 0) return 1;
  const int64_t tiles = R * ceil_div(T, 128);
  if (tiles >= num_cus) return 1;
  int64_t ks = num_cus / tiles;
  const int64_t nk = ceil_div(in_features, kBK);
  if (ks > nk / 8) ks = nk / 8;  // at least 8 chunks of 64 per part
  if (ks > 16) ks = 16;
  return ks < 2 ? 1 : (int)ks;
}

int check_rows(const int64_t* positions, const int64_t* locs, const int64_t* commit_lens,
               int64_t T, int64_t W, int64_t P, const int64_t* num_slots, int32_t L,
               int32_t* cause, int64_t* row) {
  if (cause) *cause = DSPARK_RANGE_NONE;
  if (row) *row = -1;
  if (T <= 0) return DSPARK_OK;
  int64_t min_slots = INT64_MAX;
  for (int32_t l = 0; l < L; ++l) min_slots = std::min(min_slots, num_slots[l]);
  auto fail = [&](int32_t c, int64_t t) {
    if (cause) *cause = c;
    if (row) *row = t;
    return DSPARK_E_RANGE;
  };
  std::vector<std::pair<int64_t, int64_t>> written;  // (slot, row) of the stored rows
  written.reserve((size_t)T);
  for (int64_t t = 0; t < T; ++t) {
    const int64_t loc = locs[t];
    bool valid = loc >= 0;
    if (commit_lens) valid = valid && (t % W) < commit_lens[t / W];
    if (!valid) continue;
    if (positions[t] < 0 || positions[t] >= P) return fail(DSPARK_RANGE_POSITION, t);
    if (loc >= min_slots) return fail(DSPARK_RANGE_SLOT, t);
    written.emplace_back(loc, t);
  }
  std::sort(written.begin(), written.end());
  for (size_t i = 1; i < written.size(); ++i)
    if (written[i].first == written[i - 1].first)
      return fail(DSPARK_RANGE_DUPLICATE, written[i].second);
  return DSPARK_OK;
}

}  // namespace dspark
