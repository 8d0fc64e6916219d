// Host-side logic of the library that touches no device: eligibility of a set
// of layers, argument checks of the write, the write's launch plan, the
// workspace it needs, the producer's K split, and the validate mode's row
// checks. Plain C++ (no HIP), so the CPU tests also build it with the address
// and undefined-behaviour sanitizers.
#pragma once

#include <stdint.h>

#include "../../include/dspark.h"

namespace dspark {

// Eligibility of the layers for the stacked write (the body of
// dspark_check_eligibility): DSPARK_OK, DSPARK_FALLBACK with *reason, or
// DSPARK_E_INVALID.
int check_layers(const dspark_layer_desc* layers, int32_t num_layers, int64_t hidden,
                 int32_t act_dtype, int32_t* reason);

// Argument pairing of a write (commit_lens with locs_row_width, B * W == T,
// no window fields without commit_lens): true when consistent.
bool write_window_ok(bool has_commit, int64_t num_tokens, int64_t locs_row_width,
                     int64_t num_requests);

// Pool layout the kernels support for one layer (dtype, head-major rows,
// 16-byte aligned bases and rows).
bool pool_layout_ok(const dspark_pool_desc& q, int32_t act_dtype, int64_t num_kv_heads,
                    int64_t head_dim);

// Which write kernels run, on what grid. Row tiles are 128 weight rows.
enum WriteKernel : int32_t {
  kKernelStream = DSPARK_KERNEL_STREAM,
  kKernelStreamKSplit = DSPARK_KERNEL_STREAM_KSPLIT,
  kKernelTiled = DSPARK_KERNEL_TILED,
};

struct WritePlan {
  int32_t kernel = kKernelStream;
  int32_t nb = 1;           // streaming: 32-token blocks per token split
  int64_t splits = 1;       // streaming: token splits; tiled: token tiles
  int32_t ksplits = 1;      // streaming: K parts over workgroups (1: none)
  int32_t bt = 0;           // tiled: tokens per workgroup tile
  int64_t grid = 0;         // workgroups of the main launch
  int64_t reduce_grid = 0;  // workgroups of the K-part reduce (0: none)
  bool compacts = false;    // commit-window rows numbered and projected only when written
  int64_t part_floats = 0;  // workspace: fp32 K-part sums
  int64_t rowmap_ints = 0;  // workspace: committed-row map of the token splits
  // streaming, compacted, K split: the workgroups keep K whole (splits x
  // ksplits token splits, no part sums) when the written rows do not fit
  // `splits` token splits; decided on the device
  bool adaptive = false;
};

// Commit windows of at most this many rows are compacted by the streaming
// kernel (every workgroup scans the window once per 512 rows).
constexpr int64_t kCompactMaxRows = 1024;
// Token splits of the K-split plan (each of at most 4 blocks of 32 tokens).
constexpr int64_t kKSplitTokenSplits = 4;
// Row-map entries of the K-split plan (token splits x tokens per split).
constexpr int64_t kRowMapInts = 2048;

// The plan of a write (or, with rows_out, of the producer's projection when
// its K is not split) of T tokens against R row tiles over H columns.
WritePlan plan_write(int64_t T, int64_t R, int64_t H, bool has_commit, bool rows_out,
                     int num_cus);

// Workspace bytes of a plan (16-byte multiple; 0 when it needs none).
int64_t plan_workspace_bytes(const WritePlan& p);

// Largest workspace any write plan needs on a device of num_cus compute units:
// at most one K part of a 128-row x 128-token tile per compute unit, plus the
// row map.
int64_t max_write_workspace_bytes(int num_cus);

// K parts the producer's projection is split into (1: none).
int producer_ksplits(int64_t T, int64_t R, int64_t in_features, int64_t out_features,
                     int num_cus);

// Validate mode: checks the rows a write would store (loc >= 0 and, with
// commit_lens, inside the committed prefix) for a position outside [0, P),
// a slot at or past any layer's num_slots, and a slot named by two such rows.
// Returns DSPARK_OK, or DSPARK_E_RANGE with *cause (DSPARK_RANGE_*) and *row
// (the first offending row; for a duplicate, the later of the two) set.
int check_rows(const int64_t* positions, const int64_t* locs, const int64_t* commit_lens,
               int64_t T, int64_t W, int64_t P, const int64_t* num_slots, int32_t L,
               int32_t* cause, int64_t* row);

}  // namespace dspark
