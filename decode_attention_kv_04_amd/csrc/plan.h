// Host-side planning for paged decode attention. Pure C++ (no HIP headers):
// it decides how each sequence's attended context is cut into splits and how
// large the workspace of per-split states is.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "decode_attn.h"

struct da_plan {
  da_params p;
  int32_t group = 1;           // G = H_q / H_kv
  int32_t group_tile = 1;      // compiled group width the kernels use (1, 2, 4 or 8)
  int32_t split_kernel = 0;    // 0 = vector q.K, 1 = q.K on the matrix cores, 2 = multi-token
  int32_t num_cus = 0;
  int32_t pages_per_split = 1; // c (fixed-order mode: pages per chunk)
  int32_t max_splits = 1;      // S_max: state slots per query head (fixed-order mode: chunks)
  int32_t chunks_per_group = 0;// fixed-order mode: chunks per split work-group (0 = default mode)
  int32_t split_groups = 1;    // split work-groups per (sequence, KV head): the grid's y extent
  int32_t query_len = 1;       // T new tokens per sequence
  int32_t rows_per_group = 0;  // multi-token kernel: (token, head) rows per work-group
  bool per_token = false;      // T > 1 on the single-query kernels, one launch per token
  bool balanced = false;       // balanced schedule: split_groups work-groups of pages_per_split units each
  bool fixed_multi = false;    // fixed-order mode on the multi-token kernel: one chunk (split) per work-group
  int32_t bal_overhead = 0;    // balanced schedule: units a stream weighs before its pages
  std::vector<int32_t> splits; // S_b per sequence
  int64_t active_units = 0;
  int64_t attended_keys = 0;
  size_t ws_o_offset = 0;      // [B][H_q][S_max][D] float
  size_t ws_ml_offset = 0;     // [B][H_q][S_max][2] float (m, l) after the O block
  size_t ws_cnt_offset = 0;    // balanced schedule: [B][H_kv] int32 pieces per stream, after (m, l)
  size_t ws_bytes = 0;
};

namespace da {

// Attended keys [t0, L) and attended pages [pf, pe) of one sequence.
struct SeqRange {
  int64_t t0, t1;
  int64_t pf, pe;
};
SeqRange seq_range(int64_t L, int64_t window, int64_t P);

// Group width compiled for a GQA group size (0 if none is).
int32_t group_tile_for(int32_t G);

// Whether the matrix-core split kernel covers these parameters.
bool matrix_kernel_supported(const da_params& p);

// Largest batch the balanced schedule takes (its work-groups keep the
// batch's page prefix sums in LDS).
constexpr int32_t kBalancedMaxBatch = 4096;

// Validate parameters and lengths and build a plan for `num_cus` compute
// units. On success *out owns a new plan.
da_status make_plan(const da_params* p, const int32_t* host_seq_lens, int32_t num_cus, da_plan** out);

}  // namespace da
