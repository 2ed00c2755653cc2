// Host planner: validation, split choice and workspace size.
//
// The split choice follows the two passages that pick a path on the host: the
// sharded nest is chosen from the page count and only above 256 tokens (TVM
// pull 20426, commit message and PR description), and the split threshold is
// a knob with a 256-token default (mlx-runner pull 3, GQA-shared split
// attention commit). Here the host picks one split length c (in pages) for the
// whole batch from the attended page count and the compute-unit count, so
// that the split pass launches a few work-groups per compute unit; contexts
// of at most one split run in a single pass and write their output directly.
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <new>

namespace da {

namespace {

// Splits per KV head are sized so the split pass has about this many
// work-groups per compute unit in total.
constexpr int64_t kTargetGroupsPerCu = 9;
// The multi-token kernel is fastest with one round of resident work-groups,
// so each row block's keys are split only as far as needed to fill that
// round, sized by the longest sequence (a sweep of split counts on 16..512-
// token suffixes over 0.5-8k-token contexts; and on the 4-token check over
// the long batch: 2 splits per sequence, one round of 64-row blocks, 535 us;
// 3 per sequence 591 us, the last round partly empty; 4 per sequence 548 us).
// Resident work-groups per compute unit, from those sweeps: 64-row blocks
// 4 at head_dim 64 and 2 at 128 (the 4-token checks: 4 and 2 splits per
// sequence best, 5 and 3 lose 11 %); 128-row blocks 3 at head_dim 64 and 2
// at 128; 2 at 256 (64-row blocks only).
int64_t resident_row_groups_per_cu(int32_t head_dim, int64_t rows) {
  if (head_dim == 64) return rows == 128 ? 3 : 4;
  return 2;
}
// Rows per block at head_dim 64 and 128 above 64 rows: 128 (two 16-row
// groups per wave sharing every K/V operand read) measured 15 % faster than
// 64 at head_dim 128 on 128- and 512-token suffixes (GQA 4: 512 and 2048
// rows), and on the 32-token suffix (128 rows) 33.9 against 39.8 us. Blocks
// of 16 rows or fewer (a few drafted tokens) take 16 rows at every head_dim:
// wave 0 computes them and the other waves only copy (64-row blocks would
// compute the empty rows on zero q). 17 to 64 rows take 64-row blocks, at
// every head_dim: against 128-row blocks at head_dim 128, a decode step at
// 48 query heads over one KV head, 32 x 1-8k tokens 24.4 -> 21.4 us, 32 over
// 2 heads 38.6 -> 34.1; a 4-token check at 64 over 8 heads over the long
// batch 570.9 -> 526.0, 8 tokens at 32 over 8, 32 x 1-8k 131.3 -> 118.3, a
// 16-token suffix 36.3 -> 33.8; and twice as fast as 16-row blocks
// re-reading the keys for each. At head_dim 256 blocks are 64 rows, or 16.
// da_params.rows_per_block (validated by make_plan) forces a size.
int64_t mq_rows(int64_t rows, int32_t head_dim, int32_t forced) {
  if (forced > 0) return forced;
  if (rows <= 16) return 16;
  if (rows <= 64) return 64;
  return head_dim <= 128 ? 128 : 64;
}
// A split never holds fewer attended tokens than this (the pages' 256-token
// switch-over: a dispatch whose contexts are all this short is not split);
// DECODE_ATTN_SPLIT_MIN overrides it.
constexpr int64_t kDefaultMinSplitTokens = 256;
// On the matrix-core decode kernel, once the longest attended context is
// above the switch-over, splits may be this short (3060-token Llama-8B decode
// shape: 10.8 -> 10.2 us per step with 128-token splits, 10.2 with 192;
// the vector kernel at head_dim 256 lost with them, 14.2 -> 17.0 us).
constexpr int64_t kMatrixMinSplitTokens = 128;

bool split_min_env(int64_t* v) {
  const char* s = std::getenv("DECODE_ATTN_SPLIT_MIN");
  if (s && *s) {
    char* end = nullptr;
    long x = std::strtol(s, &end, 10);
    if (end && *end == '\0' && x >= 1) {
      *v = x;
      return true;
    }
  }
  return false;
}

int64_t min_split_tokens() {
  int64_t v;
  return split_min_env(&v) ? v : kDefaultMinSplitTokens;
}

// Minimum split length of a single-query plan (decode or per-token mode).
int64_t decode_min_split_tokens(bool matrix_kernel, int64_t max_attended_tokens) {
  int64_t v;
  if (split_min_env(&v)) return v;
  if (matrix_kernel && max_attended_tokens > kDefaultMinSplitTokens) return kMatrixMinSplitTokens;
  return kDefaultMinSplitTokens;
}

// Minimum split length of a decode step on the multi-token kernel: past the
// switch-over, splits may be 64 tokens (µs per step, 64 / 128 / 256-token
// minimum: 64 query heads over 8 KV heads at 1 x 3060 tokens 9.9 / 11.0 /
// 12.1, 4 x 1024 10.1 / 9.8 / 11.5; 32 over 8 at head_dim 256 and 1 x 3060
// 11.9 / 13.3 / 15.3; longer batches fill the chip with longer splits).
constexpr int64_t kMultiDecodeMinSplitTokens = 64;

int64_t multi_decode_min_split_tokens(int64_t max_attended_tokens) {
  int64_t v;
  if (split_min_env(&v)) return v;
  return max_attended_tokens > kDefaultMinSplitTokens ? kMultiDecodeMinSplitTokens : kDefaultMinSplitTokens;
}

bool log_enabled() {
  const char* s = std::getenv("DECODE_ATTN_LOG");
  return s && s[0] == '1';
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool valid_dtype(da_dtype t) { return t == DA_F32 || t == DA_F16 || t == DA_BF16; }

// Balance of a multi-token plan: its longest work-group should stream at
// most 1/kMultiBalanceShare of the batch's page-heads. One work-group alone
// streams about 31 GB/s (four 32768-token contexts among 60 short ones,
// 64/8 heads: 32 work-groups of 16 MB in 537 us), the chip about 6.4 TB/s,
// so beyond that share the longest work-groups, not HBM, set the time (that
// batch: 537 us against 160 on the decode kernel's balanced schedule; 15
// short contexts and one of 65536 tokens: 268 against 85 with a split count
// per stream). A decode step that cannot be balanced runs on the decode
// kernels; several tokens take the limit itself as their split.
constexpr int64_t kMultiBalanceShare = 170;

// Shortest split (at least cmin pages) whose working work-groups, ceil(pages
// / c) for every block of `npages` on each of H KV heads, fit `slots`; the
// longest block's page count when no split fits. An empty block's work-group
// exits at once and holds no slot. The count of work-groups never grows with
// c, so a bisection finds it.
int64_t fit_split_pages(const std::vector<int64_t>& npages, int64_t H, int64_t slots, int64_t cmin, int64_t max_np) {
  auto groups = [&](int64_t cc) {
    int64_t n = 0;
    for (int64_t np : npages) n += ceil_div(np, cc);
    return n * H;
  };
  int64_t lo = std::min(cmin, max_np), hi = max_np;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (groups(mid) <= slots)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

// Largest split (pages) a balanced multi-token plan gives one work-group:
// 1/kMultiBalanceShare of the blocks' page-heads, or the minimum split.
int64_t balance_limit(const std::vector<int64_t>& npages, int64_t H, int64_t cmin) {
  int64_t total = 0;
  for (int64_t n : npages) total += n;
  return std::max(cmin, ceil_div(total * H, kMultiBalanceShare));
}

// Split length (pages) of a decode step on the multi-token kernel for the
// attended page counts `npages`, or 0 where that kernel would leave the
// batch unbalanced (the decode kernels then run). First the largest split
// count per stream that keeps every stream's work-groups within one round of
// resident work-groups (a round and a fraction measured worst: 24 x 4096
// tokens at 32/8 heads, 2 / 3 / 4 splits per stream 67.7 / 74.5 / 65.8 us,
// 12 x 2048 5 / 6 splits 20.5 / 23.7 us). With `fit`, where that leaves the
// longest work-groups too long, the shortest split whose working
// work-groups, ceil(pages / c) per stream, fit the round (the 65536-token
// context among 15 short ones: 67 us against 85 on the decode kernel; on
// batches of 1-8k tokens it ran 4-7 % slower than the count per stream, so
// it is only the second choice). Without `decode_kernels` (a group width
// they are not built for) an unbalanced plan takes the limit itself.
int64_t multi_decode_split_pages(const std::vector<int64_t>& npages, int64_t num_kv_heads, int64_t num_cus,
                                 int32_t head_dim, int64_t P, bool fit, bool decode_kernels = true) {
  int64_t max_np = 0;
  for (int64_t n : npages) max_np = std::max(max_np, n);
  if (max_np == 0) return 1;
  const int64_t slots = num_cus * resident_row_groups_per_cu(head_dim, 16);
  // Streams with keys: an empty one's work-group exits at once.
  int64_t nonempty = 0;
  for (int64_t n : npages) nonempty += n > 0 ? 1 : 0;
  const int64_t blocks = nonempty * num_kv_heads;
  const int64_t cmin = std::min(max_np, ceil_div(multi_decode_min_split_tokens(max_np * P), P));
  const int64_t limit = balance_limit(npages, num_kv_heads, cmin);
  const int64_t per_stream = std::max<int64_t>(1, slots / blocks);
  const int64_t c = std::min(max_np, std::max(cmin, ceil_div(max_np, per_stream)));
  if (c <= limit) return c;
  if (!fit) return 0;
  const int64_t f = fit_split_pages(npages, num_kv_heads, slots, cmin, max_np);
  if (f <= limit) return f;
  // No decode kernel for this group width: the limit itself, as for several
  // tokens (more than one round of work-groups).
  return decode_kernels ? 0 : limit;
}

}  // namespace

SeqRange seq_range(int64_t L, int64_t window, int64_t P) {
  SeqRange r;
  r.t1 = L;
  r.t0 = (window > 0 && L > window) ? L - window : 0;
  if (L == 0) {
    r.pf = r.pe = 0;
  } else {
    r.pf = r.t0 / P;
    r.pe = ceil_div(L, P);
  }
  return r;
}

bool matrix_kernel_supported(const da_params& p) {
  return p.head_dim == 128 && (p.kv_dtype == DA_F16 || p.kv_dtype == DA_BF16) && p.q_dtype == p.kv_dtype &&
         p.page_size % 16 == 0;
}

int32_t group_tile_for(int32_t G) {
  if (G == 1) return 1;
  if (G == 2) return 2;
  if (G >= 3 && G <= 4) return 4;
  if (G >= 5 && G <= 8) return 8;
  return 0;
}

namespace {

// Pages per split that give the split pass about `per_cu` work-groups per
// compute unit (kTargetGroupsPerCu by default), at least min_tokens.
int64_t heuristic_split_pages(int64_t total_np, int64_t max_np, int64_t num_kv_heads, int64_t num_cus, int64_t P,
                              int64_t min_tokens, int64_t per_cu = kTargetGroupsPerCu) {
  const int64_t work = total_np * num_kv_heads;  // page-heads to stream
  const int64_t target = num_cus * per_cu;
  int64_t c = ceil_div(work, target);
  c = std::max(c, ceil_div(min_tokens, P));
  return std::min(c, max_np);
}

// Workspace: O block [B][H_q][S_max][D] then (m, l) block [B][H_q][S_max][2].
void size_workspace(da_plan* plan) {
  const da_params& p = plan->p;
  const size_t rows = static_cast<size_t>(p.batch) * p.num_q_heads * plan->max_splits * plan->query_len;
  plan->ws_o_offset = 0;
  plan->ws_ml_offset = plan->ws_o_offset + round_up(rows * p.head_dim * sizeof(float), 256);
  plan->ws_bytes = plan->ws_ml_offset + round_up(rows * 2 * sizeof(float), 256);
}

void log_plan(const da_plan* plan) {
  if (!log_enabled()) return;
  const da_params& p = plan->p;
  std::fprintf(stderr,
               "decode_attn plan: B=%d Hq=%d Hkv=%d D=%d P=%d W=%d kernel=%s cus=%d pages/split=%d "
               "max_splits=%d split_groups=%d chunks/group=%d balanced=%d units=%lld keys=%lld ws=%zu\n",
               p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.page_size, p.window,
               plan->split_kernel ? "matrix" : "vector", plan->num_cus, plan->pages_per_split, plan->max_splits,
               plan->split_groups, plan->chunks_per_group, plan->balanced ? 1 : 0,
               static_cast<long long>(plan->active_units),
               static_cast<long long>(plan->attended_keys), plan->ws_bytes);
}

// Resident work-groups per compute unit of the matrix-core decode kernel's
// balanced-schedule instances, by compiled group width: 188-240 registers
// per lane at widths 1, 2 and 4 (two waves per SIMD of 512), 298-306 at 8
// (one); LDS 35-49 KB per work-group.
int64_t matrix_groups_per_cu(int32_t group_tile) { return group_tile == 8 ? 1 : 2; }

// Balanced schedule (matrix-core decode kernel, the planner's choice when no
// split count is forced and the split-length heuristic would need more than
// one round of resident work-groups). The batch's work is its (sequence, KV
// head) streams in order, each weighing kBalancedOverheadBytes worth of
// units for starting a piece (reading its length, q and first page id, and
// merging the waves at the end: a few dependent memory round trips) and then
// one unit per attended page (an empty stream one page, so that its zero rows
// get written). Work-group w takes units [w q, (w + 1) q): one round of
// resident work-groups with the same weight each, so no work-group waits for
// a slot and none is left running alone at the end. A stream cut by
// work-group boundaries leaves one state per piece for the combine; the
// work-group holding a stream's first page records its piece count.
// Measured before this schedule (same machine, split pass): the mixed-window
// batch's long sequences alone in 512 equal work-groups 83.3 us against 89.0
// us with the split-length heuristic; the long batch 477-485 us with 2-4
// splits against 491 us; one 32768-token sequence 24 us with 32-64 splits
// against 30 us with 256 (and the combine 5-6 against 17 us). Without the
// start weight, the mixed-window batch slowed from 96 to 128 us: a
// work-group whose share fell among short sequences started ~10 pieces.
constexpr int64_t kBalancedOverheadBytes = 64 << 10;

da_status finish_balanced_plan(da_plan* plan, const std::vector<int64_t>& npages, int64_t max_np) {
  const da_params& p = plan->p;
  const int64_t H = p.num_kv_heads;
  const int64_t P = p.page_size;
  const int64_t page_head_bytes = 2 * P * p.head_dim * (p.kv_dtype == DA_F32 ? 4 : 2);  // K and V
  const int64_t ov = ceil_div(kBalancedOverheadBytes, page_head_bytes);
  int64_t U = 0;
  for (int64_t n : npages) U += (ov + std::max<int64_t>(1, n)) * H;
  const int64_t slots = static_cast<int64_t>(plan->num_cus) * matrix_groups_per_cu(plan->group_tile);
  const int64_t min_pages = ceil_div(decode_min_split_tokens(true, max_np * P), P);
  const int64_t q = std::max(ceil_div(U, slots), min_pages);
  plan->balanced = true;
  plan->bal_overhead = static_cast<int32_t>(ov);
  plan->pages_per_split = static_cast<int32_t>(q);
  plan->split_groups = static_cast<int32_t>(ceil_div(U, q));
  plan->active_units = plan->split_groups;
  plan->splits.assign(p.batch, 1);
  int64_t smax = 1, start = 0;
  for (int32_t b = 0; b < p.batch; ++b) {
    const int64_t n = std::max<int64_t>(1, npages[b]);
    for (int64_t j = 0; j < H; ++j, start += ov + n) {
      const int64_t first_page = start + ov;
      const int64_t pieces = (first_page + n - 1) / q - first_page / q + 1;
      plan->splits[b] = static_cast<int32_t>(std::max<int64_t>(plan->splits[b], pieces));
      smax = std::max(smax, pieces);
    }
  }
  plan->max_splits = static_cast<int32_t>(smax);
  if (smax > 1) {
    size_workspace(plan);
    plan->ws_cnt_offset = plan->ws_bytes;
    plan->ws_bytes += round_up(static_cast<size_t>(p.batch) * H * sizeof(int32_t), 256);
  }
  log_plan(plan);
  return DA_OK;
}

// Fixed-order mode: chunks of fixed_chunk / P pages from each sequence's
// first attended page; a state slot per chunk; each split work-group takes
// chunks_per_group consecutive chunks; the combine always runs.
da_status finish_fixed_plan(da_plan* plan, const std::vector<int64_t>& npages, int64_t max_np, int64_t total_np) {
  const da_params& p = plan->p;
  const int64_t cp = p.fixed_chunk / p.page_size;
  int64_t max_chunks = 1;
  for (int64_t n : npages) max_chunks = std::max(max_chunks, ceil_div(n, cp));
  if (max_chunks > INT32_MAX / 2) {
    delete plan;
    return DA_ERR_UNSUPPORTED;
  }
  int64_t cpg;
  if (p.num_splits > 0) {
    cpg = ceil_div(max_chunks, std::min<int64_t>(p.num_splits, max_chunks));
  } else {
    // Each work-group takes just enough consecutive chunks to reach the
    // minimum split length (usually one): a work-group restarts its loads at
    // every chunk, and with one chunk each the other resident work-groups
    // hide that start. Long batch, 1024-token chunks: 534 us with the
    // decode target of 9 work-groups per CU (3 chunks each), 519 us with
    // one; 512-token chunks 577 -> 542 us.
    const int64_t min_pages = ceil_div(decode_min_split_tokens(plan->split_kernel == 1, max_np * p.page_size),
                                       p.page_size);
    cpg = std::min(max_chunks, std::max<int64_t>(1, ceil_div(min_pages, cp)));
  }
  cpg = std::max(cpg, ceil_div(max_chunks, 65535));  // the grid's y extent
  plan->pages_per_split = static_cast<int32_t>(cp);
  plan->max_splits = static_cast<int32_t>(max_chunks);
  plan->chunks_per_group = static_cast<int32_t>(cpg);
  plan->split_groups = static_cast<int32_t>(ceil_div(max_chunks, cpg));
  plan->splits.resize(p.batch);
  for (int32_t b = 0; b < p.batch; ++b) {
    const int64_t nc = std::max<int64_t>(1, ceil_div(npages[b], cp));
    plan->splits[b] = static_cast<int32_t>(nc);
    plan->active_units += ceil_div(nc, cpg) * p.num_kv_heads;
  }
  size_workspace(plan);
  log_plan(plan);
  return DA_OK;
}

// Several new tokens per sequence: rows (token, head) of one KV head are cut
// into blocks of rows_per_group; a block sees keys from the window start of
// its first token to its last token, and those pages are split with one split
// length for the whole batch.
da_status finish_multi_plan(da_plan* plan, const int32_t* lens, int64_t decode_pages, bool unsplit) {
  // decode_pages > 0: a decode step's split length, or (fixed_multi) the
  // fixed-order chunk in pages, which num_splits does not change. unsplit:
  // whole streams, one split per row block.
  const da_params& p = plan->p;
  const int64_t P = p.page_size;
  const int64_t T = plan->query_len;
  const int64_t G = plan->group;
  const int64_t R = T * G;
  // Four waves of 16 rows (or two groups of 16) share each key tile.
  const int64_t QB = mq_rows(R, p.head_dim, p.rows_per_block);
  const int64_t nrb = ceil_div(R, QB);
  plan->split_kernel = 2;
  plan->rows_per_group = static_cast<int32_t>(QB);
  plan->attended_keys = 0;  // counted per new token below
  if (nrb > 65535) {
    delete plan;
    return DA_ERR_UNSUPPORTED;
  }
  // Attended pages of every (sequence, row block).
  std::vector<int64_t> blk_pages(static_cast<size_t>(p.batch) * nrb);
  int64_t max_np = 0, total_np = 0;
  for (int32_t b = 0; b < p.batch; ++b) {
    const int64_t L = lens[b];
    for (int64_t rb = 0; rb < nrb; ++rb) {
      const int64_t r0 = rb * QB, r1 = std::min(R, r0 + QB) - 1;
      const int64_t hi = L - T + r1 / G + 1;
      const int64_t lo = p.window > 0 ? std::max<int64_t>(0, L - T + r0 / G + 1 - p.window) : 0;
      const int64_t np = ceil_div(hi, P) - lo / P;
      blk_pages[b * nrb + rb] = np;
      max_np = std::max(max_np, np);
      total_np += np;
    }
    for (int64_t t = 0; t < T; ++t) {
      const int64_t pos = L - T + t;
      plan->attended_keys += p.window > 0 ? std::min<int64_t>(pos + 1, p.window) : pos + 1;
    }
  }
  int64_t c;
  if (max_np == 0) {
    c = 1;
  } else if (plan->fixed_multi) {
    c = decode_pages;
  } else if (p.num_splits > 0) {
    c = ceil_div(max_np, p.num_splits);
  } else if (unsplit) {
    c = max_np;
  } else if (decode_pages > 0) {
    c = decode_pages;
  } else {
    const int64_t blocks = static_cast<int64_t>(p.batch) * p.num_kv_heads * nrb;
    const int64_t want = ceil_div(static_cast<int64_t>(plan->num_cus) * resident_row_groups_per_cu(p.head_dim, QB),
                                  blocks);
    c = ceil_div(max_np, std::max<int64_t>(1, want));
    const int64_t cmin = std::min(max_np, ceil_div(min_split_tokens(), P));
    c = std::min(max_np, std::max(c, cmin));
    // A few long contexts among short ones: the split from the longest block
    // leaves the long blocks on a few work-groups, each streaming at most
    // about 31 GB/s. Past the balance limit the shortest split that fits the
    // round, or else the limit itself (more than one round of work-groups:
    // there is no other kernel for several tokens).
    const int64_t limit = balance_limit(blk_pages, p.num_kv_heads, cmin);
    if (c > limit) {
      const int64_t slots = static_cast<int64_t>(plan->num_cus) * resident_row_groups_per_cu(p.head_dim, QB);
      const int64_t f = fit_split_pages(blk_pages, p.num_kv_heads, slots, cmin, max_np);
      c = f <= limit ? f : limit;
    }
  }
  c = std::max<int64_t>(c, 1);
  // Grid y = row blocks x splits. The fixed order cannot lengthen its chunk
  // to fit (G 8 or fewer is one row block, checked before it got here).
  if (plan->fixed_multi && ceil_div(max_np, c) > 65535 / nrb) {
    delete plan;
    return DA_ERR_UNSUPPORTED;
  }
  c = std::max<int64_t>(c, ceil_div(max_np, 65535 / nrb));
  if (c > INT32_MAX) c = INT32_MAX;
  plan->pages_per_split = static_cast<int32_t>(c);
  plan->splits.assign(p.batch, 1);
  int64_t smax = 1;
  for (int32_t b = 0; b < p.batch; ++b) {
    for (int64_t rb = 0; rb < nrb; ++rb) {
      const int64_t sb = std::max<int64_t>(1, ceil_div(blk_pages[b * nrb + rb], c));
      plan->splits[b] = static_cast<int32_t>(std::max<int64_t>(plan->splits[b], sb));
      smax = std::max(smax, sb);
      plan->active_units += sb * p.num_kv_heads;
    }
  }
  plan->max_splits = static_cast<int32_t>(smax);
  plan->split_groups = static_cast<int32_t>(nrb * smax);
  if (smax > 1) {
    const size_t rows = static_cast<size_t>(p.batch) * T * p.num_q_heads * smax;
    plan->ws_o_offset = 0;
    plan->ws_ml_offset = round_up(rows * p.head_dim * sizeof(float), 256);
    plan->ws_bytes = plan->ws_ml_offset + round_up(rows * 2 * sizeof(float), 256);
  }
  log_plan(plan);
  return DA_OK;
}

}  // namespace

da_status make_plan(const da_params* p, const int32_t* lens, int32_t num_cus, da_plan** out) {
  if (!p || !out) return DA_ERR_INVALID;
  if (p->batch < 0 || p->num_q_heads < 1 || p->num_kv_heads < 1) return DA_ERR_INVALID;
  if (p->num_q_heads % p->num_kv_heads != 0) return DA_ERR_INVALID;
  if (p->head_dim < 1 || p->page_size < 1) return DA_ERR_INVALID;
  if (p->window < 0 || p->num_splits < 0 || p->fixed_chunk < 0 || p->query_len < 0) return DA_ERR_INVALID;
  if (!std::isfinite(p->scale)) return DA_ERR_INVALID;
  if (!valid_dtype(p->q_dtype) || !valid_dtype(p->kv_dtype) || !valid_dtype(p->out_dtype))
    return DA_ERR_INVALID;
  if (num_cus < 1) return DA_ERR_INVALID;
  if (p->batch > 0 && (!lens || p->max_pages_per_seq < 1)) return DA_ERR_INVALID;
  if (p->kernel != DA_KERNEL_AUTO && p->kernel != DA_KERNEL_VECTOR && p->kernel != DA_KERNEL_MATRIX)
    return DA_ERR_INVALID;
  if (p->rows_per_block != 0 && p->rows_per_block != 16 && p->rows_per_block != 64 && p->rows_per_block != 128)
    return DA_ERR_INVALID;

  const int32_t G = p->num_q_heads / p->num_kv_heads;
  // Group width compiled in the decode kernels; 0 for G > 8, which only the
  // multi-token kernel serves (checked below).
  const int32_t gt = group_tile_for(G);
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256) return DA_ERR_UNSUPPORTED;
  if (p->page_size % 8 != 0 || p->page_size > 1024) return DA_ERR_UNSUPPORTED;
  if (p->batch > 65535 || p->num_kv_heads > 65535) return DA_ERR_UNSUPPORTED;

  const int64_t P = p->page_size;
  if (p->fixed_chunk % P != 0) return DA_ERR_INVALID;
  const bool fixed = p->fixed_chunk > 0;
  const int64_t cap = static_cast<int64_t>(p->max_pages_per_seq) * P;
  // The kernels count tokens in int32, with a few tiles of headroom.
  if (cap > static_cast<int64_t>(INT32_MAX) - 4096) return DA_ERR_UNSUPPORTED;
  for (int32_t b = 0; b < p->batch; ++b) {
    if (lens[b] < 0 || static_cast<int64_t>(lens[b]) > cap) return DA_ERR_INVALID;
  }

  const int32_t T = p->query_len > 1 ? p->query_len : 1;
  // Several new tokens: the multi-token kernels when q and K/V share f16 or
  // bf16; otherwise (or with kernel = DA_KERNEL_VECTOR) the single-query
  // kernels once per token.
  const bool multi_dtypes = p->q_dtype == p->kv_dtype && (p->kv_dtype == DA_F16 || p->kv_dtype == DA_BF16);
  const bool per_token = T > 1 && (!multi_dtypes || p->kernel == DA_KERNEL_VECTOR);
  if (T > 1 && p->kernel == DA_KERNEL_MATRIX && !multi_dtypes) return DA_ERR_UNSUPPORTED;
  // More than 8 query heads per KV head (e.g. 128 over 8): the multi-token
  // kernel only, so 16-bit q and K/V of one type, and no decode kernel forced.
  if (gt == 0 && (!multi_dtypes || per_token || (T <= 1 && p->kernel != DA_KERNEL_AUTO)))
    return DA_ERR_UNSUPPORTED;
  if (T <= 1 && p->kernel == DA_KERNEL_MATRIX && !matrix_kernel_supported(*p)) return DA_ERR_UNSUPPORTED;
  if (!per_token && p->rows_per_block == 128 && p->head_dim > 128) return DA_ERR_UNSUPPORTED;
  if (T > 1) {
    if (fixed) return DA_ERR_UNSUPPORTED;
    // T is the combine grid's y extent; T * G rows are counted in int32.
    if (T > 65535 || static_cast<int64_t>(T) * G > (static_cast<int64_t>(1) << 24)) return DA_ERR_UNSUPPORTED;
    for (int32_t b = 0; b < p->batch; ++b)
      if (lens[b] < T) return DA_ERR_INVALID;  // the new tokens' keys are in the cache
  }

  da_plan* plan = new (std::nothrow) da_plan();
  if (!plan) return DA_ERR_INVALID;
  plan->p = *p;
  plan->query_len = T;
  plan->per_token = per_token;
  plan->group = G;
  plan->group_tile = gt;
  plan->num_cus = num_cus;

  // Attended pages per sequence.
  std::vector<int64_t> npages(p->batch);
  int64_t max_np = 0, total_np = 0;
  for (int32_t b = 0; b < p->batch; ++b) {
    SeqRange r = seq_range(lens[b], p->window, P);
    npages[b] = r.pe - r.pf;
    if (per_token) {
      // Token t attends the keys of a sequence of L - (T-1-t): with a window
      // the page count depends on the window's alignment, so the splits must
      // cover the largest count over the tokens. The counts repeat with the
      // length modulo P (and only grow with L below the window), so the last
      // P + 1 tokens hold the largest.
      for (int64_t t = std::max<int64_t>(0, T - P - 1); t < T; ++t) {
        const SeqRange rt = seq_range(static_cast<int64_t>(lens[b]) - (T - 1 - t), p->window, P);
        npages[b] = std::max(npages[b], rt.pe - rt.pf);
      }
    }
    max_np = std::max(max_np, npages[b]);
    total_np += npages[b];
    plan->attended_keys += r.t1 - r.t0;
  }

  // q.K as a 16 x 32 x 16 matrix-core product per 16-key tile where the
  // parameters allow it and at least two query heads share the keys: then it
  // is a dense contraction, and it takes the dot products and lane sums off
  // the VALU. One head per group (a dot product per key) stays on the vector
  // kernel. Measured, vector / matrix step time, f16 and bf16: G 1 0.998 over
  // 6.2 M attended key-heads, 0.99-1.01 at 0.8-1.5 M, 1.02-1.03 at 0.26-0.39 M;
  // G 2 0.997-0.998 over 6.2 M, 1.00-1.01 over 1.5 M, 1.01-1.02 at 0.79 M,
  // 1.08-1.10 at 0.26-0.39 M.
  plan->split_kernel = matrix_kernel_supported(*p) && p->kernel != DA_KERNEL_VECTOR &&
                               (p->kernel == DA_KERNEL_MATRIX || G >= 2)
                           ? 1
                           : 0;

  // Single-query decode on 16-bit q and K/V runs on the multi-token kernel
  // as one token (a 16-row block, both products on the matrix cores) with 5
  // to 8 query heads per KV head, and with 3 or 4 where the matrix-core
  // decode kernel does not apply (head_dim 64 or 256, pages not a multiple of
  // 16) or the batch has fewer (sequence, KV head) streams than compute
  // units; in each case only if its plan is balanced (see
  // multi_decode_split_pages). The decode kernels keep P.V on the vector
  // ALUs: at 8 heads that is 8 x 8 accumulators per lane and one wave per
  // SIMD, and the vector kernel's q.K is a lane sum per key. Measured, us per
  // step (decode kernels -> this): 64 query heads over 8 KV heads, f16,
  // head_dim 128: the long batch 580 -> 498, 48 heads 578 -> 498, 32 x 1-8k
  // tokens 142 -> 115, the mixed-window batch 155 -> 97, 8 x 8-24k 120 -> 97,
  // 1 x 32k 38.4 -> 25.5, 1 x 3060 13.4 -> 9.9; at head_dim 64 and 256 over
  // 32 x 1-8k tokens 168 -> 66 and 489 -> 216; 32 query heads over 8,
  // head_dim 64 and 256: 32 x 1-8k 74 -> 63 and 245 -> 215, 1 x 3060 10.8
  // -> 8.5 and 20.0 -> 11.4; page size 8 at head_dim 128 129 -> 116; 32 over
  // 8 at head_dim 128 with few streams: 1 x 3060 10.4 -> 9.5, 4 x 3060 18.1
  // -> 13.9, 1 x 32k 30.9 -> 26.8, 16 x 8192 90.1 -> 84.8, 24 x 4096 71.8 ->
  // 68.1. From one stream per compute unit on, the matrix-core decode kernel
  // wins at 3 or 4 heads per KV head (the long batch 482 against 490, the
  // mixed-window batch 95 against 99, 32 x 2048 42.5 against 45.0). With 2
  // heads per KV head (2 of 16 rows used) it lost: 4 x 1-4k tokens at
  // head_dim 256 14.5 -> 16.3. An empty context there has no tiles and its
  // row is written as zeros, as on the decode kernels. More than 8 heads per
  // KV head have no decode kernel and always take this one.
  // At 3 or 4 heads on head_dim 128 (the matrix-core decode kernel built)
  // only the planner's own split choice, and only a plan that splits: an
  // unsplit stream's tiles run through one computing wave there, against
  // four waves on the decode kernel (1 x 100 tokens 5.9 against 8.4 us, 8 x
  // 256 7.3 against 10.2; at 8 heads or head_dim 64 and 256 the two are even
  // or this is faster: 64 heads over 8, 64 x 200 tokens 20.7 -> 11.7).
  // Whole streams: with at least one (sequence, KV head) stream per compute
  // unit and about equal attended lengths (the longest within 10 % of the
  // mean), one unsplit work-group per stream already fills the chip evenly,
  // and splitting only adds the combine launch and the piece starts.
  // Measured on the Llama shape, µs per step, unsplit vs the split choice:
  // 32 x 512 tokens 13.9 vs 20.5, 32 x 1024 24.7 vs 30.3, 32 x 2048 43.6 vs
  // 50.1, 32 x 4096 82.4 vs 88.9, 64 x 1024 43.3 vs 45.3, 128 x 512 43.9 vs
  // 47.1, 48 x 3060 103.3 vs 104.8; with unequal lengths it loses (the long
  // batch 512.9 vs 483.7, 32 x 1-8k tokens 123.2 vs 117.2, the mixed-window
  // batch 106.7 vs 96.6) and so does a batch of fewer streams than compute
  // units (8 x 4096 tokens 47.4 vs 29.7).
  const bool whole_streams = p->num_splits == 0 && max_np > 0 &&
                             static_cast<int64_t>(p->batch) * p->num_kv_heads >= num_cus &&
                             max_np * p->batch * 10 <= total_np * 11;
  // Where the decode kernels are weak: group width 8, 3-4 query heads
  // without the matrix-core decode kernel, and 2 at head_dim 64 unless the
  // batch runs as whole streams (16/8 heads, 32 x 1-8k tokens: 43.4 -> 34.1
  // us; whole streams of 64 x 2048 and 64 x 8192 tokens stay faster on the
  // vector kernel, 23.2 against 25.1 and 82.3 against 83.7 us; at head_dim
  // 256 and with 8-token pages G 2 was even on batches and lost on the 4 x
  // 1-4k wide-head batch, 15.5 -> 16.3). With fewer streams than compute
  // units at head_dim 128 (the planner's split choice, a plan that splits)
  // 1 to 4 query heads per KV head take it too: 16/8 heads, 4 x 3060 tokens
  // 16.1 -> 13.2 us, 1 x 32768 28.3 -> 25.0; 8/8, 4 x 3060 14.3 -> 12.5;
  // 1 x 3060 even. At head_dim 256 only from 8192 attended tokens: 16/8
  // heads, 1 x 8192 17.6 -> 16.0, 4 x 16384 90.4 -> 85.7, 1 x 32768 47.4 ->
  // 45.3; the 4 x 1-4k wide-head batch lost, 14.1 -> 15.7. Not at head_dim
  // 64: 8/8 heads, 4 x 3060 9.9 -> 11.0, 1 x 8192 8.5 -> 9.6, 1 x 16384
  // 10.5 -> 11.5 (a gain only at 32768, 16.8 -> 14.9).
  const bool few_streams = static_cast<int64_t>(p->batch) * p->num_kv_heads < num_cus;
  const bool weak_decode = gt == 0 || gt == 8 || (gt == 4 && !matrix_kernel_supported(*p)) ||
                           (gt == 2 && p->head_dim == 64 && !whole_streams);
  bool mq_decode = T == 1 && (weak_decode || (gt <= 4 && few_streams && p->num_splits == 0 &&
                    (p->head_dim == 128 || (p->head_dim == 256 && max_np * P >= 8192)))) && multi_dtypes &&
                   p->kernel == DA_KERNEL_AUTO && !fixed;
  int64_t mq_pages = 0;
  // Whole streams on this kernel too, at head_dim 128 where the rows of a KV
  // head fit one 16-row block (5 to 16 query heads per KV head, or a few
  // tokens: T x G <= 16): one unsplit work-group per stream. 64 over 8 KV
  // heads, 32 x 4096 tokens 84.1 -> 81.2 us, 32 x 2048 45.4 -> 42.8; 128
  // over 8, 32 x 4096 86.0 -> 80.9; 32 x 512 even; a 4-token check over
  // 32 x 4096 85.8 -> 81.4, over 32 x 2048 46.8 -> 43.5. Not at head_dim 64
  // or 256, where one work-group streams too slowly to fill the chip (32
  // over 8, 32 x 2048 tokens: 25.7 -> 34.5 and 84.9 -> 91.4), nor with more
  // rows (a 4-token check at 64 over 8: 91.5 -> 127.5).
  const bool mq_whole = whole_streams && p->head_dim == 128 && static_cast<int64_t>(T) * G <= 16 &&
                        (p->rows_per_block == 0 || p->rows_per_block == 16);
  if (mq_decode && mq_whole && G >= 5) {
    mq_pages = max_np;
  } else if (mq_decode && p->num_splits == 0) {
    mq_pages = multi_decode_split_pages(npages, p->num_kv_heads, num_cus, p->head_dim, P, weak_decode, gt != 0);
    if (!weak_decode && mq_pages >= max_np) mq_pages = 0;
    mq_decode = mq_pages > 0;
  }
  // The fixed-order mode where the decode kernels are weak (see above) runs
  // on the multi-token kernel too: its splits of `fixed_chunk` tokens from
  // each sequence's first attended page are the mode's chunks, one per
  // work-group, each state computed from its own keys alone; num_splits
  // does not enter the plan, so the output is the same bits for every
  // value. Rows of one chunk are written by the split pass; the combine
  // merges the others in chunk order. 1024-token chunks, us per step,
  // decode kernels -> this: 64 query heads over 8 KV heads, the long batch
  // 608 -> 539, at head_dim 64 over 32 x 1-8k tokens 156 -> 64; 32 over 8 at
  // head_dim 256, 32 x 1-8k 246 -> 229.
  bool mq_fixed = fixed && T == 1 && weak_decode && multi_dtypes && p->kernel == DA_KERNEL_AUTO;
  if (mq_fixed) mq_fixed = ceil_div(max_np, p->fixed_chunk / P) <= 65535;  // the grid's y extent
  if (fixed && gt == 0 && !mq_fixed) {
    delete plan;
    return DA_ERR_UNSUPPORTED;
  }
  if (mq_fixed) {
    plan->fixed_multi = true;
    mq_decode = true;
    mq_pages = p->fixed_chunk / P;
  }
  if ((plan->query_len > 1 && !per_token) || mq_decode) {
    const da_status st = finish_multi_plan(plan, lens, mq_pages, mq_whole && !plan->fixed_multi);
    if (st == DA_OK) *out = plan;
    return st;
  }
  if (fixed) {
    const da_status st = finish_fixed_plan(plan, npages, max_np, total_np);
    if (st == DA_OK) *out = plan;
    return st;
  }

  int64_t c;
  if (max_np == 0) {
    c = 1;
  } else if (p->num_splits > 0) {
    c = ceil_div(max_np, p->num_splits);
  } else if (whole_streams) {
    c = max_np;
  } else {
    c = heuristic_split_pages(total_np, max_np, p->num_kv_heads, num_cus, P,
                              decode_min_split_tokens(plan->split_kernel == 1, max_np * P));
  }
  c = std::max<int64_t>(c, 1);
  // The split index is the grid's y dimension (at most 65535 splits).
  c = std::max<int64_t>(c, ceil_div(max_np, 65535));
  if (c > INT32_MAX) c = INT32_MAX;
  plan->pages_per_split = static_cast<int32_t>(c);

  plan->splits.resize(p->batch);
  int64_t smax = 1;
  for (int32_t b = 0; b < p->batch; ++b) {
    int64_t s = std::max<int64_t>(1, ceil_div(npages[b], c));
    plan->splits[b] = static_cast<int32_t>(s);
    smax = std::max(smax, s);
    plan->active_units += s * p->num_kv_heads;
  }
  // The balanced schedule instead, where the matrix-core kernel runs a
  // single-query step with the planner's split choice, some context is
  // longer than the switch-over (a dispatch of short contexts alone is not
  // split), and these splits would take more than one round of resident
  // work-groups (within one round every work-group has its own slot anyway,
  // and the balanced schedule's start - the batch's prefix sums - only adds
  // latency: 3060-token Llama-8B decode 10.4 -> 12.1 us).
  if (plan->split_kernel == 1 && !per_token && p->num_splits == 0 && !whole_streams &&
      p->batch <= kBalancedMaxBatch &&
      max_np * P > std::max(kDefaultMinSplitTokens, decode_min_split_tokens(true, max_np * P)) &&
      plan->active_units > static_cast<int64_t>(num_cus) * matrix_groups_per_cu(gt) &&
      (total_np + p->batch) * static_cast<int64_t>(p->num_kv_heads) * 64 < static_cast<int64_t>(INT32_MAX) / 2) {
    plan->active_units = 0;
    const da_status st = finish_balanced_plan(plan, npages, max_np);
    if (st == DA_OK) *out = plan;
    return st;
  }
  plan->max_splits = static_cast<int32_t>(smax);
  plan->split_groups = plan->max_splits;
  if (per_token) {
    // Token t runs as a decode over L - (T - 1 - t) keys: the splits above
    // (from the full lengths) cover every token; the workspace holds every
    // token's states; the attended keys are counted per token.
    plan->attended_keys = 0;
    for (int32_t b = 0; b < p->batch; ++b)
      for (int64_t t = 0; t < T; ++t) {
        const int64_t pos = static_cast<int64_t>(lens[b]) - T + t;
        plan->attended_keys += p->window > 0 ? std::min<int64_t>(pos + 1, p->window) : pos + 1;
      }
    plan->active_units *= T;
  }
  if (smax > 1) size_workspace(plan);
  log_plan(plan);
  *out = plan;
  return DA_OK;
}

}  // namespace da
