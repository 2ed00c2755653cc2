// Combine pass of paged decode attention for gfx950.
//
// Merges the per-split online-softmax states (m_s, l_s, O_s) of one
// (sequence, query head) into the output row (TVM pull 20426, sharded-nest
// commit message: the per-shard online-softmax states are merged; mlx-runner
// pull 3, GQA-shared split attention commit: a combine kernel merges the
// split partials in a fixed order):
//     M = max_s m_s,  w_s = 2^(m_s - M),  out = sum_s w_s O_s / sum_s w_s l_s
// A split with no attended key (m_s = -inf) gets weight 0 (never -inf minus
// -inf). The order of the sums is fixed, so results are identical run to run.
// In the fixed-order mode the states are those of fixed-length chunks, whose
// count depends only on the sequence, so the merge is the same whatever the
// number of split work-groups.
//
// Decode: one wave64 per (query head, sequence), four waves per work-group;
// lane i owns elements i, i+64, ... of the row, so every load of O_s is one
// contiguous 256-byte-per-64-lane read. A decode step planned on the
// multi-token split kernel (one token: a single row block per KV head, split
// s of the attended pages in state slot s of row b H_q + h) has the decode
// kernels' split ranges and state layout, so it takes this merge too.
// Several new tokens per sequence (many more rows, few splits each): 32
// lanes per row, two rows per wave.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_attn.h"
#include "device_common.h"
#include "kernels.h"

namespace da {
namespace {

constexpr int kRowsPerGroup = 4;  // one wave per row, four rows per work-group

__device__ __forceinline__ float ldf(const float* p) { return *p; }

// States loaded together by the single-row merges.
constexpr int kMergeBatch = 16;

// The first batch of the states [s_lo, s_lo + avail) of query row `qrow`:
// the O rows of the first min(avail, kMergeBatch) states (lane i takes
// elements i, i + 64, ...) and the (m, l) of state s_lo + lane for lanes below
// avail. `avail` may exceed the range later merged (every slot below
// max_splits lies inside the workspace): entries past the range are never
// used.
template <int D>
__device__ __forceinline__ void load_first(const KernelArgs& a, int64_t qrow, int s_lo, int avail, int lane,
                                           float (&ov)[kMergeBatch][D / 64], float& m0, float& l0) {
  constexpr int N = D / 64;
  const int64_t base = qrow * a.max_splits + s_lo;
  const float* ml = a.ws_ml + base * 2;
  const float* os = a.ws_o + base * D;
#pragma unroll
  for (int j = 0; j < kMergeBatch; ++j)
    if (j < avail)
#pragma unroll
      for (int i = 0; i < N; ++i) ov[j][i] = ldf(os + static_cast<int64_t>(j) * D + lane + 64 * i);
  m0 = -INFINITY;
  l0 = 0.0f;
  if (lane < avail) {
    m0 = ldf(ml + 2 * lane);
    l0 = ldf(ml + 2 * lane + 1);
  }
}

// Merge states [s_lo, s_hi) of query row `qrow` (the flat index of
// (sequence, query head), or of (sequence, new token, query head)) in one
// wave; lane i owns elements i, i + 64, ... of the row:
//     M = max_s m_s,  w_s = 2^(m_s - M),  acc = sum_s w_s O_s,  lsum = sum_s w_s l_s
// A state with m_s = -inf gets weight 0; an empty range gives M = -inf and
// zeros. `ov`, `m0`, `l0` hold the range's first batch (load_first); lane j
// holds (m, l) of state s_lo + j of each chunk of 64, later O rows are loaded
// kMergeBatch at a time, and the weights are broadcast with readlane. The
// order of every sum is fixed, so results are identical run to run.
template <int D>
__device__ __forceinline__ void merge_range_wave(const KernelArgs& a, int64_t qrow, int s_lo, int s_hi, int lane,
                                                 float& M_out, float& lsum_out, float (&acc)[D / 64],
                                                 float (&ov)[kMergeBatch][D / 64], float m0, float l0) {
  constexpr int N = D / 64;
  constexpr int BATCH = kMergeBatch;
  const int cnt_all = s_hi > s_lo ? s_hi - s_lo : 0;
  const int64_t base = qrow * a.max_splits + s_lo;
  const float* ml = a.ws_ml + base * 2;
  const float* os = a.ws_o + base * D;
  auto load_rows = [&](int first, int cnt) {
#pragma unroll
    for (int j = 0; j < BATCH; ++j)
      if (j < cnt)
#pragma unroll
        for (int i = 0; i < N; ++i) ov[j][i] = ldf(os + static_cast<int64_t>(first + j) * D + lane + 64 * i);
  };

  // state `lane` of the first chunk; a slot past the range is replaced here
  m0 = lane < cnt_all ? m0 : -INFINITY;
  l0 = lane < cnt_all ? l0 : 0.0f;
  float M = m0;
  for (int s = 64 + lane; s < cnt_all; s += 64) M = fmaxf(M, ldf(ml + 2 * s));
  M = wave_max(M);
  const float Mu = (M == -INFINITY) ? 0.0f : M;

  float lsum = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = 0.0f;
  for (int s0 = 0; s0 < cnt_all; s0 += 64) {
    float mk = m0, lk = l0;
    if (s0 > 0) {
      mk = -INFINITY;
      lk = 0.0f;
      if (s0 + lane < cnt_all) {
        mk = ldf(ml + 2 * (s0 + lane));
        lk = ldf(ml + 2 * (s0 + lane) + 1);
      }
    }
    float w = 0.0f;
    if (s0 + lane < cnt_all) {
      w = exp2_fast(mk - Mu);
      lsum += w * lk;
    }
    const int cnt = cnt_all - s0 < 64 ? cnt_all - s0 : 64;
    for (int j0 = 0; j0 < cnt; j0 += BATCH) {
      if (s0 + j0 > 0) load_rows(s0 + j0, cnt - j0);
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        if (j0 + j < cnt) {
          const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j0 + j));
#pragma unroll
          for (int i = 0; i < N; ++i) acc[i] = fmaf(wj, ov[j][i], acc[i]);
        }
      }
    }
  }
  lsum_out = wave_sum(lsum);
  M_out = M;
}

// States to merge for query head h of sequence b; 0 if the split pass wrote
// the row itself (a single split, outside the fixed-order mode).
__device__ __forceinline__ int split_count(const KernelArgs& a, int b, int h) {
  int64_t nsplit;
  if (a.ws_cnt != nullptr) {
    // Balanced schedule: the split pass recorded the pieces of each
    // (sequence, KV head) stream.
    nsplit = a.ws_cnt[static_cast<int64_t>(b) * a.num_kv_heads + h / a.group];
  } else {
    const int P = a.page_size;
    const int64_t L = a.seq_lens[b] - a.len_offset;
    const int64_t t0 = (a.window > 0 && L > a.window) ? L - a.window : 0;
    const int64_t pf = L > 0 ? t0 / P : 0;
    const int64_t pe = L > 0 ? (L + P - 1) / P : 0;
    nsplit = (pe - pf + a.pages_per_split - 1) / a.pages_per_split;
  }
  if (nsplit > a.max_splits) nsplit = a.max_splits;
  if (a.chunks_per_group > 0) return nsplit < 1 ? 1 : static_cast<int>(nsplit);  // fixed order: every row
  return nsplit <= 1 ? 0 : static_cast<int>(nsplit);
}

template <int D>
__global__ __launch_bounds__(64 * kRowsPerGroup) void combine_kernel(const KernelArgs a) {
  const int h = blockIdx.x * kRowsPerGroup + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  if (h >= a.num_q_heads) return;  // whole wave
  const int64_t qrow = static_cast<int64_t>(b) * a.rows_per_seq + a.row_base + h;
  // The first states' loads go out before the row's state count is known:
  // a dependent memory round trip less.
  constexpr int N = D / 64;
  float ov[kMergeBatch][N], m0, l0;
  load_first<D>(a, qrow, 0, a.max_splits, lane, ov, m0, l0);
  const int nsplit = split_count(a, b, h);
  if (nsplit <= 0) return;  // the split pass wrote this row
  float M, lsum, acc[N];
  merge_range_wave<D>(a, qrow, 0, nsplit, lane, M, lsum, acc, ov, m0, l0);
  const int64_t row = qrow * D;
#pragma unroll
  for (int i = 0; i < N; ++i) store_elem(a.out, row + lane + 64 * i, a.out_dtype, lsum > 0.0f ? acc[i] / lsum : 0.0f);
}

// Rows with many states (plans with more than kWideSplits states per row):
// four waves per row, one row per work-group. Wave w merges the row's states
// among slots [w S / 4, (w + 1) S / 4), S = max_splits (merge_range_wave),
// then the four partial states are merged through LDS in wave order:
//     M = max_w M_w,  a_w = 2^(M_w - M),  out = sum_w a_w acc_w / sum_w a_w lsum_w
// (a_w = 0 for a wave with no state). The ranges depend only on the plan,
// so each wave's first loads go out before the row's state count is known,
// a dependent memory round trip less (the 3060-token Llama shape at batch
// 1, 48 states per row: 9.5 -> 9.0 us per step, 32 such layers in a graph
// 334.6 -> 320.1 us; rows that need no merge waste those loads: 15 short
// contexts and one of 65536 tokens at 64/8 heads 65.5 -> 66.6 us). Results
// are identical run to run (and, in the fixed-order mode, for every split
// count: S is the chunk count).
constexpr int kWideSplits = 32;

template <int D>
__global__ __launch_bounds__(256) void combine_wide_kernel(const KernelArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t qrow = static_cast<int64_t>(b) * a.rows_per_seq + a.row_base + h;
  constexpr int N = D / 64;
  __shared__ float sh_acc[4][D];
  __shared__ float sh_ml[4][2];
  float M, lsum, acc[N];
  const int S = a.max_splits;
  const int s_lo = wave * S / 4;
  const int s_hi = (wave + 1) * S / 4;
  float ov[kMergeBatch][N], m0, l0;
  load_first<D>(a, qrow, s_lo, s_hi - s_lo, lane, ov, m0, l0);
  const int nsplit = split_count(a, b, h);
  if (nsplit <= 0) return;  // the split pass wrote this row (uniform over the work-group)
  const int lo = s_lo < nsplit ? s_lo : nsplit;
  const int hi = s_hi < nsplit ? s_hi : nsplit;
  merge_range_wave<D>(a, qrow, lo, hi, lane, M, lsum, acc, ov, m0, l0);
#pragma unroll
  for (int i = 0; i < N; ++i) sh_acc[wave][lane + 64 * i] = acc[i];
  if (lane == 0) {
    sh_ml[wave][0] = M;
    sh_ml[wave][1] = lsum;
  }
  __syncthreads();
  float Mt = sh_ml[0][0];
#pragma unroll
  for (int w = 1; w < 4; ++w) Mt = fmaxf(Mt, sh_ml[w][0]);
  const float Mu = (Mt == -INFINITY) ? 0.0f : Mt;
  float aw[4], lt = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    aw[w] = exp2_fast(sh_ml[w][0] - Mu);
    lt += aw[w] * sh_ml[w][1];
  }
  for (int d = threadIdx.x; d < D; d += 256) {
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) o = fmaf(aw[w], sh_acc[w][d], o);
    store_elem(a.out, qrow * D + d, a.out_dtype, lt > 0.0f ? o / lt : 0.0f);
  }
}

// Merge of one row by 32 lanes (half a wave): lane j owns elements E j ..
// E j + E - 1 of the row (E = D / 32), so each split's O row is one
// contiguous read of 4 E bytes per lane, and every lane reads the (m, l)
// pairs itself (the 32 lanes share each address), so nothing crosses lanes.
// Splits are taken BATCH at a time, every load of a batch in flight
// together; across batches the running state is rescaled to the new maximum:
//     M = max_s m_s,  w_s = 2^(m_s - M),  out = sum_s w_s O_s / sum_s w_s l_s
// with the sums in split order (identical results run to run). A state with
// m_s = -inf (no attended key) gets weight 0.
template <int D>
__device__ __forceinline__ void merge_row_halfwave(const KernelArgs& a, int64_t qrow, int nsplit, int hl) {
  constexpr int E = D / 32;
  constexpr int BATCH = 8;
  static_assert(E == 2 || E % 4 == 0, "vector width of the O loads");
  const float* ml = a.ws_ml + qrow * a.max_splits * 2;
  const float* os = a.ws_o + qrow * a.max_splits * D + hl * E;
  float M = -INFINITY, lsum = 0.0f;
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.0f;
  for (int s0 = 0; s0 < nsplit; s0 += BATCH) {
    float ov[BATCH][E], mv[BATCH], lv[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      mv[j] = -INFINITY;
      lv[j] = 0.0f;
#pragma unroll
      for (int i = 0; i < E; ++i) ov[j][i] = 0.0f;
      if (s0 + j < nsplit) {
        const float* o = os + static_cast<int64_t>(s0 + j) * D;
        if constexpr (E == 2) {
          const float2 x = *reinterpret_cast<const float2*>(o);
          ov[j][0] = x.x;
          ov[j][1] = x.y;
        } else {
#pragma unroll
          for (int i = 0; i < E; i += 4) {
            const float4 x = *reinterpret_cast<const float4*>(o + i);
            ov[j][i] = x.x;
            ov[j][i + 1] = x.y;
            ov[j][i + 2] = x.z;
            ov[j][i + 3] = x.w;
          }
        }
        const float2 st = *reinterpret_cast<const float2*>(ml + 2 * (s0 + j));
        mv[j] = st.x;
        lv[j] = st.y;
      }
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < BATCH; ++j) Mn = fmaxf(Mn, mv[j]);
    const float Mu = (Mn == -INFINITY) ? 0.0f : Mn;
    const float alpha = exp2_fast(M - Mu);  // 0 before the first state
    lsum *= alpha;
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      if (s0 + j < nsplit) {
        const float w = exp2_fast(mv[j] - Mu);
        lsum += w * lv[j];
#pragma unroll
        for (int i = 0; i < E; ++i) acc[i] = fmaf(w, ov[j][i], acc[i]);
      }
    }
    M = Mn;
  }
  const int64_t row = qrow * D + hl * E;
#pragma unroll
  for (int i = 0; i < E; ++i) store_elem(a.out, row + i, a.out_dtype, lsum > 0.0f ? acc[i] / lsum : 0.0f);
}

// Several new tokens per sequence: two (query head, token, sequence) rows per
// wave, 32 lanes each, eight rows per work-group. The split count of a row is
// that of its row block (rows_per_group consecutive (token, head) rows of one
// KV head), whose keys run from the window start of its first token to its
// last token.
constexpr int kMultiRowsPerGroup = 8;

template <int D>
__global__ __launch_bounds__(256) void combine_multi_kernel(const KernelArgs a) {
  const int h = blockIdx.x * kMultiRowsPerGroup + static_cast<int>(threadIdx.x >> 5);
  const int t = blockIdx.y;
  const int b = blockIdx.z;
  const int hl = threadIdx.x & 31;
  if (h >= a.num_q_heads) return;  // whole half-wave
  const int T = a.query_len;
  constexpr int E = D / 32;
  constexpr int BATCH = 8;
  const int64_t qrow = (static_cast<int64_t>(b) * T + t) * a.num_q_heads + h;
  const float* ml = a.ws_ml + qrow * a.max_splits * 2;
  const float* os = a.ws_o + qrow * a.max_splits * D + hl * E;
  // The first BATCH states' loads go out before the split count is known
  // (their slots lie inside the workspace); slots past the count are
  // replaced below by select, so whatever they hold is never used.
  const int first = a.max_splits < BATCH ? a.max_splits : BATCH;
  float ov[BATCH][E], mv[BATCH], lv[BATCH];
#pragma unroll
  for (int j = 0; j < BATCH; ++j) {
    mv[j] = -INFINITY;
    lv[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) ov[j][i] = 0.0f;
    if (j < first) {
      const float* o = os + static_cast<int64_t>(j) * D;
      if constexpr (E == 2) {
        const float2 x = *reinterpret_cast<const float2*>(o);
        ov[j][0] = x.x;
        ov[j][1] = x.y;
      } else {
#pragma unroll
        for (int i = 0; i < E; i += 4) {
          const float4 x = *reinterpret_cast<const float4*>(o + i);
          ov[j][i] = x.x;
          ov[j][i + 1] = x.y;
          ov[j][i + 2] = x.z;
          ov[j][i + 3] = x.w;
        }
      }
      const float2 st = *reinterpret_cast<const float2*>(ml + 2 * j);
      mv[j] = st.x;
      lv[j] = st.y;
    }
  }
  const int G = a.group;
  const int R = T * G;
  const int P = a.page_size;
  const int L = a.seq_lens[b];
  const int r = t * G + (h - (h / G) * G);
  const int r_first = r / a.rows_per_group * a.rows_per_group;
  const int r_last = (r_first + a.rows_per_group < R ? r_first + a.rows_per_group : R) - 1;
  int hi_blk = L - T + r_last / G + 1;
  hi_blk = hi_blk < 0 ? 0 : hi_blk;
  int lo_blk = a.window > 0 ? L - T + r_first / G + 1 - a.window : 0;
  lo_blk = lo_blk < 0 ? 0 : (lo_blk > hi_blk ? hi_blk : lo_blk);
  const int pf = lo_blk / P;
  const int pe = (hi_blk + P - 1) / P;
  int nsplit = (pe - pf + a.pages_per_split - 1) / a.pages_per_split;
  if (nsplit > a.max_splits) nsplit = a.max_splits;
  if (nsplit <= 1) return;  // the split pass wrote this row
#pragma unroll
  for (int j = 0; j < BATCH; ++j) {
    const bool use = j < nsplit;
    mv[j] = use ? mv[j] : -INFINITY;
    lv[j] = use ? lv[j] : 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) ov[j][i] = use ? ov[j][i] : 0.0f;
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < BATCH; ++j) M = fmaxf(M, mv[j]);
  const float Mu0 = (M == -INFINITY) ? 0.0f : M;
  float lsum = 0.0f;
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < BATCH; ++j) {
    if (j < nsplit) {
      const float w = exp2_fast(mv[j] - Mu0);
      lsum += w * lv[j];
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] = fmaf(w, ov[j][i], acc[i]);
    }
  }
  // Further states (more than BATCH splits), BATCH at a time as in the
  // single-row merge.
  for (int s0 = BATCH; s0 < nsplit; s0 += BATCH) {
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      mv[j] = -INFINITY;
      lv[j] = 0.0f;
#pragma unroll
      for (int i = 0; i < E; ++i) ov[j][i] = 0.0f;
      if (s0 + j < nsplit) {
        const float* o = os + static_cast<int64_t>(s0 + j) * D;
        if constexpr (E == 2) {
          const float2 x = *reinterpret_cast<const float2*>(o);
          ov[j][0] = x.x;
          ov[j][1] = x.y;
        } else {
#pragma unroll
          for (int i = 0; i < E; i += 4) {
            const float4 x = *reinterpret_cast<const float4*>(o + i);
            ov[j][i] = x.x;
            ov[j][i + 1] = x.y;
            ov[j][i + 2] = x.z;
            ov[j][i + 3] = x.w;
          }
        }
        const float2 st = *reinterpret_cast<const float2*>(ml + 2 * (s0 + j));
        mv[j] = st.x;
        lv[j] = st.y;
      }
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < BATCH; ++j) Mn = fmaxf(Mn, mv[j]);
    const float Mu = (Mn == -INFINITY) ? 0.0f : Mn;
    const float alpha = exp2_fast(M - Mu);  // 0 while no state had a key
    lsum *= alpha;
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      if (s0 + j < nsplit) {
        const float w = exp2_fast(mv[j] - Mu);
        lsum += w * lv[j];
#pragma unroll
        for (int i = 0; i < E; ++i) acc[i] = fmaf(w, ov[j][i], acc[i]);
      }
    }
    M = Mn;
  }
  const int64_t row = qrow * D + hl * E;
#pragma unroll
  for (int i = 0; i < E; ++i) store_elem(a.out, row + i, a.out_dtype, lsum > 0.0f ? acc[i] / lsum : 0.0f);
}

}  // namespace

hipError_t launch_combine(const KernelArgs& a, int head_dim, hipStream_t stream) {
  if (a.query_len > 1) {
    const dim3 grid((a.num_q_heads + kMultiRowsPerGroup - 1) / kMultiRowsPerGroup, a.query_len, a.batch);
    const dim3 block(256);
    switch (head_dim) {
      case 64: hipLaunchKernelGGL(combine_multi_kernel<64>, grid, block, 0, stream, a); break;
      case 128: hipLaunchKernelGGL(combine_multi_kernel<128>, grid, block, 0, stream, a); break;
      case 256: hipLaunchKernelGGL(combine_multi_kernel<256>, grid, block, 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (a.max_splits > kWideSplits) {
    const dim3 grid(a.num_q_heads, a.batch);
    switch (head_dim) {
      case 64: hipLaunchKernelGGL(combine_wide_kernel<64>, grid, dim3(256), 0, stream, a); break;
      case 128: hipLaunchKernelGGL(combine_wide_kernel<128>, grid, dim3(256), 0, stream, a); break;
      case 256: hipLaunchKernelGGL(combine_wide_kernel<256>, grid, dim3(256), 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const dim3 grid((a.num_q_heads + kRowsPerGroup - 1) / kRowsPerGroup, a.batch);
  const dim3 block(64 * kRowsPerGroup);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(combine_kernel<64>, grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL(combine_kernel<128>, grid, block, 0, stream, a); break;
    case 256: hipLaunchKernelGGL(combine_kernel<256>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace da
