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
// One wave64 per (query head, sequence), four waves per work-group; lane i
// owns elements i, i+64, ... of the row, so every load of O_s is one
// contiguous 256-byte-per-64-lane read.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_attn.h"
#include "device_common.h"
#include "kernels.h"

namespace da {
namespace {

constexpr int kRowsPerGroup = 4;  // one wave per row, four rows per work-group

template <int D>
__global__ __launch_bounds__(64 * kRowsPerGroup) void combine_kernel(const KernelArgs a) {
  const int h = blockIdx.x * kRowsPerGroup + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  if (h >= a.num_q_heads) return;  // whole wave

  const int P = a.page_size;
  const int64_t L = a.seq_lens[b] - a.len_offset;
  const int64_t t0 = (a.window > 0 && L > a.window) ? L - a.window : 0;
  const int64_t pf = L > 0 ? t0 / P : 0;
  const int64_t pe = L > 0 ? (L + P - 1) / P : 0;
  int64_t nsplit = (pe - pf + a.pages_per_split - 1) / a.pages_per_split;
  if (nsplit > a.max_splits) nsplit = a.max_splits;
  if (a.chunks_per_group > 0) {
    if (nsplit < 1) nsplit = 1;  // fixed-order mode: every row is merged here
  } else if (nsplit <= 1) {
    return;  // the split pass wrote this row
  }

  merge_head_wave<D>(a, static_cast<int64_t>(b) * a.rows_per_seq + a.row_base + h, static_cast<int>(nsplit), lane);
}

// Several new tokens per sequence: one wave per (query head, token, sequence).
// The split count of a row is that of its row block (rows_per_group
// consecutive (token, head) rows of one KV head), whose keys run from the
// window start of its first token to its last token.
template <int D>
__global__ __launch_bounds__(64 * kRowsPerGroup) void combine_multi_kernel(const KernelArgs a) {
  const int h = blockIdx.x * kRowsPerGroup + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  if (h >= a.num_q_heads) return;  // whole wave
  const int T = a.query_len;
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
  merge_head_wave<D>(a, (static_cast<int64_t>(b) * T + t) * a.num_q_heads + h, nsplit, lane);
}

}  // namespace

hipError_t launch_combine(const KernelArgs& a, int head_dim, hipStream_t stream) {
  if (a.query_len > 1) {
    const dim3 grid((a.num_q_heads + kRowsPerGroup - 1) / kRowsPerGroup, a.query_len, a.batch);
    const dim3 block(64 * kRowsPerGroup);
    switch (head_dim) {
      case 64: hipLaunchKernelGGL(combine_multi_kernel<64>, grid, block, 0, stream, a); break;
      case 128: hipLaunchKernelGGL(combine_multi_kernel<128>, grid, block, 0, stream, a); break;
      case 256: hipLaunchKernelGGL(combine_multi_kernel<256>, grid, block, 0, stream, a); break;
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
