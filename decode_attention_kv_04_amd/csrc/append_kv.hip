// Append new K/V rows to the paged cache (the step before decode attention).
//
// llm-web pull 8, commit on the batched suffix prefill: the new tokens' K/V
// are scattered into the cache at an offset equal to the resident prefix.
// Sequence b holds L_b keys; its T new rows go to positions L_b .. L_b+T-1:
//     pool[page_table[b][pos / P]][j][pos % P][:] = new[b][t][j][:]
// One work-group per (new token, sequence) copies the H_kv rows of K and of
// V with 16-byte loads and stores; a token's H_kv rows of one pool are
// H_kv runs of D elements, P rows apart. Rows whose position is outside the page
// table (pos >= max_pages_per_seq * P) or negative are skipped.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "decode_attn.h"
#include "kernels.h"

namespace da {
namespace {

constexpr int kMaxThreads = 256;

__global__ __launch_bounds__(kMaxThreads) void append_kernel(const AppendArgs a) {
  const int t = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t pos = static_cast<int64_t>(a.seq_lens[b]) + t;
  if (pos < 0 || pos >= static_cast<int64_t>(a.max_pages) * a.page_size) return;  // uniform
  const int64_t page = a.page_table[static_cast<int64_t>(b) * a.max_pages + pos / a.page_size];
  const int64_t slot = pos % a.page_size;
  const int row_vec = a.row_bytes / 16;                 // 16-byte vectors per row
  const int nvec = a.num_kv_heads * row_vec;            // per tensor
  const int64_t src_row0 = (static_cast<int64_t>(b) * a.tokens + t) * a.num_kv_heads;
  for (int i = threadIdx.x; i < nvec; i += blockDim.x) {
    const int j = i / row_vec;
    const int v = i - j * row_vec;
    const int64_t src = (src_row0 + j) * row_vec + v;
    const int64_t dst = ((page * a.num_kv_heads + j) * a.page_size + slot) * row_vec + v;
    const uint4 kx = static_cast<const uint4*>(a.k_new)[src];
    const uint4 vx = static_cast<const uint4*>(a.v_new)[src];
    static_cast<uint4*>(a.k_pool)[dst] = kx;
    static_cast<uint4*>(a.v_pool)[dst] = vx;
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  // One thread per 16-byte vector of a token's K (and V) rows, in whole waves.
  const int nvec = a.num_kv_heads * (a.row_bytes / 16);
  const int threads = std::min(kMaxThreads, std::max(64, (nvec + 63) / 64 * 64));
  hipLaunchKernelGGL(append_kernel, dim3(a.tokens, a.batch), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace da
