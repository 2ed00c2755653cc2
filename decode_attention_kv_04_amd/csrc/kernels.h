// Launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace da {

// Arguments of both passes (plain pointers and sizes; passed by value).
struct KernelArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  void* out;
  float* ws_o;   // [B][H_q][S_max][D]
  float* ws_ml;  // [B][H_q][S_max][2]  (m in log2 units, l)
  int32_t* ws_cnt;  // balanced schedule: [B][H_kv] pieces per (sequence, KV head) stream, else null
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;          // G (<= the compiled group width)
  int32_t page_size;
  int32_t max_pages;      // page-table row stride
  int32_t window;
  int32_t pages_per_split;  // pages per split (fixed-order mode: per chunk)
  int32_t max_splits;       // state slots per query head in the workspace
  int32_t chunks_per_group; // 0 = default mode; else fixed-order mode, chunks per work-group
  int32_t split_groups;     // split work-groups per (sequence, KV head)
  int32_t query_len;        // T new tokens per sequence (1 = single-query decode)
  // Single-query kernels run once per new token when the multi-token kernels
  // do not cover the dtypes: token t sees L - len_offset keys and its q, out
  // and workspace rows are b * rows_per_seq + row_base + h. Decode: 0, H_q, 0.
  int32_t len_offset;
  int32_t rows_per_seq;
  int32_t row_base;
  int32_t rows_per_group;   // multi-token kernel: query rows (token, head) per work-group
  int32_t balanced;         // 1 = balanced schedule: work-group w takes units [w q, (w+1) q) of the
                            // batch's (sequence, KV head) streams, q = pages_per_split
  int32_t bal_overhead;     // balanced schedule: units a stream weighs before its pages
  int32_t q_dtype;        // da_dtype
  int32_t out_dtype;      // da_dtype
  float scale_log2;       // scale * log2(e): scores are kept in base-2 units
};

// Arguments of the K/V append.
struct AppendArgs {
  const void* k_new;  // [B][T][H_kv][D]
  const void* v_new;
  const int32_t* page_table;
  const int32_t* seq_lens;  // keys before the append
  void* k_pool;
  void* v_pool;
  int32_t batch;
  int32_t tokens;  // T
  int32_t num_kv_heads;
  int32_t page_size;
  int32_t max_pages;
  int32_t row_bytes;  // D * elt, a multiple of 16
};

// Enqueue the K/V append (grid T x B) on `stream`.
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

// Enqueue the split pass on `stream`. Returns hipSuccess or the launch error;
// hipErrorInvalidValue if no kernel is compiled for (head_dim, kv_dtype,
// group_tile).
hipError_t launch_split(const KernelArgs& a, int head_dim, int kv_dtype, int group_tile, hipStream_t stream);

// Enqueue the split pass with q.K on the matrix cores (q and K/V share a
// 16-bit type, head_dim 128, page size a multiple of 16).
hipError_t launch_split_mfma(const KernelArgs& a, int head_dim, int kv_dtype, int group_tile, hipStream_t stream);

// Enqueue the multi-token split pass (query_len >= 1) on `stream`.
hipError_t launch_multi(const KernelArgs& a, int head_dim, int kv_dtype, int rows_per_group, hipStream_t stream);

// Enqueue the combine pass on `stream`.
hipError_t launch_combine(const KernelArgs& a, int head_dim, hipStream_t stream);

// Device address of `device`'s static scratch (DECODE_ATTN_SCRATCH_BYTES,
// 256-byte aligned); looked up once per device, then cached.
hipError_t scratch_address(int device, void** ptr);

}  // namespace da
