// C ABI of the decode-attention library: argument checks, device query,
// workspace carving and the two launches. Errors are status codes only
// (llm-web pull 8, pipeline-creation commit: failures surface to the caller,
// which chooses the fallback; the library has none).
#include <cmath>
#include <cstdint>
#include <mutex>
#include <unordered_map>

#include <hip/hip_runtime_api.h>

#include "decode_attn.h"
#include "kernels.h"
#include "plan.h"

namespace {

std::mutex g_cu_mutex;
std::unordered_map<int, int> g_cu_count;

da_status device_cus(int device, int32_t* cus) {
  {
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    auto it = g_cu_count.find(device);
    if (it != g_cu_count.end()) {
      *cus = it->second;
      return DA_OK;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return DA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  g_cu_count[device] = n;
  *cus = n;
  return DA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Checks shared by run and split; fills the kernel arguments.
da_status prepare(const da_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* page_table, const int32_t* seq_lens, void* out, void* workspace,
                  size_t workspace_bytes, da::KernelArgs* a) {
  if (!plan) return DA_ERR_INVALID;
  const da_params& p = plan->p;
  if (p.batch > 0) {
    if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !out) return DA_ERR_INVALID;
    if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16)) return DA_ERR_INVALID;
    if (!aligned(page_table, 4) || !aligned(seq_lens, 4)) return DA_ERR_INVALID;
  }
  if (plan->ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan->ws_bytes) return DA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return DA_ERR_INVALID;
  }
  a->q = q;
  a->k_pool = k_pool;
  a->v_pool = v_pool;
  a->page_table = page_table;
  a->seq_lens = seq_lens;
  a->out = out;
  char* ws = static_cast<char*>(workspace);
  const bool has_ws = plan->ws_bytes > 0;
  a->ws_o = has_ws ? reinterpret_cast<float*>(ws + plan->ws_o_offset) : nullptr;
  a->ws_ml = has_ws ? reinterpret_cast<float*>(ws + plan->ws_ml_offset) : nullptr;
  a->ws_cnt = has_ws && plan->balanced ? reinterpret_cast<int32_t*>(ws + plan->ws_cnt_offset) : nullptr;
  a->balanced = plan->balanced ? 1 : 0;
  a->bal_overhead = plan->bal_overhead;
  a->batch = p.batch;
  a->num_q_heads = p.num_q_heads;
  a->num_kv_heads = p.num_kv_heads;
  a->group = plan->group;
  a->page_size = p.page_size;
  a->max_pages = p.max_pages_per_seq;
  a->window = p.window;
  a->pages_per_split = plan->pages_per_split;
  a->max_splits = plan->max_splits;
  a->chunks_per_group = plan->chunks_per_group;
  a->split_groups = plan->split_groups;
  a->query_len = plan->query_len;
  a->rows_per_group = plan->rows_per_group;
  a->len_offset = 0;
  a->rows_per_seq = p.num_q_heads;
  a->row_base = 0;
  a->q_dtype = p.q_dtype;
  a->out_dtype = p.out_dtype;
  a->scale_log2 = static_cast<float>(static_cast<double>(p.scale) * 1.4426950408889634);
  return DA_OK;
}

// The combine pass runs when some sequence has several splits, and always in
// the fixed-order mode (every row goes through the chunk-order merge).
bool needs_combine(const da_plan* plan) { return plan->max_splits > 1 || plan->chunks_per_group > 0; }

da_status enqueue_one(const da_plan* plan, const da::KernelArgs& a, bool split, bool combine, hipStream_t st);

da_status enqueue(const da_plan* plan, const da::KernelArgs& a, bool split, bool combine, void* stream) {
  if (plan->p.batch == 0) return DA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // start from a clean error state
  if (!plan->per_token) return enqueue_one(plan, a, split, combine, st);
  // One single-query pass per new token t: L - (T - 1 - t) keys, rows of
  // token t (q, out and workspace hold all T tokens' rows).
  const int32_t T = plan->query_len;
  for (int32_t t = 0; t < T; ++t) {
    da::KernelArgs at = a;
    at.query_len = 1;
    at.len_offset = T - 1 - t;
    at.rows_per_seq = T * plan->p.num_q_heads;
    at.row_base = t * plan->p.num_q_heads;
    const da_status s = enqueue_one(plan, at, split, combine, st);
    if (s != DA_OK) return s;
  }
  return DA_OK;
}

da_status enqueue_one(const da_plan* plan, const da::KernelArgs& a, bool split, bool combine, hipStream_t st) {
  if (split) {
    hipError_t e;
    if (plan->split_kernel == 2)
      e = da::launch_multi(a, plan->p.head_dim, plan->p.kv_dtype, plan->rows_per_group, st);
    else if (plan->split_kernel == 1)
      e = da::launch_split_mfma(a, plan->p.head_dim, plan->p.kv_dtype, plan->group_tile, st);
    else
      e = da::launch_split(a, plan->p.head_dim, plan->p.kv_dtype, plan->group_tile, st);
    if (e != hipSuccess) return DA_ERR_HIP;
  }
  if (combine && needs_combine(plan)) {
    if (da::launch_combine(a, plan->p.head_dim, st) != hipSuccess) return DA_ERR_HIP;
  }
  return DA_OK;
}

}  // namespace

extern "C" {

da_status decode_attn_plan(const da_params* p, const int32_t* host_seq_lens, int device, da_plan_t* plan_out,
                           size_t* workspace_bytes_out) {
  if (!p || !plan_out) return DA_ERR_INVALID;
  int32_t cus = 0;
  da_status st = device_cus(device, &cus);
  if (st != DA_OK) return st;
  return decode_attn_plan_for_cus(p, host_seq_lens, cus, plan_out, workspace_bytes_out);
}

da_status decode_attn_plan_for_cus(const da_params* p, const int32_t* host_seq_lens, int32_t num_cus,
                                   da_plan_t* plan_out, size_t* workspace_bytes_out) {
  if (!plan_out) return DA_ERR_INVALID;
  da_plan* plan = nullptr;
  da_status st = da::make_plan(p, host_seq_lens, num_cus, &plan);
  if (st != DA_OK) return st;
  *plan_out = plan;
  if (workspace_bytes_out) *workspace_bytes_out = plan->ws_bytes;
  return DA_OK;
}

da_status decode_attn_plan_info(da_plan_t plan, da_plan_info* info) {
  if (!plan || !info) return DA_ERR_INVALID;
  info->pages_per_split = plan->pages_per_split;
  info->max_splits = plan->max_splits;
  info->num_cus = plan->num_cus;
  info->split_work_groups =
      plan->balanced ? plan->split_groups : plan->split_groups * plan->p.num_kv_heads * plan->p.batch;
  info->active_units = plan->active_units;
  info->attended_keys = plan->attended_keys;
  info->workspace_bytes = plan->ws_bytes;
  info->split_kernel = plan->split_kernel;
  info->chunks_per_work_group = plan->fixed_multi ? 1 : plan->chunks_per_group;
  info->balanced = plan->balanced ? 1 : 0;
  return DA_OK;
}

int32_t decode_attn_plan_splits(da_plan_t plan, int32_t b) {
  if (!plan || b < 0 || b >= plan->p.batch) return 0;
  return plan->splits[b];
}

da_status decode_attn_run(da_plan_t plan, const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* page_table, const int32_t* seq_lens, void* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  da::KernelArgs a;
  da_status st = prepare(plan, q, k_pool, v_pool, page_table, seq_lens, out, workspace, workspace_bytes, &a);
  if (st != DA_OK) return st;
  return enqueue(plan, a, true, true, stream);
}

da_status decode_attn_split(da_plan_t plan, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* page_table, const int32_t* seq_lens, void* out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  da::KernelArgs a;
  da_status st = prepare(plan, q, k_pool, v_pool, page_table, seq_lens, out, workspace, workspace_bytes, &a);
  if (st != DA_OK) return st;
  return enqueue(plan, a, true, false, stream);
}

da_status decode_attn_combine(da_plan_t plan, const int32_t* seq_lens, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!plan) return DA_ERR_INVALID;
  if (plan->p.batch > 0) {
    if (!seq_lens || !out) return DA_ERR_INVALID;
    if (!aligned(seq_lens, 4) || !aligned(out, 16)) return DA_ERR_INVALID;
  }
  if (plan->ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan->ws_bytes) return DA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return DA_ERR_INVALID;
  }
  if (!needs_combine(plan)) return DA_OK;
  da::KernelArgs a{};
  const da_params& p = plan->p;
  a.seq_lens = seq_lens;
  a.out = out;
  a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan->ws_o_offset);
  a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan->ws_ml_offset);
  a.ws_cnt = plan->balanced ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan->ws_cnt_offset)
                            : nullptr;
  a.balanced = plan->balanced ? 1 : 0;
  a.bal_overhead = plan->bal_overhead;
  a.batch = p.batch;
  a.num_q_heads = p.num_q_heads;
  a.num_kv_heads = p.num_kv_heads;
  a.group = plan->group;
  a.page_size = p.page_size;
  a.max_pages = p.max_pages_per_seq;
  a.window = p.window;
  a.pages_per_split = plan->pages_per_split;
  a.max_splits = plan->max_splits;
  a.chunks_per_group = plan->chunks_per_group;
  a.split_groups = plan->split_groups;
  a.query_len = plan->query_len;
  a.rows_per_group = plan->rows_per_group;
  a.len_offset = 0;
  a.rows_per_seq = p.num_q_heads;
  a.row_base = 0;
  a.q_dtype = p.q_dtype;
  a.out_dtype = p.out_dtype;
  return enqueue(plan, a, false, true, stream);
}

da_status decode_attn_append_kv(const da_params* p, int32_t tokens, const void* k_new, const void* v_new,
                                const int32_t* page_table, const int32_t* seq_lens, void* k_pool, void* v_pool,
                                void* stream) {
  if (!p || tokens < 0 || p->batch < 0 || p->num_kv_heads < 1 || p->page_size < 1 || p->max_pages_per_seq < 1)
    return DA_ERR_INVALID;
  if (p->kv_dtype != DA_F32 && p->kv_dtype != DA_F16 && p->kv_dtype != DA_BF16) return DA_ERR_INVALID;
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256) return DA_ERR_UNSUPPORTED;
  if (p->batch > 65535 || tokens > 2147483647 / 2) return DA_ERR_UNSUPPORTED;
  if (p->batch == 0 || tokens == 0) return DA_OK;
  if (!k_new || !v_new || !page_table || !seq_lens || !k_pool || !v_pool) return DA_ERR_INVALID;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16)) return DA_ERR_INVALID;
  if (!aligned(page_table, 4) || !aligned(seq_lens, 4)) return DA_ERR_INVALID;
  da::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.batch = p->batch;
  a.tokens = tokens;
  a.num_kv_heads = p->num_kv_heads;
  a.page_size = p->page_size;
  a.max_pages = p->max_pages_per_seq;
  a.row_bytes = p->head_dim * (p->kv_dtype == DA_F32 ? 4 : 2);
  (void)hipGetLastError();
  if (da::launch_append(a, static_cast<hipStream_t>(stream)) != hipSuccess) return DA_ERR_HIP;
  return DA_OK;
}

da_status decode_attn_run_noalloc(da_plan_t plan, const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* page_table, const int32_t* seq_lens, void* out, void* stream) {
  if (!plan) return DA_ERR_INVALID;
  if (plan->ws_bytes > DECODE_ATTN_SCRATCH_BYTES) return DA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan->ws_bytes > 0) {
    hipDevice_t dev = 0;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess ||
        da::scratch_address(dev, &ws) != hipSuccess) {
      (void)hipGetLastError();
      return DA_ERR_HIP;
    }
  }
  return decode_attn_run(plan, q, k_pool, v_pool, page_table, seq_lens, out, ws, plan->ws_bytes, stream);
}

void decode_attn_plan_destroy(da_plan_t plan) { delete plan; }

const char* decode_attn_status_str(da_status s) {
  switch (s) {
    case DA_OK: return "DA_OK: success";
    case DA_ERR_INVALID: return "DA_ERR_INVALID: invalid parameter, pointer, alignment or length";
    case DA_ERR_UNSUPPORTED: return "DA_ERR_UNSUPPORTED: no kernel is built for these parameters";
    case DA_ERR_WORKSPACE: return "DA_ERR_WORKSPACE: workspace missing or too small";
    case DA_ERR_HIP: return "DA_ERR_HIP: HIP runtime error";
  }
  return "unknown da_status";
}

}  // extern "C"
