/* A C99 caller that runs decode attention on the GPU through the library's C
 * ABI alone: it allocates every device buffer itself with hipMalloc, copies
 * the inputs in, plans (decode_attn_plan on device 0), runs one step with
 * decode_attn_run, the same step as decode_attn_split + decode_attn_combine,
 * and once more with decode_attn_run_noalloc, and writes the three outputs
 * back. Built and driven by tests/test_gpu_c_abi_run.py with gcc.
 *
 * usage: c_abi_run DIR
 *   DIR/params.txt  batch num_q_heads num_kv_heads head_dim page_size
 *                   max_pages_per_seq window scale q_dtype kv_dtype out_dtype
 *                   num_splits num_pages   (whitespace separated)
 *   DIR/q.bin DIR/k.bin DIR/v.bin   raw q, K pool, V pool in their dtypes
 *   DIR/table.bin DIR/lens.bin      int32 page table and lengths
 * writes DIR/out_run.bin, DIR/out_two.bin, DIR/out_noalloc.bin (out_dtype).
 * Exit status 0 on success; a message on stderr otherwise. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "decode_attn.h"

static int fail(const char* what, const char* detail) {
  fprintf(stderr, "c_abi_run: %s: %s\n", what, detail);
  return 1;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes ? bytes : 1);
  if (p && bytes && fread(p, 1, bytes, f) != bytes) {
    free(p);
    p = NULL;
  }
  fclose(f);
  return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  const int bad = fwrite(p, 1, bytes, f) != bytes;
  return fclose(f) != 0 || bad;
}

static size_t elt(int dtype) { return dtype == DA_F32 ? 4 : 2; }

/* hipMalloc + copy from the host; NULL on failure. */
static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 16) != hipSuccess) return NULL;
  if (bytes && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(d);
    return NULL;
  }
  return d;
}

int main(int argc, char** argv) {
  if (argc != 2) return fail("usage", "c_abi_run DIR");
  const char* dir = argv[1];
  char path[4096];
  snprintf(path, sizeof path, "%s/params.txt", dir);
  FILE* pf = fopen(path, "r");
  if (!pf) return fail("open", path);
  da_params p;
  memset(&p, 0, sizeof p);
  int qd, kvd, od;
  long num_pages;
  const int n = fscanf(pf, "%d %d %d %d %d %d %d %f %d %d %d %d %ld", &p.batch, &p.num_q_heads, &p.num_kv_heads,
                       &p.head_dim, &p.page_size, &p.max_pages_per_seq, &p.window, &p.scale, &qd, &kvd, &od,
                       &p.num_splits, &num_pages);
  fclose(pf);
  if (n != 13) return fail("params.txt", "expected 13 values");
  p.q_dtype = (da_dtype)qd;
  p.kv_dtype = (da_dtype)kvd;
  p.out_dtype = (da_dtype)od;

  const size_t B = (size_t)p.batch, HQ = (size_t)p.num_q_heads, D = (size_t)p.head_dim;
  const size_t q_bytes = B * HQ * D * elt(qd);
  const size_t out_bytes = B * HQ * D * elt(od);
  const size_t pool_bytes = (size_t)num_pages * (size_t)p.num_kv_heads * (size_t)p.page_size * D * elt(kvd);
  const size_t table_bytes = B * (size_t)p.max_pages_per_seq * 4;
  const size_t lens_bytes = B * 4;
  void* hq = read_file(dir, "q.bin", q_bytes);
  void* hk = read_file(dir, "k.bin", pool_bytes);
  void* hv = read_file(dir, "v.bin", pool_bytes);
  int32_t* ht = (int32_t*)read_file(dir, "table.bin", table_bytes);
  int32_t* hl = (int32_t*)read_file(dir, "lens.bin", lens_bytes);
  if (!hq || !hk || !hv || !ht || !hl) return fail("read", "an input file is missing or short");

  if (hipSetDevice(0) != hipSuccess) return fail("hipSetDevice", "device 0");
  void* dq = to_device(hq, q_bytes);
  void* dk = to_device(hk, pool_bytes);
  void* dv = to_device(hv, pool_bytes);
  void* dt = to_device(ht, table_bytes);
  void* dl = to_device(hl, lens_bytes);
  void* dout = NULL;
  if (!dq || !dk || !dv || !dt || !dl || hipMalloc(&dout, out_bytes) != hipSuccess)
    return fail("hipMalloc", "inputs");

  da_plan_t plan = NULL;
  size_t ws_bytes = 0;
  da_status st = decode_attn_plan(&p, hl, 0, &plan, &ws_bytes);
  if (st != DA_OK) return fail("decode_attn_plan", decode_attn_status_str(st));
  void* dws = NULL;
  if (ws_bytes > 0 && hipMalloc(&dws, ws_bytes) != hipSuccess) return fail("hipMalloc", "workspace");
  hipStream_t stream = NULL;
  if (hipStreamCreate(&stream) != hipSuccess) return fail("hipStreamCreate", "");

  void* host_out = malloc(out_bytes ? out_bytes : 1);
  static const char* names[3] = {"out_run.bin", "out_two.bin", "out_noalloc.bin"};
  for (int pass = 0; pass < 3; ++pass) {
    /* NaN bit patterns (0xFF bytes) in the output: an unwritten row shows. */
    if (hipMemsetAsync(dout, 0xFF, out_bytes, stream) != hipSuccess) return fail("hipMemsetAsync", "out");
    if (pass == 0) {
      st = decode_attn_run(plan, dq, dk, dv, dt, dl, dout, dws, ws_bytes, stream);
    } else if (pass == 1) {
      st = decode_attn_split(plan, dq, dk, dv, dt, dl, dout, dws, ws_bytes, stream);
      if (st == DA_OK) st = decode_attn_combine(plan, dl, dout, dws, ws_bytes, stream);
    } else {
      st = decode_attn_run_noalloc(plan, dq, dk, dv, dt, dl, dout, stream);
    }
    if (st != DA_OK) return fail(names[pass], decode_attn_status_str(st));
    if (hipStreamSynchronize(stream) != hipSuccess) return fail("hipStreamSynchronize", names[pass]);
    if (hipMemcpy(host_out, dout, out_bytes, hipMemcpyDeviceToHost) != hipSuccess) return fail("hipMemcpy", "out");
    if (write_file(dir, names[pass], host_out, out_bytes)) return fail("write", names[pass]);
  }

  /* Errors come back as status codes: a workspace one byte short. */
  if (ws_bytes > 0 &&
      decode_attn_run(plan, dq, dk, dv, dt, dl, dout, dws, ws_bytes - 1, stream) != DA_ERR_WORKSPACE)
    return fail("decode_attn_run", "a short workspace was not refused");

  decode_attn_plan_destroy(plan);
  (void)hipStreamDestroy(stream);
  (void)hipFree(dq);
  (void)hipFree(dk);
  (void)hipFree(dv);
  (void)hipFree(dt);
  (void)hipFree(dl);
  (void)hipFree(dout);
  if (dws) (void)hipFree(dws);
  free(hq);
  free(hk);
  free(hv);
  free(ht);
  free(hl);
  free(host_out);
  printf("c_abi_run: ok (workspace %zu bytes)\n", ws_bytes);
  return 0;
}
