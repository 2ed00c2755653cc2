/* A C99 caller of the library's C ABI, built by tests/test_c_abi.py with gcc:
 * plans the batched long-context decode shape (32 sequences, 32 query and 8
 * KV heads, head_dim 128, fp16, 16-token pages) for 256 compute units without
 * a GPU, prints the plan's numbers, and checks that invalid parameters come
 * back as DA_ERR_INVALID. Exit status 0 on success. */
#include <stdio.h>
#include <string.h>

#include "decode_attn.h"

int main(void) {
  da_params p;
  memset(&p, 0, sizeof p);
  p.batch = 32;
  p.num_q_heads = 32;
  p.num_kv_heads = 8;
  p.head_dim = 128;
  p.page_size = 16;
  p.max_pages_per_seq = 2048;
  p.window = 0;
  p.scale = 0.08838834764831845f;
  p.q_dtype = DA_F16;
  p.kv_dtype = DA_F16;
  p.out_dtype = DA_F16;
  int32_t lens[32];
  for (int b = 0; b < 32; ++b) lens[b] = 16384 + (b * 523) % 16384;

  da_plan_t plan = NULL;
  size_t ws = 0;
  da_status st = decode_attn_plan_for_cus(&p, lens, 256, &plan, &ws);
  if (st != DA_OK || plan == NULL) {
    printf("plan failed: %s\n", decode_attn_status_str(st));
    return 1;
  }
  da_plan_info info;
  st = decode_attn_plan_info(plan, &info);
  if (st != DA_OK) return 2;
  printf("pages_per_split %d max_splits %d split_work_groups %d split_kernel %d balanced %d attended_keys %lld "
         "workspace %zu\n",
         info.pages_per_split, info.max_splits, info.split_work_groups, info.split_kernel, info.balanced,
         (long long)info.attended_keys, ws);
  for (int b = 0; b < 3; ++b) printf("splits[%d] %d\n", b, decode_attn_plan_splits(plan, b));
  decode_attn_plan_destroy(plan);

  p.num_kv_heads = 5; /* does not divide 32 query heads */
  plan = NULL;
  st = decode_attn_plan_for_cus(&p, lens, 256, &plan, &ws);
  printf("invalid: %s\n", decode_attn_status_str(st));
  return st == DA_ERR_INVALID && plan == NULL ? 0 : 3;
}
