/*
 * decode_attn.h - paged decode attention on MI355X (gfx950).
 *
 * One decode step: every sequence b has one query token with H_q heads and a
 * KV cache of L_b keys stored in fixed-size pages. For every query head h the
 * library computes
 *
 *     out[b,h,:] = softmax_t(scale * <q[b,h,:], K[b,j,t,:]>) V[b,j,t,:]
 *
 * over the attended keys t, where j = floor(h / G) is the KV head that the G =
 * H_q / H_kv consecutive query heads of a GQA group share, and the attended
 * keys are the last `window` keys (all L_b keys when window = 0 or window >=
 * L_b). A sequence with no attended key gets a zero row.
 *
 * With query_len = T > 1 (da_params) every sequence has T new tokens, the
 * last T keys of its cache: token t sits at position L_b - T + t and attends
 * the keys at positions <= its own (the last `window` of them). An optional
 * fixed-order mode makes the output bitwise independent of the split count,
 * and decode_attn_append_kv writes new K/V rows into the pages.
 *
 * Where the operations come from (each declaration below cites its own
 * passage as well; pages are cited by title and section):
 *   - TVM pull 20426 "webgpu-decode-attention", commit message of the sharded
 *     nest: decode attention over a paged cache in which the context is cut
 *     into shards, each shard summarised by an online-softmax state, the
 *     states then merged; the host chooses between the paths from the page
 *     count. PR description: the sharded path takes over above 256 tokens,
 *     and sliding windows are among its tested cases.
 *   - mlx-runner pull 3, commit "GQA-shared split attention" and PR
 *     description "Changes": one work-group serves every query head that
 *     shares a KV head, so K/V is streamed once per GQA group rather than
 *     once per query head; the split pass writes partial states and a
 *     separate combine pass merges them in a fixed order; the token count at
 *     which splitting starts is a tunable (256 by default). Its split decode
 *     attention test: with one fixed merge order the split and unsplit paths
 *     give identical bits.
 *   - llm-web pull 8, commits on build-time constants and on pipeline
 *     creation errors: head_dim, dtype and window are fixed per pipeline
 *     before any launch; a rejected configuration is reported to the caller
 *     at creation, and the caller chooses the fallback. Its commit on the
 *     batched suffix prefill: new tokens' K/V are written behind the
 *     resident prefix and several new tokens attend the cache together. Its
 *     commit on engine ownership: the owner releases what it created.
 *
 * Conventions
 *   - Pointers are device pointers unless their name starts with host_.
 *   - Every device buffer is owned by the caller. The library never allocates
 *     or frees device memory. A plan is a small host object owned by the
 *     caller and released with decode_attn_plan_destroy.
 *   - Tensors are dense and row-major:
 *       q           [B][H_q][D] ([B][T][H_q][D] when T > 1)   q_dtype
 *       k_pool      [num_pages][H_kv][P][D]          kv_dtype
 *       v_pool      [num_pages][H_kv][P][D]          kv_dtype
 *       page_table  [B][max_pages_per_seq]           int32, logical -> physical page
 *       seq_lens    [B]                              int32, keys in the cache
 *       out         [B][H_q][D] ([B][T][H_q][D] when T > 1)   out_dtype
 *     Key t of sequence b, KV head j, is row t % P of block
 *     (page_table[b][t / P], j) of the pools. Only the pages holding attended
 *     keys are read; rows outside the attended range (the tail of the last
 *     page, keys before the window) may hold anything, NaN included.
 *   - q, k_pool, v_pool and out must be 16-byte aligned; page_table and
 *     seq_lens 4-byte aligned; workspace 256-byte aligned.
 *   - Status codes are the only error channel; nothing is printed unless the
 *     environment sets DECODE_ATTN_LOG=1 (plan decisions go to stderr).
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DA_OK = 0,
  DA_ERR_INVALID = 1,     /* a parameter, pointer, alignment or length is invalid       */
  DA_ERR_UNSUPPORTED = 2, /* valid, but no kernel is built for it (head_dim, group...)  */
  DA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the plan requires        */
  DA_ERR_HIP = 4          /* the HIP runtime reported an error (device query or launch) */
} da_status;

typedef enum { DA_F32 = 0, DA_F16 = 1, DA_BF16 = 2 } da_dtype;

/* Which single-query split kernel a plan uses (da_params.kernel). */
typedef enum {
  DA_KERNEL_AUTO = 0,   /* the planner chooses (matrix cores from 2 query heads per KV head on;
                           a decode step with 5 or more of them, 3-4 where the
                           decode matrix-core kernel is not built, 1-4 at
                           head_dim 128 (at 256 from 8192 attended tokens)
                           when the batch has fewer (sequence, KV head)
                           streams than compute units, or 2 at head_dim 64,
                           on the multi-token
                           kernel as one token when its plan is balanced)      */
  DA_KERNEL_VECTOR = 1, /* vector q.K; with query_len > 1: the single-query kernels per token   */
  DA_KERNEL_MATRIX = 2  /* q.K on the matrix cores; DA_ERR_UNSUPPORTED where not built           */
} da_kernel;

typedef struct {
  int32_t batch;             /* B >= 0                                              */
  int32_t num_q_heads;       /* H_q >= 1                                            */
  int32_t num_kv_heads;      /* H_kv >= 1, divides H_q; G = H_q / H_kv. G 1..8 on
                                every kernel; G > 8 (e.g. 128 query heads over 8,
                                or many over one KV head) only on the multi-token
                                kernel: q and K/V sharing f16 or bf16, kernel
                                DA_KERNEL_AUTO for decode (DA_KERNEL_VECTOR for
                                query_len > 1 is the per-token path), and in the
                                fixed-order mode at most 65535 row blocks x
                                chunks per sequence; else DA_ERR_UNSUPPORTED   */
  int32_t head_dim;          /* D in {64, 128, 256}                                 */
  int32_t page_size;         /* P: a multiple of 8, 8..1024                         */
  int32_t max_pages_per_seq; /* row stride of page_table; >= ceil(L_b / P)          */
  int32_t window;            /* 0 = none; else attend the last `window` keys        */
  float scale;               /* score scale, e.g. 1/sqrt(D); finite                 */
  da_dtype q_dtype, kv_dtype, out_dtype;
  int32_t num_splits;        /* 0 = the planner decides; > 0 caps the splits of the
                                longest sequence at this count (1 = no split)       */
  int32_t fixed_chunk;       /* 0 = default mode. > 0 = fixed-order mode: the
                                attended range of each sequence is cut into chunks
                                of this many tokens (a multiple of page_size),
                                counted from its first attended page; each chunk's
                                softmax state is computed the same way whichever
                                work-group computes it, and the states are merged
                                in chunk order, so the output is bitwise the same
                                for every num_splits (mlx-runner pull 3, split
                                decode attention test: split and unsplit paths
                                agree bit for bit because the partials are merged
                                in one fixed order). num_splits then counts
                                work-groups per sequence and KV head, each taking
                                consecutive chunks; on the multi-token kernel
                                (DA_KERNEL_AUTO with G 5 or more, 2 at head_dim
                                64, or 3-4 where the decode matrix-core kernel
                                is not built; q and K/V sharing f16 or bf16)
                                every chunk has its own work-group and
                                num_splits does not apply.                       */
  int32_t query_len;         /* T, new tokens per sequence; 0 or 1 = one query
                                token (decode). T > 1 (llm-web pull 8, commit on
                                the batched suffix prefill: several new tokens
                                attend the cache after their K/V were written
                                behind the resident prefix): q and out are
                                [B][T][H_q][D]; token t of sequence b sits at
                                position L_b - T + t and attends the keys at
                                positions <= its own (the last `window` of them
                                if window > 0). Needs L_b >= T, T <= 65535
                                and fixed_chunk == 0. q and K/V sharing f16 or
                                bf16 run the multi-token kernels (both products
                                on the matrix cores); other dtype combinations
                                (or kernel = DA_KERNEL_VECTOR) run the
                                single-query kernels once per token (meant for
                                a few tokens).                                 */
  int32_t kernel;            /* da_kernel: DA_KERNEL_AUTO (0) unless a caller
                                wants one split kernel (benchmarks, tests).
                                Decode: DA_KERNEL_MATRIX needs q and K/V
                                sharing f16 or bf16, head_dim 128 and page_size
                                a multiple of 16. query_len > 1:
                                DA_KERNEL_MATRIX = the multi-token kernels
                                (needs q and K/V sharing f16 or bf16),
                                DA_KERNEL_VECTOR = the single-query kernels
                                once per token. DA_ERR_UNSUPPORTED where the
                                choice is not built; other values
                                DA_ERR_INVALID. Only DA_KERNEL_AUTO takes a
                                decode step to the multi-token kernel.          */
  int32_t rows_per_block;    /* On the multi-token kernels (also a decode plan
                                that takes them): the (token, head) rows of a
                                KV head per work-group. 0 = the planner
                                chooses; 16, 64, or 128 (128 only at head_dim
                                64 and 128, else DA_ERR_UNSUPPORTED for every
                                plan); other values are DA_ERR_INVALID. The
                                decode kernels ignore it.                       */
} da_params;

typedef struct da_plan* da_plan_t;

/* What a plan decided (for logging, tests and benchmarks). */
typedef struct {
  int32_t pages_per_split;   /* c: pages of attended context per split              */
  int32_t max_splits;        /* S_max over the batch (1 = no combine pass)          */
  int32_t num_cus;           /* compute units the plan was made for                 */
  int32_t split_work_groups; /* work-groups the split kernel launches               */
  int64_t active_units;      /* sum over b of splits(b) * H_kv                      */
  int64_t attended_keys;     /* sum over b of attended keys                         */
  size_t workspace_bytes;    /* bytes of device workspace `run` needs (0 if none)   */
  int32_t split_kernel;      /* 0 = vector q.K (any parameters); 1 = q.K on the
                                matrix cores (q and K/V share f16 or bf16,
                                head_dim 128, page size a multiple of 16, at
                                least two query heads per KV head);
                                da_params.kernel forces 0 or 1. 2 = the
                                multi-token kernels (q.K and P.V on the matrix
                                cores): the T*G rows of a KV head in blocks of
                                16 (16 rows or fewer: one wave computes, three
                                copy), 64 (17 to 64 rows; more rows at
                                head_dim 256) or 128 (more than 64 rows at
                                head_dim 64 and 128);
                                da_params.rows_per_block forces one. Decode
                                plans (query_len <= 1) with DA_KERNEL_AUTO
                                take 2 when q and K/V share f16 or bf16 and G
                                is above 8 (always), 5 to 8, 2 at head_dim 64,
                                3 to 4 where 1 is not built, or 1 to 4 at
                                head_dim 128 (256 with a context of at least
                                8192 attended tokens) when (num_splits 0, and
                                the plan splits) B * H_kv is below num_cus;
                                and (num_splits 0) only if no work-group of
                                that plan holds more than about 1/170 of the
                                batch's attended page-heads (else the decode
                                kernels and their balanced schedule run; G
                                above 8 then takes that limit). In the
                                fixed-order mode they take 2 for G 5 or more,
                                2 at head_dim 64, or 3 to 4 where 1 is not
                                built. A query_len > 1
                                plan with 0 runs the vector kernel once per
                                token.                                        */
  int32_t chunks_per_work_group; /* fixed-order mode: consecutive chunks each
                                work-group computes (1 on the multi-token
                                kernel; 0 in the default mode). In
                                that mode pages_per_split is the chunk length in
                                pages and max_splits the most chunks of a sequence. */
  int32_t balanced;          /* 1 = balanced schedule (the matrix-core decode
                                kernel when num_splits is 0): the batch's
                                (sequence, KV head, attended page) units in that
                                order, an empty stream counting one, are dealt
                                to split_work_groups work-groups, pages_per_split
                                consecutive units each (about one round of
                                resident work-groups of equal work); a stream cut
                                by their boundaries has one state per piece,
                                max_splits at most. 0 = grid schedule: split s of
                                every sequence is pages_per_split attended pages. */
} da_plan_info;

/*
 * decode_attn_plan: validate `p` and the B host-side lengths, pick how the
 * attended context is cut into splits (pages per split, from the context
 * lengths and the device's compute-unit count), and size the workspace. Host
 * only: no device work, no allocation on the device. `device` is a HIP device
 * ordinal; its compute-unit count is read once and cached.
 * Follows: TVM pull 20426, commit message of the sharded nest (the host picks
 * the path from the page count) and PR description (sharding only above 256
 * tokens); mlx-runner pull 3, commit "GQA-shared split attention" (the split
 * threshold is a tunable with a 256-token default; here it is the shortest
 * split, and the environment variable DECODE_ATTN_SPLIT_MIN overrides it);
 * llm-web pull 8, commits on build-time constants (head_dim, dtype and
 * window fixed before launch) and on pipeline creation errors (every
 * rejection is reported here, before any launch).
 *   host_seq_lens  [B] int32 host array (may be NULL when B = 0); values in
 *                  0 .. max_pages_per_seq * P.
 *   plan_out       receives a new plan on DA_OK (unchanged otherwise).
 *   workspace_bytes_out (may be NULL) receives the workspace size run needs.
 * Returns DA_ERR_INVALID / DA_ERR_UNSUPPORTED for bad or unbuilt parameters,
 * DA_ERR_HIP if the device cannot be queried.
 */
da_status decode_attn_plan(const da_params* p, const int32_t* host_seq_lens, int device,
                           da_plan_t* plan_out, size_t* workspace_bytes_out);

/*
 * decode_attn_plan_for_cus: as decode_attn_plan, for an explicit compute-unit
 * count instead of a device query (num_cus >= 1). Makes no HIP call, so it
 * also works on a host without a GPU.
 */
da_status decode_attn_plan_for_cus(const da_params* p, const int32_t* host_seq_lens, int32_t num_cus,
                                   da_plan_t* plan_out, size_t* workspace_bytes_out);

/* decode_attn_plan_info: copy a plan's decisions into *info. Follows: TVM
 * pull 20426, commit message of the sharded nest (which path the host chose
 * from the page count) - exposed so callers and benchmarks can see it. */
da_status decode_attn_plan_info(da_plan_t plan, da_plan_info* info);

/* decode_attn_plan_splits: number of splits of sequence b (1 .. max_splits);
 * 0 for a NULL plan or b outside 0 .. B-1. Follows: TVM pull 20426, commit
 * message of the sharded nest (the shards a sequence's context is cut into). */
int32_t decode_attn_plan_splits(da_plan_t plan, int32_t b);

/*
 * decode_attn_run: enqueue one decode-attention step on `stream` (a
 * hipStream_t; NULL = the null stream): the split pass, then, if the plan has
 * more than one split, the combine pass. Returns after enqueueing; no host
 * synchronisation and no allocation, so it can be captured in a HIP graph.
 * Follows: TVM pull 20426, commit message of the sharded nest (shards of the
 * paged context, one online-softmax state each, merged in a second phase) and
 * PR description (sliding windows); mlx-runner pull 3, commit "GQA-shared
 * split attention" (K/V read once per GQA group; split partials merged by a
 * combine kernel).
 *   q, k_pool, v_pool, page_table, seq_lens   read-only inputs (layouts above).
 *   seq_lens   must hold the same lengths the plan was made from.
 *   out        [B][H_q][D] out_dtype, fully written.
 *   workspace  >= the plan's workspace_bytes (may be NULL if that is 0);
 *              scratch for per-split states, contents undefined afterwards.
 * Contents of page_table and seq_lens are not checked on the device: entries
 * that point outside the pools are undefined behaviour. A device fault shows
 * up at the caller's next synchronisation.
 * Calls that share a workspace must be ordered on one stream.
 */
da_status decode_attn_run(da_plan_t plan, const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* page_table, const int32_t* seq_lens, void* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * decode_attn_split: the first pass of decode_attn_run alone. Every split of
 * every sequence writes its online-softmax state (running max m, sum l,
 * unnormalised O) to the workspace; sequences with a single split write their
 * final output rows directly. Same arguments and checks as decode_attn_run.
 * Follows: TVM pull 20426, commit message of the sharded nest (the per-shard
 * online-softmax states); mlx-runner pull 3, commit "GQA-shared split
 * attention" (the split kernel writing per-split partials).
 */
da_status decode_attn_split(da_plan_t plan, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* page_table, const int32_t* seq_lens, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * decode_attn_combine: the second pass alone. Merges the split states that a
 * preceding decode_attn_split (same plan, same seq_lens, same workspace) left
 * in the workspace into the output rows of sequences with more than one split.
 * Enqueues nothing when the plan has a single split. Same status codes as
 * decode_attn_run (seq_lens and out are checked; q and the pools are not
 * used).
 * Follows: TVM pull 20426, commit message of the sharded nest (the merge of
 * the shard states); mlx-runner pull 3, commit "GQA-shared split attention"
 * (a combine kernel merging the partials in one fixed order).
 */
da_status decode_attn_combine(da_plan_t plan, const int32_t* seq_lens, void* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * decode_attn_append_kv: write T new K and V rows per sequence into the paged
 * cache, after the keys it already holds (llm-web pull 8, commit on the
 * batched suffix prefill: the new tokens' K/V are scattered at an offset
 * equal to the resident prefix). For every b, t < T and KV head j, with
 * pos = seq_lens[b] + t:
 *     k_pool[page_table[b][pos / P]][j][pos % P][:] = k_new[b][t][j][:]
 * and the same for V. No other byte of the pools changes.
 *   p         uses batch, num_kv_heads, head_dim, page_size,
 *             max_pages_per_seq and kv_dtype (the other fields are ignored).
 *   k_new, v_new  [B][T][H_kv][D] kv_dtype, 16-byte aligned.
 *   seq_lens  [B] int32, keys before the append (not updated here; the
 *             caller adds T for the next step).
 *   page_table must map every page the new rows land in; a row whose
 *   position is negative or >= max_pages_per_seq * P is skipped.
 * Enqueues one kernel on `stream`; no allocation, no host synchronisation.
 * Returns DA_ERR_INVALID / DA_ERR_UNSUPPORTED for bad arguments.
 */
da_status decode_attn_append_kv(const da_params* p, int32_t tokens, const void* k_new, const void* v_new,
                                const int32_t* page_table, const int32_t* seq_lens, void* k_pool, void* v_pool,
                                void* stream);

/*
 * decode_attn_run_noalloc: decode_attn_run for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): it takes no workspace. The split states
 * go to a static scratch array of DECODE_ATTN_SCRATCH_BYTES (64 MiB) that the
 * library holds on every GPU it runs on, until the process ends. The call
 * allocates nothing; its first call on a device looks up that device's
 * scratch address once. The GPU is the stream's (hipStreamGetDevice; the null
 * stream: the current device).
 *   Arguments, checks and results as decode_attn_run (the same kernels run).
 *   Returns DA_ERR_WORKSPACE if the plan's workspace_bytes exceeds
 *   DECODE_ATTN_SCRATCH_BYTES (plan with fewer splits, or use
 *   decode_attn_run), DA_ERR_HIP if the scratch cannot be looked up.
 * All calls on one GPU share its scratch, which keeps the last call's
 * contents (no call needs it cleared: every state a call reads, that call
 * wrote). Calls whose work overlaps in time on one GPU (different streams,
 * or unordered threads) race: order them on one stream.
 */
#define DECODE_ATTN_SCRATCH_BYTES (64u * 1024u * 1024u)
da_status decode_attn_run_noalloc(da_plan_t plan, const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* page_table, const int32_t* seq_lens, void* out, void* stream);

/* decode_attn_plan_destroy: free a plan (NULL is ignored); the plan must not
 * be used afterwards. Follows: llm-web pull 8, commit on engine ownership
 * (the owner of an object releases it explicitly, at once). */
void decode_attn_plan_destroy(da_plan_t plan);

/* decode_attn_status_str: static text for a status code (never NULL; an
 * unknown code gets a fixed "unknown" text). Follows: llm-web pull 8, commit
 * on pipeline creation errors (failures are reported to the caller, which
 * chooses what to do). */
const char* decode_attn_status_str(da_status s);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
