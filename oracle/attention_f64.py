"""CPU float64 oracle for paged single-query decode attention.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module. It shares no code with the HIP
library and never calls it.

What it computes (the plain definition; the split-context method reaches the
same result exactly, up to rounding order, because online softmax with a
merge of shard states is an exact rewrite of softmax):

For every sequence b and query head h, with GQA group size G = H_q / H_kv,
KV head j = floor(h / G) (consecutive query heads share a KV head), and the
attended keys T_b = { t : L_b - L_eff,b <= t < L_b }, L_eff,b = min(L_b, W)
for a window W > 0 and L_b otherwise:

    K_b,j[t] = k_pool[page_table[b][t // P], j, t % P, :]      (V likewise)
    s_t      = scale * <q[b,h], K_b,j[t]>
    m        = max_t s_t
    out[b,h] = sum_t exp(s_t - m) V_b,j[t] / sum_t exp(s_t - m)

and out[b,h] = 0 when T_b is empty.

Sources (cited by page title and passage):
* TVM pull 20426 "webgpu-decode-attention", commit message of the sharded
  nest: paged decode attention with one query per sequence, context cut into
  shards whose online-softmax states are merged; accuracy stated as relative
  L2 against an f64 reference; the PR description adds sliding windows.
* mlx-runner pull 3, commit message "GQA-shared split attention": a split
  kernel covering all query heads of a GQA group, whose per-split partial
  states a combine kernel merges.
* llm-web pull 8, build-time constants commit: head_dim and WINDOW are
  per-pipeline constants.

Readings where the pages are silent (each also listed in the design notes):
* window: the last W keys including the newest; W = 0 or W >= L means none.
* the query is the newest token; its key is already in the cache, so there is
  no causal mask beyond the window.
* head mapping: j = floor(h / G).
* scale: a float32 parameter; the oracle uses float64(float32(scale)).
* L_b = 0 gives a zero row.

Every function here is pinned by tests against brute force, a library
attention routine in float64, closed forms and invariants (no function is
"parity unpinned").
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np


def kv_head_of(h: int, group: int) -> int:
    """KV head read by query head h: consecutive query heads share one."""
    return h // group


def attended_range(L: int, window: int) -> Tuple[int, int]:
    """[t0, L): the keys query b attends, the last `window` ones if window > 0."""
    if window > 0 and L > window:
        return L - window, L
    return 0, L


def gather_rows(pool: np.ndarray, table_row: np.ndarray, kv_head: int, t0: int, t1: int,
                page_size: int) -> np.ndarray:
    """Own page walk: rows t0..t1-1 of one KV head, as float64 [t1-t0][D]."""
    t = np.arange(t0, t1)
    pages = np.asarray(table_row)[t // page_size]
    slots = t % page_size
    return pool[pages, kv_head, slots, :].astype(np.float64)


def attend_one(qv: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V for one query vector, two-pass, float64."""
    D = V.shape[1]
    if K.shape[0] == 0:
        return np.zeros(D, dtype=np.float64)
    s = float(scale) * (K @ qv.astype(np.float64))
    m = s.max()
    e = np.exp(s - m)
    return (e @ V) / e.sum()


def decode_attention(q, k_pool, v_pool, page_table, seq_lens, page_size: int, scale: float,
                     window: int = 0) -> np.ndarray:
    """out[b, h, :] for every sequence and query head, float64 [B][H_q][D].

    q [B][H_q][D], pools [pages][H_kv][P][D], page_table [B][max_pages],
    seq_lens [B]; any float dtype that holds the stored values exactly."""
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        t0, t1 = attended_range(int(seq_lens[b]), int(window))
        for j in range(Hkv):
            K = gather_rows(k_pool, page_table[b], j, t0, t1, page_size)
            V = gather_rows(v_pool, page_table[b], j, t0, t1, page_size)
            for h in range(Hq):
                if kv_head_of(h, G) != j:
                    continue
                out[b, h] = attend_one(q[b, h], K, V, scale64)
    return out


# ---------------------------------------------------------------------------
# Shard states and their merge: the split-context pass written out in f64.
# A shard of keys [lo, hi) summarises itself as (m, l, O) with
#   m = max s_t,  l = sum exp(s_t - m),  O = sum exp(s_t - m) V[t]
# (m = -inf, l = 0, O = 0 for an empty shard). The merge rescales every state
# to the global maximum M: w_s = exp(m_s - M) (0 for an empty shard), then
# out = sum w_s O_s / sum w_s l_s.
# ---------------------------------------------------------------------------

def shard_state(qv: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, lo: int, hi: int):
    D = V.shape[1]
    if hi <= lo:
        return -math.inf, 0.0, np.zeros(D, dtype=np.float64)
    s = float(scale) * (K[lo:hi] @ qv.astype(np.float64))
    m = s.max()
    e = np.exp(s - m)
    return float(m), float(e.sum()), e @ V[lo:hi]


def merge_states(states: Sequence[Tuple[float, float, np.ndarray]]) -> np.ndarray:
    D = states[0][2].shape[0]
    M = max(m for m, _, _ in states)
    if M == -math.inf:
        return np.zeros(D, dtype=np.float64)
    num = np.zeros(D, dtype=np.float64)
    den = 0.0
    for m, l, O in states:
        if m == -math.inf:
            continue
        w = math.exp(m - M)
        num += w * O
        den += w * l
    return num / den


def decode_attention_sharded(q, k_pool, v_pool, page_table, seq_lens, page_size: int, scale: float,
                             window: int, shard_keys: int) -> np.ndarray:
    """Same output as decode_attention, computed as contiguous shards of
    `shard_keys` attended keys each whose states are then merged."""
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        t0, t1 = attended_range(int(seq_lens[b]), int(window))
        n = t1 - t0
        bounds = list(range(0, n, shard_keys)) + [n]
        if n == 0:
            bounds = [0, 0]
        for h in range(Hq):
            j = kv_head_of(h, G)
            K = gather_rows(k_pool, page_table[b], j, t0, t1, page_size)
            V = gather_rows(v_pool, page_table[b], j, t0, t1, page_size)
            states = [shard_state(q[b, h], K, V, scale64, bounds[i], bounds[i + 1])
                      for i in range(len(bounds) - 1)]
            out[b, h] = merge_states(states)
    return out


# ---------------------------------------------------------------------------
# Reference rounding of an f64 result to a storage dtype, round to nearest
# even, directly from float64 (no double rounding through float32).
# ---------------------------------------------------------------------------

def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to f32 / f16 / bf16 (returned as float64)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        # bf16 keeps 8 significant bits: drop the low 45 of float64's 52
        # fraction bits with round-half-to-even (values stay in bf16's normal
        # range for attention outputs; NaN/inf pass through).
        bits = x.view(np.uint64).copy()
        finite = np.isfinite(x)
        drop = np.uint64(45)
        half = np.uint64(1) << np.uint64(44)
        lsb = (bits >> drop) & np.uint64(1)
        rounded = (bits + (half - np.uint64(1)) + lsb) >> drop << drop
        bits = np.where(finite, rounded, bits)
        return bits.view(np.float64)
    raise ValueError(dtype)


def relative_l2(out: np.ndarray, ref: np.ndarray) -> float:
    """||out - ref||_2 / ||ref||_2 over the whole array, in float64."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.sqrt(np.sum(ref * ref))
    num = np.sqrt(np.sum((out - ref) ** 2))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return float(num / den)


def relative_l2_per_row(out: np.ndarray, ref: np.ndarray) -> List[float]:
    """relative_l2 over each sequence's rows (axis 0)."""
    return [relative_l2(out[b], ref[b]) for b in range(ref.shape[0])]
