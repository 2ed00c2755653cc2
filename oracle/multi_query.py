"""CPU float64 oracle for attention of several new tokens over a paged cache.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; it shares no code with the HIP
library.

What it computes (llm-web pull 8, commit on the batched suffix prefill: the
new tokens of a prompt whose prefix is already cached go through one batched
pass, their K/V scattered after the resident prefix and their attention
reading the cache): sequence b holds L_b keys, the last T of which belong to
the T new tokens (their K/V were appended first). New token t sits at
position p = L_b - T + t and, being causal, attends the keys at positions
<= p, the last W of them for a window W > 0:

    keys(b, t) = [max(0, p + 1 - W), p + 1)   (W > 0),   [0, p + 1)   (W = 0)
    out[b, t, h] = softmax(scale * K q[b, t, h]) V   over keys(b, t)

with the head mapping, scale and paging of the single-query decode oracle.
For T = 1 this is exactly that oracle. Readings: the new tokens' own keys are
in the cache (a token attends itself); the window is counted back from each
query's own position; every sequence has the same T and L_b >= T.
"""
from __future__ import annotations

import numpy as np

from .attention_f64 import attend_one, attended_range, gather_rows, kv_head_of


def query_position(L: int, T: int, t: int) -> int:
    """Position in the cache of the t-th of the T new tokens (the last T keys)."""
    return L - T + t


def query_keys(L: int, T: int, t: int, window: int):
    """[k0, k1): the keys new token t attends (causal, windowed from itself)."""
    p = query_position(L, T, t)
    return attended_range(p + 1, window)


def prefill_attention(q, k_pool, v_pool, page_table, seq_lens, page_size: int, scale: float,
                      window: int = 0) -> np.ndarray:
    """out[b, t, h, :] as float64 [B][T][H_q][D]; q is [B][T][H_q][D] and
    seq_lens counts the new tokens."""
    q = np.asarray(q)
    B, T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.zeros((B, T, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L < T:
            raise ValueError(f"sequence {b}: {L} keys cannot hold {T} new tokens")
        for t in range(T):
            k0, k1 = query_keys(L, T, t, int(window))
            for j in range(Hkv):
                K = gather_rows(k_pool, page_table[b], j, k0, k1, page_size)
                V = gather_rows(v_pool, page_table[b], j, k0, k1, page_size)
                for h in range(Hq):
                    if kv_head_of(h, G) == j:
                        out[b, t, h] = attend_one(q[b, t, h], K, V, scale64)
    return out
