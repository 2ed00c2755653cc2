"""CPU oracle for appending new K/V rows to a paged cache.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; it shares no code with the HIP
library.

What it computes (llm-web pull 8, commit on the batched suffix prefill: the
new tokens' K/V are scattered into the cache at an offset equal to the
resident prefix): sequence b holds L_b keys before the append; its T new rows
go to positions L_b .. L_b + T - 1, i.e. for every KV head j

    k_pool[page_table[b][(L_b + t) // P], j, (L_b + t) % P, :] = k_new[b, t, j, :]

(V likewise). Every other byte of the pools is unchanged. Reading: a row
whose position falls at or beyond max_pages_per_seq * P (outside the page
table) is not written. The function only copies elements, so it works on any
element type, including integer views of bf16 data for bitwise checks.
"""
from __future__ import annotations

import numpy as np


def new_position(seq_len_before: int, t: int) -> int:
    """Logical position of the t-th new token: right after the resident keys."""
    return int(seq_len_before) + t


def page_and_slot(table_row, pos: int, page_size: int):
    """Physical page and slot of logical position `pos` (paged layout: page
    pos // P of the sequence's table, row pos % P inside it)."""
    return int(table_row[pos // page_size]), pos % page_size


def append_kv(k_pool, v_pool, page_table, seq_lens_before, k_new, v_new, page_size: int):
    """Return new (k_pool, v_pool) with the rows of k_new / v_new
    ([B][T][H_kv][D]) written after each sequence's current length."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    B, T, Hkv, D = np.asarray(k_new).shape
    cap = np.asarray(page_table).shape[1] * page_size
    for b in range(B):
        for t in range(T):
            pos = new_position(seq_lens_before[b], t)
            if pos < 0 or pos >= cap:
                continue
            page, slot = page_and_slot(page_table[b], pos, page_size)
            for j in range(Hkv):
                k_out[page, j, slot, :] = k_new[b][t][j]
                v_out[page, j, slot, :] = v_new[b][t][j]
    return k_out, v_out
