"""Pins for the K/V append oracle: the appended cache is read back through
mechanisms that do not share its indexing (dense per-sequence views made by
concatenating whole pages, attention over a dense concatenation of old and
new keys), and planted mistakes in its steps must fail them."""
import numpy as np
import pytest
import torch

import oracle
from oracle import paged_cache as opc


def paged_case(rng, lens, T, Hkv=2, D=4, P=4, spare_pages=0, cap_pages=None):
    """Shuffled pages holding each sequence's lens[b] keys plus room for T
    more (or cap_pages pages per sequence); every other slot is NaN."""
    need = [max(1, -(-(L + T) // P)) for L in lens]
    maxp = cap_pages or max(need)
    need = [min(n, maxp) for n in need]
    total = sum(need) + spare_pages
    perm = rng.permutation(total)
    table = np.full((len(lens), maxp), total, dtype=np.int64)   # unmapped entries point at a NaN page
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    kp = np.full((total + 1, Hkv, P, D), np.nan)
    vp = np.full_like(kp, np.nan)
    for b, L in enumerate(lens):
        for t in range(L):
            kp[table[b, t // P], :, t % P] = rng.standard_normal((Hkv, D))
            vp[table[b, t // P], :, t % P] = rng.standard_normal((Hkv, D))
    kn = rng.standard_normal((len(lens), T, Hkv, D))
    vn = rng.standard_normal((len(lens), T, Hkv, D))
    return kp, vp, table, np.array(lens), kn, vn


def dense(pool, table_row, n):
    """First n keys of a sequence as [H_kv][n][D], by concatenating its pages
    whole (torch.cat along the slot axis), not by per-position indexing."""
    P = pool.shape[2]
    npg = -(-n // P)
    if npg == 0:
        return np.zeros((pool.shape[1], 0, pool.shape[3]))
    return torch.cat([torch.as_tensor(pool[int(table_row[p])]) for p in range(npg)], dim=1)[:, :n].numpy()


def sdpa_dense(q, K, V, scale):
    """torch float64 SDPA over dense per-head keys (GQA by repeating heads)."""
    Hq = q.shape[0]
    K = torch.as_tensor(K).repeat_interleave(Hq // K.shape[0], dim=0)
    V = torch.as_tensor(V).repeat_interleave(Hq // V.shape[0], dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(torch.as_tensor(q)[:, None, :], K, V, scale=scale)
    return o[:, 0, :].numpy()


CASES = [
    ([0], 1, 4),
    ([3], 1, 4),
    ([4], 1, 4),          # the new row opens a page
    ([5, 0, 8], 3, 4),
    ([1, 6], 9, 2),       # new rows span several pages
    ([7, 2, 11, 0], 5, 8),
]


@pytest.mark.parametrize("lens,T,P", CASES)
def test_dense_view_is_old_keys_then_new_keys(lens, T, P):
    rng = np.random.default_rng(len(lens) * 100 + T)
    kp, vp, table, L, kn, vn = paged_case(rng, lens, T, P=P, spare_pages=2)
    k2, v2 = oracle.append_kv(kp, vp, table, L, kn, vn, P)
    for b, n in enumerate(lens):
        for before, after, new in ((kp, k2, kn), (vp, v2, vn)):
            d = dense(after, table[b], n + T)
            np.testing.assert_array_equal(d[:, :n], dense(before, table[b], n))
            np.testing.assert_array_equal(d[:, n:], np.transpose(new[b], (1, 0, 2)))


@pytest.mark.parametrize("lens,T,P", CASES)
def test_only_the_new_rows_change(lens, T, P):
    rng = np.random.default_rng(7 + T)
    kp, vp, table, L, kn, vn = paged_case(rng, lens, T, P=P, spare_pages=3)
    k2, v2 = oracle.append_kv(kp, vp, table, L, kn, vn, P)
    for before, after in ((kp, k2), (vp, v2)):
        # NaN-safe change mask over (page, head, slot) rows
        changed = ~np.all((before == after) | (np.isnan(before) & np.isnan(after)), axis=-1)
        assert int(changed.sum()) == len(lens) * T * before.shape[1]
        # the spare pages and the NaN page stay untouched
        used = set(int(x) for x in table[:, :].ravel())
        for p in range(before.shape[0]):
            if p not in used:
                assert not changed[p].any()


def test_append_to_empty_sequence_fills_identity_pages_in_order():
    """Closed form: with an identity page table and L = 0 the pool read in
    storage order is the new rows, T = a whole number of pages."""
    rng = np.random.default_rng(3)
    P, T, Hkv, D = 4, 12, 2, 3
    kp = np.zeros((3, Hkv, P, D))
    kn = rng.standard_normal((1, T, Hkv, D))
    k2, _ = oracle.append_kv(kp, kp, np.arange(3)[None, :], [0], kn, kn, P)
    # pool [page][head][slot][d] -> [head][page*P+slot][d]
    np.testing.assert_array_equal(np.transpose(k2, (1, 0, 2, 3)).reshape(Hkv, T, D),
                                  np.transpose(kn[0], (1, 0, 2)))


def test_rows_past_the_page_table_are_skipped():
    rng = np.random.default_rng(4)
    P = 4
    kp, vp, table, L, kn, vn = paged_case(rng, [6], 5, P=P, cap_pages=2)   # capacity 8: rows 6, 7 fit
    k2, v2 = oracle.append_kv(kp, vp, table, L, kn, vn, P)
    d = dense(k2, table[0], 8)
    np.testing.assert_array_equal(d[:, 6:8], np.transpose(kn[0, :2], (1, 0, 2)))
    changed = ~np.all((kp == k2) | (np.isnan(kp) & np.isnan(k2)), axis=-1)
    assert int(changed.sum()) == 2 * kp.shape[1]


def test_attention_after_append_equals_dense_concatenation():
    """Decode attention over the appended cache at length L + T equals SDPA
    over the old keys concatenated with the new ones."""
    rng = np.random.default_rng(5)
    P, Hq, Hkv, D = 4, 4, 2, 8
    lens, T = [9, 0, 14], 3
    kp, vp, table, L, kn, vn = paged_case(rng, lens, T, Hkv=Hkv, D=D, P=P)
    k2, v2 = oracle.append_kv(kp, vp, table, L, kn, vn, P)
    q = rng.standard_normal((3, Hq, D))
    got = oracle.decode_attention(q, k2, v2, table, L + T, P, 0.3)
    for b, n in enumerate(lens):
        K = np.concatenate([dense(kp, table[b], n), np.transpose(kn[b], (1, 0, 2))], axis=1)
        V = np.concatenate([dense(vp, table[b], n), np.transpose(vn[b], (1, 0, 2))], axis=1)
        np.testing.assert_allclose(got[b], sdpa_dense(q[b], K, V, float(np.float32(0.3))), rtol=1e-12, atol=1e-14)


def test_integer_views_are_copied_bitwise():
    """bf16 data travels as int16 bit patterns; the append moves bits, NaN
    payloads included."""
    rng = np.random.default_rng(6)
    kp = rng.integers(-2**15, 2**15, size=(4, 1, 4, 8), dtype=np.int16)
    kn = rng.integers(-2**15, 2**15, size=(1, 2, 1, 8), dtype=np.int16)
    k2, _ = oracle.append_kv(kp, kp, np.array([[2, 0, 3]]), [3], kn, kn, 4)
    np.testing.assert_array_equal(k2[2, 0, 3], kn[0, 0, 0])
    np.testing.assert_array_equal(k2[0, 0, 0], kn[0, 1, 0])
    assert k2.dtype == np.int16


# ---------------------------------------------------------------------------
# Planted mistakes
# ---------------------------------------------------------------------------

def _append_pins_pass():
    try:
        for lens, T, P in CASES:
            test_dense_view_is_old_keys_then_new_keys(lens, T, P)
            test_only_the_new_rows_change(lens, T, P)
        test_append_to_empty_sequence_fills_identity_pages_in_order()
        test_rows_past_the_page_table_are_skipped()
        test_attention_after_append_equals_dense_concatenation()
    except (AssertionError, IndexError):
        return False
    return True


def test_unmutated_append_passes_the_pins():
    assert _append_pins_pass()


APPEND_MUTATIONS = {
    "position_off_by_one": ("new_position", lambda L, t: int(L) + t + 1),
    "overwrites_last_resident_key": ("new_position", lambda L, t: int(L) + t - 1),
    "page_table_ignored": ("page_and_slot", lambda row, pos, P: (pos // P, pos % P)),
    "page_and_slot_swapped": ("page_and_slot", lambda row, pos, P: (int(row[pos % P]), pos // P)),
    "every_token_at_the_first_new_slot": ("new_position", lambda L, t: int(L)),
}


@pytest.mark.parametrize("name", sorted(APPEND_MUTATIONS))
def test_planted_append_mistake_is_caught(name, monkeypatch):
    attr, fn = APPEND_MUTATIONS[name]
    monkeypatch.setattr(opc, attr, fn)
    assert not _append_pins_pass(), f"planted mistake {name} was not caught"
