"""Pins for the multi-token (causal) oracle: T = 1 is the decode oracle,
each new token equals decode over the cache truncated at its position,
float64 SDPA with an explicit causal+window mask, scalar brute force, a
closed form, and planted mistakes that must fail them."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import multi_query as omq


def case(rng, B, T, Hq, Hkv, D, P, lens, window=0):
    """Shuffled pages, every slot a sequence attends filled, the rest NaN."""
    npages = [(L + P - 1) // P for L in lens]
    total = sum(npages)
    perm = rng.permutation(total)
    table = np.full((B, max(1, max(npages))), total, dtype=np.int64)
    off = 0
    for b, n in enumerate(npages):
        table[b, :n] = perm[off:off + n]
        off += n
    kp = np.full((total + 1, Hkv, P, D), np.nan)
    vp = np.full_like(kp, np.nan)
    for b, L in enumerate(lens):
        first = max(0, L - T + 1 - window) if window > 0 else 0     # earliest key any new token sees
        for t in range(first, L):
            kp[table[b, t // P], :, t % P] = rng.standard_normal((Hkv, D))
            vp[table[b, t // P], :, t % P] = rng.standard_normal((Hkv, D))
    q = rng.standard_normal((B, T, Hq, D))
    return q, kp, vp, table, np.array(lens)


def brute(q, kp, vp, table, lens, P, scale, window):
    """Scalar loops: key position s is seen by the query at position p iff
    s <= p and (no window or p - s < window); exp without a max shift."""
    B, T, Hq, D = q.shape
    Hkv = kp.shape[1]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((B, T, Hq, D))
    for b in range(B):
        L = int(lens[b])
        for t in range(T):
            p = L - T + t
            keys = [s for s in range(L) if s <= p and (window == 0 or p - s < window)]
            for h in range(Hq):
                j = h // G
                ws = [math.exp(sc * math.fsum(q[b, t, h, d] * kp[table[b, s // P], j, s % P, d] for d in range(D)))
                      for s in keys]
                den = math.fsum(ws)
                for d in range(D):
                    out[b, t, h, d] = math.fsum(w * vp[table[b, s // P], j, s % P, d] for w, s in zip(ws, keys)) / den
    return out


def sdpa_masked(q, kp, vp, table, lens, P, scale, window):
    """torch float64 SDPA over each sequence's dense keys (pages
    concatenated whole) with a boolean mask built from positions."""
    B, T, Hq, D = q.shape
    Hkv = kp.shape[1]
    out = np.zeros((B, T, Hq, D))
    for b in range(B):
        L = int(lens[b])
        n = (L + P - 1) // P
        K = torch.cat([torch.as_tensor(kp[table[b, i]]) for i in range(n)], dim=1)[:, :L]
        V = torch.cat([torch.as_tensor(vp[table[b, i]]) for i in range(n)], dim=1)[:, :L]
        K = torch.nan_to_num(K).repeat_interleave(Hq // Hkv, dim=0)            # masked keys may be NaN
        V = torch.nan_to_num(V).repeat_interleave(Hq // Hkv, dim=0)
        pos_q = torch.arange(L - T, L)[:, None]
        pos_k = torch.arange(L)[None, :]
        mask = pos_k <= pos_q
        if window > 0:
            mask &= (pos_q - pos_k) < window
        Q = torch.as_tensor(q[b]).transpose(0, 1)                                # [Hq][T][D]
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=float(np.float32(scale)))
        out[b] = o.transpose(0, 1).numpy()
    return out


SHAPES = [
    # B, T, Hq, Hkv, D, P, lens, window
    (1, 1, 2, 1, 4, 4, [7], 0),
    (1, 3, 2, 1, 4, 4, [3], 0),            # the new tokens are the whole context
    (2, 4, 4, 2, 4, 2, [9, 4], 0),
    (2, 5, 4, 1, 3, 4, [13, 6], 3),
    (3, 2, 2, 2, 4, 4, [2, 11, 17], 1),
    (1, 6, 4, 4, 2, 2, [20], 4),
    (2, 3, 32, 2, 4, 4, [7, 3], 0),        # 16 query heads per KV head
    (1, 2, 24, 1, 3, 2, [9], 3),           # 24 over one KV head, window
]


@pytest.mark.parametrize("B,T,Hq,Hkv,D,P,lens,W", SHAPES)
def test_matches_brute_force(B, T, Hq, Hkv, D, P, lens, W):
    rng = np.random.default_rng(B * 31 + T)
    c = case(rng, B, T, Hq, Hkv, D, P, lens, W)
    got = oracle.prefill_attention(*c, P, 0.7, W)
    np.testing.assert_allclose(got, brute(*c, P, 0.7, W), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("T,W", [(1, 0), (7, 0), (16, 0), (16, 5), (33, 64), (64, 16)])
def test_matches_masked_sdpa(T, W):
    rng = np.random.default_rng(100 + T + W)
    c = case(rng, 3, T, 8, 2, 16, 8, [T, T + 37, 300], W)
    got = oracle.prefill_attention(*c, 8, 0.25, W)
    np.testing.assert_allclose(got, sdpa_masked(*c, 8, 0.25, W), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("W", [0, 3, 50])
def test_one_new_token_is_the_decode_oracle(W):
    rng = np.random.default_rng(7)
    q, kp, vp, table, lens = case(rng, 3, 1, 4, 2, 8, 4, [1, 30, 61], W)
    got = oracle.prefill_attention(q, kp, vp, table, lens, 4, 0.5, W)
    ref = oracle.decode_attention(q[:, 0], kp, vp, table, lens, 4, 0.5, W)
    np.testing.assert_array_equal(got[:, 0], ref)


@pytest.mark.parametrize("W", [0, 4])
def test_each_token_is_decode_over_the_truncated_cache(W):
    """Causality: new token t equals single-query decode on the same pages
    with the length cut at its own position + 1."""
    rng = np.random.default_rng(8)
    T = 6
    q, kp, vp, table, lens = case(rng, 2, T, 4, 2, 8, 4, [11, 25], W)
    got = oracle.prefill_attention(q, kp, vp, table, lens, 4, 0.5, W)
    for t in range(T):
        cut = lens - T + t + 1
        ref = oracle.decode_attention(q[:, t], kp, vp, table, cut, 4, 0.5, W)
        np.testing.assert_array_equal(got[:, t], ref)


def test_future_keys_do_not_matter():
    rng = np.random.default_rng(9)
    T = 5
    q, kp, vp, table, lens = case(rng, 1, T, 2, 1, 4, 4, [12], 0)
    got = oracle.prefill_attention(q, kp, vp, table, lens, 4, 1.0, 0)
    # poison the keys after the third new token; rows 0..2 must not change
    kp2, vp2 = kp.copy(), vp.copy()
    for s in range(12 - T + 3, 12):
        kp2[table[0, s // 4], :, s % 4] = np.nan
        vp2[table[0, s // 4], :, s % 4] = np.nan
    got2 = oracle.prefill_attention(q, kp2, vp2, table, lens, 4, 1.0, 0)
    np.testing.assert_array_equal(got[:, :3], got2[:, :3])
    assert np.isnan(got2[:, 3:]).all()


def test_closed_form_two_tokens_one_dim():
    """L = T = 2, D = 1: token 0 sees only key 0, so its output is v0; token
    1 sees both: sigma(s0 - s1) v0 + sigma(s1 - s0) v1 with s_i = q1 k_i."""
    q = np.array([[[[0.3]], [[1.5]]]])                    # [1][2][1][1]
    kp = np.array([[[[2.0], [-1.0]]]])                    # one page [1][1][2][1]
    vp = np.array([[[[10.0], [4.0]]]])
    out = oracle.prefill_attention(q, kp, vp, np.array([[0]]), np.array([2]), 2, 1.0, 0)
    assert out[0, 0, 0, 0] == 10.0
    s0, s1 = 1.5 * 2.0, 1.5 * -1.0
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    assert abs(out[0, 1, 0, 0] - (w0 * 10.0 + (1.0 - w0) * 4.0)) < 1e-13


def test_too_few_keys_is_an_error():
    rng = np.random.default_rng(10)
    q, kp, vp, table, lens = case(rng, 1, 3, 1, 1, 2, 2, [3], 0)
    with pytest.raises(ValueError):
        oracle.prefill_attention(q, kp, vp, table, np.array([2]), 2, 1.0, 0)


# ---------------------------------------------------------------------------
# Planted mistakes
# ---------------------------------------------------------------------------

def _pins_pass():
    try:
        for args in SHAPES:
            test_matches_brute_force(*args)
        test_each_token_is_decode_over_the_truncated_cache(0)
        test_each_token_is_decode_over_the_truncated_cache(4)
        test_closed_form_two_tokens_one_dim()
    except (AssertionError, IndexError, ValueError):
        return False
    return True


def test_unmutated_oracle_passes_the_pins():
    assert _pins_pass()


MUTATIONS = {
    "sees_the_next_token": ("query_position", lambda L, T, t: L - T + t + 1),
    "does_not_see_itself": ("query_position", lambda L, T, t: L - T + t - 1),
    "positions_from_the_start": ("query_position", lambda L, T, t: t),
    "no_causal_mask": ("query_keys", lambda L, T, t, w: omq.attended_range(L, w)),
    "window_from_the_newest_token": ("query_keys",
                                     lambda L, T, t, w: (omq.attended_range(L, w)[0], L - T + t + 1)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(omq, attr, fn)
    assert not _pins_pass(), f"planted mistake {name} was not caught"
