"""Pins for the CPU oracle: it is checked against computations other than
itself (scalar brute force, torch's float64 scaled_dot_product_attention,
closed forms, hand-derived cases, invariants), chosen so that a plausible
mistake in any of its steps fails at least one of them. The planted-mistake
tests at the end show that they do.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention_f64 as odm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


# ---------------------------------------------------------------------------
# Independent computations used as pins
# ---------------------------------------------------------------------------

def brute_force(q, k_pool, v_pool, table, lens, P, scale, window):
    """Scalar loops over the page table, one-pass softmax without a max shift,
    exact sums with math.fsum. Inputs: nested lists or arrays of floats."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(lens[b])
        # walk logical pages, keep keys whose distance from the newest key is
        # below the window
        keys = []
        for p in range((L + P - 1) // P):
            phys = int(table[b][p])
            for slot in range(P):
                t = p * P + slot
                if t >= L:
                    break
                if window > 0 and (L - 1 - t) >= window:
                    continue
                keys.append((phys, slot))
        for j in range(Hkv):
            for h in [j * G + i for i in range(G)]:  # the G consecutive heads of group j
                if not keys:
                    continue
                ws = []
                for phys, slot in keys:
                    s = sc * math.fsum(float(q[b, h, d]) * float(k_pool[phys, j, slot, d]) for d in range(D))
                    ws.append(math.exp(s))
                den = math.fsum(ws)
                for d in range(D):
                    out[b, h, d] = math.fsum(w * float(v_pool[phys, j, slot, d])
                                             for w, (phys, slot) in zip(ws, keys)) / den
    return out


def sdpa_f64(q, k_pool, v_pool, table, lens, P, scale, window):
    """torch's scaled_dot_product_attention in float64 on a dense copy of each
    sequence's keys, made by concatenating whole pages; GQA by repeating KV
    heads; the window by keeping the dense tail."""
    q = torch.as_tensor(np.asarray(q, dtype=np.float64))
    kp = torch.as_tensor(np.asarray(k_pool, dtype=np.float64))
    vp = torch.as_tensor(np.asarray(v_pool, dtype=np.float64))
    B, Hq, D = q.shape
    Hkv = kp.shape[1]
    out = torch.zeros((B, Hq, D), dtype=torch.float64)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        n = (L + P - 1) // P
        Kd = torch.cat([kp[int(table[b][p])] for p in range(n)], dim=1)[:, :L]  # [Hkv][L][D]
        Vd = torch.cat([vp[int(table[b][p])] for p in range(n)], dim=1)[:, :L]
        if window > 0 and L > window:
            Kd, Vd = Kd[:, L - window:], Vd[:, L - window:]
        Kd = Kd.repeat_interleave(Hq // Hkv, dim=0)
        Vd = Vd.repeat_interleave(Hq // Hkv, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(
            q[b][:, None, :], Kd, Vd, scale=float(np.float32(scale)))
        out[b] = o[:, 0, :]
    return out.numpy()


def rand_case(rng, B, Hq, Hkv, D, P, lens, window=0, shuffle=True, poison=True):
    """Random paged inputs: shuffled physical pages, NaN in every slot the
    attention must not read (unless poison=False)."""
    npages = [(L + P - 1) // P for L in lens]
    total = sum(npages)
    perm = rng.permutation(total) if shuffle else np.arange(total)
    maxp = max(1, max(npages))
    table = np.full((B, maxp), total, dtype=np.int64)
    off = 0
    for b, n in enumerate(npages):
        table[b, :n] = perm[off:off + n]
        off += n
    fill = np.nan if poison else 0.0
    kp = np.full((total + 1, Hkv, P, D), fill)
    vp = np.full((total + 1, Hkv, P, D), fill)
    for b, L in enumerate(lens):
        for t in range(L):
            if window > 0 and (L - 1 - t) >= window and poison:
                continue
            ph = table[b, t // P]
            kp[ph, :, t % P] = rng.standard_normal((Hkv, D))
            vp[ph, :, t % P] = rng.standard_normal((Hkv, D))
    q = rng.standard_normal((B, Hq, D))
    return q, kp, vp, table, np.array(lens)


def run_oracle(case, P, scale, window):
    q, kp, vp, table, lens = case
    return oracle.decode_attention(q, kp, vp, table, lens, P, scale, window)


# ---------------------------------------------------------------------------
# Brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,Hq,Hkv,D,P,lens,window", [
    (1, 1, 1, 4, 2, [1], 0),
    (1, 1, 1, 8, 4, [16], 0),
    (2, 4, 2, 4, 4, [5, 11], 0),
    (3, 4, 1, 8, 2, [7, 0, 13], 0),
    (2, 4, 4, 3, 4, [9, 16], 3),
    (2, 8, 2, 4, 4, [12, 2], 5),
    (1, 2, 1, 4, 8, [15], 15),
    (1, 2, 1, 4, 8, [15], 16),
    (2, 3, 1, 5, 2, [6, 3], 1),
    (1, 32, 2, 4, 4, [9], 0),           # 16 query heads per KV head
    (2, 48, 1, 4, 2, [5, 3], 2),        # 48 over one KV head, window
])
def test_oracle_matches_brute_force(B, Hq, Hkv, D, P, lens, window):
    rng = np.random.default_rng(B * 100 + D * 10 + P + window)
    case = rand_case(rng, B, Hq, Hkv, D, P, lens, window)
    scale = 1.0 / math.sqrt(D)
    ref = brute_force(*case, P, scale, window)
    got = run_oracle(case, P, scale, window)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# Library attention in float64
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,Hq,Hkv,D,P,lens,window", [
    (2, 8, 2, 64, 16, [200, 37], 0),
    (3, 4, 4, 128, 16, [1, 48, 300], 0),
    (2, 8, 4, 256, 16, [513, 96], 0),
    (2, 8, 8, 64, 32, [700, 33], 100),
    (1, 6, 2, 32, 8, [257], 256),
    (2, 128, 8, 64, 16, [300, 5], 0),   # 16 query heads per KV head
])
def test_oracle_matches_sdpa_f64(B, Hq, Hkv, D, P, lens, window):
    rng = np.random.default_rng(7 + D + P)
    case = rand_case(rng, B, Hq, Hkv, D, P, lens, window)
    scale = 1.0 / math.sqrt(D)
    ref = sdpa_f64(*case, P, scale, window)
    got = run_oracle(case, P, scale, window)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_oracle_matches_sdpa_on_long_spiky_heads():
    """The long-batch shape (32 query / 8 KV heads, D 128, fp16 values, 1 %
    of keys x8) on one 16k-token sequence."""
    from decode_attention_kv_04_amd import workloads
    spec = workloads.LONG_BATCH.replace(batch=1, lengths=("fixed", 16411), max_pages_per_seq=None)
    w = workloads.make_workload(spec, "cpu")
    a = workloads.to_numpy_inputs(w)
    args = (a["q"], a["k_pool"], a["v_pool"], a["page_table"], a["seq_lens"], a["page_size"], a["scale"], a["window"])
    ref = sdpa_f64(*args)
    got = oracle.decode_attention(*args)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------
# Closed forms and hand-derived cases
# ---------------------------------------------------------------------------

def load_golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", load_golden(), ids=lambda c: c["name"])
def test_oracle_hand_cases(case):
    got = oracle.decode_attention(np.array(case["q"]), np.array(case["k_pool"]), np.array(case["v_pool"]),
                                  np.array(case["page_table"]), np.array(case["seq_lens"]),
                                  case["page_size"], case["scale"], case["window"])
    np.testing.assert_allclose(got, np.array(case["expected"]), rtol=0, atol=case["tol"])


def test_single_key_returns_its_value():
    rng = np.random.default_rng(1)
    q, kp, vp, table, lens = rand_case(rng, 2, 4, 2, 16, 4, [1, 9], window=0)
    got = oracle.decode_attention(q, kp, vp, table, lens, 4, 0.25, 0)
    for h in range(4):
        assert np.array_equal(got[0, h], vp[table[0, 0], h // 2, 0])
    # window 1 keeps only the newest key
    got = oracle.decode_attention(q, kp, vp, table, np.array([9, 9]), 4, 0.25, 1)
    for h in range(4):
        assert np.array_equal(got[1, h], vp[table[1, 2], h // 2, 0])


def test_constant_values_come_back():
    rng = np.random.default_rng(2)
    q, kp, vp, table, lens = rand_case(rng, 1, 2, 1, 8, 4, [23], poison=False)
    v = rng.standard_normal(8)
    vp[:, 0, :, :] = v
    got = oracle.decode_attention(q, kp, vp, table, lens, 4, 0.3, 0)
    np.testing.assert_allclose(got[0], np.stack([v, v]), rtol=1e-14)


def test_zero_query_gives_mean_of_attended_values():
    rng = np.random.default_rng(3)
    L, W, P = 37, 11, 8
    q, kp, vp, table, lens = rand_case(rng, 1, 1, 1, 6, P, [L], window=W)
    q[:] = 0.0
    got = oracle.decode_attention(q, kp, vp, table, lens, P, 0.5, W)
    rows = [vp[table[0, t // P], 0, t % P] for t in range(L - W, L)]
    np.testing.assert_allclose(got[0, 0], np.mean(rows, axis=0), rtol=1e-13)


def test_two_keys_logistic_form():
    rng = np.random.default_rng(4)
    q, kp, vp, table, lens = rand_case(rng, 1, 1, 1, 5, 2, [2])
    sc = 0.7
    got = oracle.decode_attention(q, kp, vp, table, lens, 2, sc, 0)
    s0 = float(np.float32(sc)) * float(q[0, 0] @ kp[table[0, 0], 0, 0])
    s1 = float(np.float32(sc)) * float(q[0, 0] @ kp[table[0, 0], 0, 1])
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    expect = sig(s0 - s1) * vp[table[0, 0], 0, 0] + sig(s1 - s0) * vp[table[0, 0], 0, 1]
    np.testing.assert_allclose(got[0, 0], expect, rtol=1e-13)


def test_empty_sequence_is_zero_row():
    rng = np.random.default_rng(5)
    q, kp, vp, table, lens = rand_case(rng, 2, 2, 1, 4, 4, [0, 5])
    got = oracle.decode_attention(q, kp, vp, table, lens, 4, 0.5, 0)
    assert np.array_equal(got[0], np.zeros((2, 4)))
    assert np.all(np.isfinite(got[1]))


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def test_page_permutation_is_exact():
    rng = np.random.default_rng(6)
    q, kp, vp, table, lens = rand_case(rng, 2, 4, 2, 8, 4, [13, 30])
    base = oracle.decode_attention(q, kp, vp, table, lens, 4, 0.3, 0)
    perm = rng.permutation(kp.shape[0])          # new physical position of page p is perm[p]
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    got = oracle.decode_attention(q, kp2, vp2, perm[table], lens, 4, 0.3, 0)
    assert np.array_equal(got, base)


@pytest.mark.parametrize("shard", [1, 3, 7, 16, 1000])
def test_shard_merge_equals_direct(shard):
    rng = np.random.default_rng(8 + shard)
    case = rand_case(rng, 3, 4, 2, 16, 4, [0, 29, 64], window=0)
    a = oracle.decode_attention(*case, 4, 0.25, 0)
    b = oracle.decode_attention_sharded(*case, 4, 0.25, 0, shard)
    np.testing.assert_allclose(b, a, rtol=1e-13, atol=1e-15)


def test_shard_merge_with_window_and_spikes():
    rng = np.random.default_rng(9)
    q, kp, vp, table, lens = rand_case(rng, 2, 2, 1, 16, 8, [100, 50], window=40)
    kp[np.isfinite(kp)] *= 8.0  # large scores: the merge must rescale states correctly
    a = oracle.decode_attention(q, kp, vp, table, lens, 8, 0.25, 40)
    b = oracle.decode_attention_sharded(q, kp, vp, table, lens, 8, 0.25, 40, 9)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-14)
    ref = brute_force(q, kp, vp, table, lens, 8, 0.25, 40)
    np.testing.assert_allclose(a, ref, rtol=1e-11)


def test_window_equals_truncation():
    rng = np.random.default_rng(10)
    P, W = 4, 9
    q, kp, vp, table, lens = rand_case(rng, 2, 2, 2, 8, P, [23, 6], window=W)
    got = oracle.decode_attention(q, kp, vp, table, lens, P, 0.4, W)
    # re-page only the last W keys of each sequence into a fresh pool
    for b in range(2):
        L = int(lens[b])
        keep = list(range(max(0, L - W), L))
        n = len(keep)
        npg = (n + P - 1) // P
        kp2 = np.full((npg, 2, P, 8), np.nan)
        vp2 = np.full((npg, 2, P, 8), np.nan)
        for i, t in enumerate(keep):
            kp2[i // P, :, i % P] = kp[table[b, t // P], :, t % P]
            vp2[i // P, :, i % P] = vp[table[b, t // P], :, t % P]
        ref = oracle.decode_attention(q[b:b + 1], kp2, vp2, np.arange(npg)[None, :], np.array([n]), P, 0.4, 0)
        np.testing.assert_allclose(got[b:b + 1], ref, rtol=1e-14)


def test_window_at_least_length_is_no_window():
    rng = np.random.default_rng(11)
    case = rand_case(rng, 2, 2, 1, 8, 4, [17, 5])
    a = oracle.decode_attention(*case, 4, 0.4, 0)
    for W in (17, 18, 1000):
        assert np.array_equal(oracle.decode_attention(*case, 4, 0.4, W)[0], a[0])
    assert np.array_equal(oracle.decode_attention(*case, 4, 0.4, 5)[1], a[1])


@pytest.mark.parametrize("G", [3, 16])
def test_gqa_equals_mha_with_repeated_kv(G):
    rng = np.random.default_rng(12 + G)
    q, kp, vp, table, lens = rand_case(rng, 2, 2 * G, 2, 8, 4, [14, 21])
    a = oracle.decode_attention(q, kp, vp, table, lens, 4, 0.3, 0)
    kr = np.repeat(kp, G, axis=1)  # KV head j becomes heads jG..jG+G-1
    vr = np.repeat(vp, G, axis=1)
    b = oracle.decode_attention(q, kr, vr, table, lens, 4, 0.3, 0)
    assert np.array_equal(a, b)


def test_duplicated_tokens_leave_output_unchanged():
    rng = np.random.default_rng(13)
    P = 4
    q, kp, vp, table, lens = rand_case(rng, 1, 2, 1, 8, P, [11], poison=False)
    a = oracle.decode_attention(q, kp, vp, table, lens, P, 0.3, 0)
    L = 11
    n2 = 2 * L
    npg = (n2 + P - 1) // P
    kp2 = np.zeros((npg, 1, P, 8))
    vp2 = np.zeros((npg, 1, P, 8))
    for t in range(L):
        for c in range(2):
            i = 2 * t + c
            kp2[i // P, :, i % P] = kp[table[0, t // P], :, t % P]
            vp2[i // P, :, i % P] = vp[table[0, t // P], :, t % P]
    b = oracle.decode_attention(q, kp2, vp2, np.arange(npg)[None, :], np.array([n2]), P, 0.3, 0)
    np.testing.assert_allclose(b, a, rtol=1e-13)


def test_scaling_values_scales_output_exactly():
    rng = np.random.default_rng(14)
    q, kp, vp, table, lens = rand_case(rng, 2, 4, 2, 8, 4, [9, 30])
    a = oracle.decode_attention(q, kp, vp, table, lens, 4, 0.3, 0)
    b = oracle.decode_attention(q, kp, 2.0 * vp, table, lens, 4, 0.3, 0)
    assert np.array_equal(b, 2.0 * a)


def test_batch_independence():
    rng = np.random.default_rng(15)
    q, kp, vp, table, lens = rand_case(rng, 3, 2, 1, 8, 4, [9, 30, 1])
    a = oracle.decode_attention(q, kp, vp, table, lens, 4, 0.3, 0)
    for b in range(3):
        one = oracle.decode_attention(q[b:b + 1], kp, vp, table[b:b + 1], lens[b:b + 1], 4, 0.3, 0)
        assert np.array_equal(one[0], a[b])


def test_unattended_slots_do_not_matter():
    rng = np.random.default_rng(16)
    args = (2, 4, 2, 8, 4, [10, 27])
    q, kp, vp, table, lens = rand_case(np.random.default_rng(16), *args, window=12, poison=True)
    assert np.isnan(kp).any() and np.isnan(vp).any()
    kp2 = np.where(np.isnan(kp), rng.standard_normal(kp.shape) * 100, kp)
    vp2 = np.where(np.isnan(vp), rng.standard_normal(vp.shape) * 100, vp)
    a = oracle.decode_attention(q, kp, vp, table, lens, 4, 0.3, 12)
    b = oracle.decode_attention(q, kp2, vp2, table, lens, 4, 0.3, 12)
    assert np.all(np.isfinite(a))
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# Reference rounding and the pages' accuracy figure
# ---------------------------------------------------------------------------

def test_round_to_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(17)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ours = oracle.round_to(x.astype(np.float64), "bf16")
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, lib)


def test_round_to_f16_and_f32_match_numpy_casts():
    rng = np.random.default_rng(18)
    x = rng.standard_normal(10000) * 3
    assert np.array_equal(oracle.round_to(x, "f16"), x.astype(np.float16).astype(np.float64))
    assert np.array_equal(oracle.round_to(x, "f32"), x.astype(np.float32).astype(np.float64))


def test_relative_l2_definition():
    ref = np.array([[3.0, 4.0]])
    assert oracle.relative_l2(ref + np.array([[0.0, 0.5]]), ref) == pytest.approx(0.1)
    assert oracle.relative_l2(ref, ref) == 0.0
    assert oracle.relative_l2_per_row(np.stack([ref, 2 * ref]), np.stack([ref, ref]))[1] == pytest.approx(1.0)


@pytest.mark.parametrize("L", [256, 3060])
def test_fp16_output_rounding_is_the_pages_accuracy_figure(L):
    """The sharded-nest commit message (TVM pull 20426) reports 0.02 %
    relative L2 against an f64 reference, "to f16 rounding". Rounding the
    exact output of the Llama-3.1-8B shape to fp16 alone gives that figure."""
    from decode_attention_kv_04_amd import workloads
    spec = workloads.LLAMA8B_3060.replace(lengths=("fixed", L))
    a = workloads.to_numpy_inputs(workloads.make_workload(spec, "cpu"))
    ref = oracle.decode_attention(a["q"], a["k_pool"], a["v_pool"], a["page_table"], a["seq_lens"],
                                  a["page_size"], a["scale"], a["window"])
    err = oracle.relative_l2(oracle.round_to(ref, "f16"), ref)
    assert 1.0e-4 < err < 3.0e-4


# ---------------------------------------------------------------------------
# Planted mistakes: each must be caught by the pins above
# ---------------------------------------------------------------------------

def _pin_suite_passes():
    """A small brute-force / SDPA pin run; True if the oracle passes it."""
    for seed, (B, Hq, Hkv, D, P, lens, W) in enumerate([
        (2, 4, 2, 4, 4, [6, 11], 0),
        (2, 4, 2, 4, 4, [9, 14], 5),
        (1, 2, 1, 4, 2, [2], 0),
    ]):
        rng = np.random.default_rng(100 + seed)
        case = rand_case(rng, B, Hq, Hkv, D, P, lens, W)
        ref = brute_force(*case, P, 0.5, W)
        try:
            got = run_oracle(case, P, 0.5, W)
            sh = oracle.decode_attention_sharded(*case, P, 0.5, W, 3)
        except Exception:
            return False
        if not (np.allclose(got, ref, rtol=1e-12, atol=1e-14) and np.allclose(sh, ref, rtol=1e-12, atol=1e-14)):
            return False
    return True


def test_unmutated_oracle_passes_the_pins():
    assert _pin_suite_passes()


MUTATIONS = {
    "gqa_modulo_mapping": ("kv_head_of", lambda h, g: h % g),
    "window_off_by_one_short": ("attended_range",
                                lambda L, w: (L - w + 1, L) if (w > 0 and L > w) else (0, L)),
    "window_off_by_one_long": ("attended_range",
                               lambda L, w: (max(0, L - w - 1), L) if (w > 0 and L > w) else (0, L)),
    "window_ignored": ("attended_range", lambda L, w: (0, L)),
    "page_index_swapped": ("gather_rows",
                           lambda pool, row, j, t0, t1, P: pool[np.asarray(row)[np.arange(t0, t1) % P],
                                                                j, np.arange(t0, t1) // P].astype(np.float64)),
    "page_table_ignored": ("gather_rows",
                           lambda pool, row, j, t0, t1, P: pool[np.arange(t0, t1) // P, j,
                                                                np.arange(t0, t1) % P].astype(np.float64)),
    "scale_dropped": ("attend_one",
                      lambda qv, K, V, s: (lambda e: (e @ V) / e.sum())(np.exp(K @ qv - (K @ qv).max()))
                      if K.shape[0] else np.zeros(V.shape[1])),
    "keys_as_values": ("attend_one",
                       lambda qv, K, V, s: (lambda e: (e @ K) / e.sum())(np.exp(s * (K @ qv) - (s * (K @ qv)).max()))
                       if K.shape[0] else np.zeros(V.shape[1])),
    "mean_instead_of_softmax_normaliser": ("attend_one",
                                           lambda qv, K, V, s: (lambda e: (e @ V) / len(e))(np.exp(s * (K @ qv) - (s * (K @ qv)).max()))
                                           if K.shape[0] else np.zeros(V.shape[1])),
    "merge_weight_sign_flipped": ("merge_states", None),
}


def _bad_merge(states):
    D = states[0][2].shape[0]
    M = max(m for m, _, _ in states)
    if M == -math.inf:
        return np.zeros(D)
    num = np.zeros(D)
    den = 0.0
    for m, l, O in states:
        if m == -math.inf:
            continue
        w = math.exp(M - m)
        num += w * O
        den += w * l
    return num / den


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    if fn is None:
        fn = _bad_merge
    monkeypatch.setattr(odm, attr, fn)
    assert not _pin_suite_passes(), f"planted mistake {name} was not caught"
