"""Planner invariants over seeded random parameters (host only, no GPU):
whatever kernel and schedule a plan picks, its launch fits the grid limits,
every sequence has between 1 and max_splits states, the workspace holds
every state, the fixed order keeps its chunk length, and the attended key
count follows from the lengths and the window. Rejections are only the
documented status codes."""
import math

import numpy as np
import pytest

from decode_attention_kv_04_amd import binding as B

from test_abi_plan import params, status_of


def draw(i):
    rng = np.random.default_rng(90000 + i)
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 48, 128]))
    Hkv = int(rng.choice([1, 2, 8]))
    D = int(rng.choice([64, 128, 256]))
    P = int(rng.choice([8, 16, 24, 32, 64]))
    kv = str(rng.choice(["f32", "f16", "bf16"]))
    q = kv if rng.random() < 0.7 else str(rng.choice(["f32", "f16", "bf16"]))
    T = int(rng.choice([0, 1, 1, 1, 2, 4, 16, 100]))
    Bn = int(rng.choice([0, 1, 3, 32, 300]))
    mp = int(rng.choice([16, 256, 4096]))
    lens = []
    for _ in range(Bn):
        if rng.random() < 0.1:
            L = 0
        else:
            L = int(min(mp * P, rng.choice([rng.integers(1, 300), rng.integers(1, 40000), mp * P])))
        lens.append(max(L, T if T > 1 else 0))
    lens = [min(L, mp * P) for L in lens]
    kw = dict(batch=Bn, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, page_size=P, max_pages_per_seq=mp,
              window=int(rng.choice([0, 0, 1, 100, 4096])), q_dtype=q, kv_dtype=kv,
              out_dtype=str(rng.choice(["f32", "f16", "bf16"])), query_len=T,
              num_splits=int(rng.choice([0, 0, 1, 3, 1000, 100000])),
              kernel=str(rng.choice(["auto", "auto", "vector", "matrix"])),
              rows_per_block=int(rng.choice([0, 0, 16, 64, 128])))
    if T <= 1 and rng.random() < 0.3:
        kw["fixed_chunk"] = P * int(rng.choice([1, 4, 64]))
    return kw, lens


def attended(L, T, W):
    keys = 0
    for t in range(max(T, 1)):
        pos = L - max(T, 1) + t
        keys += min(pos + 1, W) if W > 0 else pos + 1
    return keys


@pytest.mark.parametrize("chunk", range(8))
def test_random_plans_keep_their_invariants(lib, chunk):
    seen = {}
    for i in range(chunk * 400, (chunk + 1) * 400):
        kw, lens = draw(i)
        if any(L < kw["query_len"] for L in lens if kw["query_len"] > 1):
            continue
        st = status_of(params(**kw), lens)
        assert st in (B.DA_OK, B.DA_ERR_UNSUPPORTED), (i, kw, lens, st)
        if st != B.DA_OK:
            seen["unsupported"] = seen.get("unsupported", 0) + 1
            continue
        pl = B.decode_attn_plan_for_cus(params(**kw), lens, 256)
        info = pl.info
        Bn, Hkv, Hq, D, T = kw["batch"], kw["num_kv_heads"], kw["num_q_heads"], kw["head_dim"], kw["query_len"]
        seen[info.split_kernel] = seen.get(info.split_kernel, 0) + 1
        assert pl.max_splits >= 1 and pl.pages_per_split >= 1, (i, kw)
        assert info.attended_keys == sum(attended(L, T, kw["window"]) for L in lens), (i, kw, lens)
        for b in range(Bn):
            assert 1 <= pl.splits(b) <= pl.max_splits, (i, kw, b)
        if Bn and not info.balanced:
            assert info.split_work_groups % (Hkv * Bn) == 0, (i, kw)
            if info.split_kernel == 2:
                # grid (H_kv, row blocks x splits, B): y within 65535
                assert info.split_work_groups // (Hkv * Bn) <= 65535, (i, kw)
        if info.split_kernel == 2 and kw.get("fixed_chunk", 0) and any(lens):
            assert pl.pages_per_split == kw["fixed_chunk"] // kw["page_size"], (i, kw)
            assert info.chunks_per_work_group == 1
        if info.split_kernel == 2 and pl.max_splits > 1:
            need = Bn * max(T, 1) * Hq * pl.max_splits * (D + 2) * 4
            assert pl.workspace_bytes >= need, (i, kw)
        if info.split_kernel == 2 and T <= 1 and kw["kernel"] != "auto":
            raise AssertionError((i, kw, "a forced decode kernel ran the multi-token kernel"))
    assert seen.get(2, 0) > 0 and seen.get(0, 0) > 0, seen


def test_fixed_order_wide_group_chunks_fit_the_grid(lib):
    # 48 query heads over one KV head in forced 16-row blocks: 3 row blocks,
    # so at most 21845 chunks per sequence; a longer context is refused
    # rather than given longer chunks.
    kw = dict(batch=1, num_q_heads=48, num_kv_heads=1, fixed_chunk=16, max_pages_per_seq=70000, rows_per_block=16)
    assert status_of(params(**kw), [16 * 21845]) == B.DA_OK
    assert status_of(params(**kw), [16 * 21846]) == B.DA_ERR_UNSUPPORTED
    pl = B.decode_attn_plan_for_cus(params(**kw), [16 * 21845], 256)
    assert pl.pages_per_split == 1 and pl.max_splits == 21845
    assert math.ceil(48 / 16) * pl.max_splits <= 65535
