"""Several new tokens per sequence (causal attention over the paged cache)
on the GPU through the C-ABI, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_kv_04_amd import workloads as wl

from gpu_util import TORCH_DT, check, host64, oracle_for, run_lib, say

pytestmark = pytest.mark.gpu


def spec_of(T, G, D, kv, out, P, lens, W, Hkv=2, seed=41):
    return wl.WorkloadSpec(f"mq_T{T}_G{G}_D{D}_{kv}_P{P}_W{W}", len(lens), G * Hkv, Hkv, D, kv, kv, out, P,
                           ("list", tuple(lens)), seed=seed, window=W, query_len=T)


GRID = [
    # T, G, D, kv, out, P, lens, W
    (2, 4, 128, "f16", "f16", 16, (2, 3, 100, 1000), 0),
    (3, 1, 64, "bf16", "f32", 16, (3, 17, 600), 0),
    (8, 8, 128, "bf16", "f32", 8, (8, 9, 31, 777), 0),
    (16, 4, 64, "f16", "f32", 32, (16, 50, 2000), 0),
    (16, 4, 128, "f16", "f16", 16, (16, 300, 3000), 100),
    (33, 3, 128, "bf16", "bf16", 24, (33, 34, 500), 0),
    (64, 2, 256, "bf16", "f32", 16, (64, 70, 1500), 0),
    (128, 4, 128, "f16", "f16", 16, (128, 130, 1000), 0),
    (128, 4, 128, "f16", "f32", 16, (200, 1500), 64),
    (5, 8, 256, "f16", "f32", 64, (5, 900), 7),
    # head_dim-128 row blocks over large pages (a tile inside one page; the
    # copies' page cursor steps within it) and the largest page size
    (40, 4, 128, "f16", "f32", 64, (40, 700, 5000), 0),
    (20, 2, 128, "bf16", "bf16", 1024, (20, 3000), 500),
    (130, 1, 128, "f16", "f16", 8, (130, 131, 2000), 0),
    # exactly 16 rows (four drafted tokens, GQA 4): one 64-row block with
    # three waves past the rows
    (4, 4, 128, "f16", "f16", 16, (4, 1000, 5000), 0),
    (4, 4, 64, "bf16", "f32", 32, (4, 2000), 300),
]


@pytest.mark.parametrize("T,G,D,kv,out,P,lens,W", GRID)
@pytest.mark.parametrize("splits", [0, 3])
def test_matches_oracle(gpu, T, G, D, kv, out, P, lens, W, splits):
    spec = spec_of(T, G, D, kv, out, P, lens, W)
    say(f"[multi] {spec.name} lens={lens} splits={splits}")
    w = wl.make_workload(spec, gpu)
    got, plan = run_lib(w, num_splits=splits)
    assert plan.info.split_kernel == 2
    err, worst = check(got, oracle_for(w), kv, out, spec.name)
    say(f"  rel L2 {err:.2e}, worst sequence {worst:.2e}")


# Forced block sizes at head_dim 64 and 128, whatever the row count: 64- and
# 128-row blocks for 16 rows or fewer (48 or more rows of the block empty),
# and 16-row blocks (wave 0 computes, waves 1-3 copy) for more rows.
@pytest.mark.parametrize("rows", ["16", "64", "128"])
@pytest.mark.parametrize("T,G,D,kv,out,P,lens,W", [GRID[0], GRID[1], GRID[3], GRID[4], GRID[13], GRID[14]])
def test_forced_block_shapes_match_oracle(gpu, rows, T, G, D, kv, out, P, lens, W):
    spec = spec_of(T, G, D, kv, out, P, lens, W)
    say(f"[multi] {spec.name} rows={rows}")
    w = wl.make_workload(spec, gpu)
    got, plan = run_lib(w, num_splits=2, rows_per_block=int(rows))
    assert plan.info.split_kernel == 2
    err, worst = check(got, oracle_for(w), kv, out, f"{spec.name} rows {rows}")
    say(f"  rel L2 {err:.2e}, worst sequence {worst:.2e}")


# 16 rows or fewer: the 16-row blocks (wave 0 computes, waves 1-3 only copy)
# do the same arithmetic per row as 64- and 128-row blocks whose other row
# groups are empty, so the outputs agree bitwise.
@pytest.mark.parametrize("T,G,D,kv,out,P,lens,W", [GRID[0], GRID[1], GRID[13], GRID[14]])
def test_few_row_blocks_equal_wider_blocks_bitwise(gpu, T, G, D, kv, out, P, lens, W):
    spec = spec_of(T, G, D, kv, out, P, lens, W)
    assert T * G <= 16
    say(f"[multi] {spec.name} 16-row vs wider blocks")
    w = wl.make_workload(spec, gpu)
    base, _ = run_lib(w, num_splits=2)
    for rows in ("64", "128"):
        got, _ = run_lib(w, num_splits=2, rows_per_block=int(rows))
        assert torch.equal(got, base), f"{rows}-row blocks differ from 16-row blocks"


# Both block sizes of the head_dim-128 kernel (one or two 16-row groups per
# wave), with forced splits so that blocks start and end inside pages and
# tiles; the two must agree with each other to the f16-P rounding.
@pytest.mark.parametrize("rows", ["64", "128"])
@pytest.mark.parametrize("T,G,D,kv,out,P,lens,W", [g for g in GRID if g[2] == 128])
def test_row_block_sizes_match_oracle(gpu, rows, T, G, D, kv, out, P, lens, W):
    spec = spec_of(T, G, D, kv, out, P, lens, W)
    say(f"[multi] {spec.name} rows={rows}")
    w = wl.make_workload(spec, gpu)
    got, plan = run_lib(w, num_splits=3, rows_per_block=int(rows))
    assert plan.info.split_kernel == 2
    err, worst = check(got, oracle_for(w), kv, out, f"{spec.name} rows {rows}")
    say(f"  rel L2 {err:.2e}, worst sequence {worst:.2e}")


def test_llama_shape_heads(gpu):
    spec = spec_of(24, 4, 128, "bf16", "f32", 16, (24, 900, 2500), 0, Hkv=8)
    w = wl.make_workload(spec, gpu)
    got, _ = run_lib(w)
    check(got, oracle_for(w), "bf16", "f32", spec.name)


def test_split_counts_agree_within_tolerance(gpu):
    spec = spec_of(16, 4, 128, "f16", "f32", 16, (16, 3000, 1234), 0)
    w = wl.make_workload(spec, gpu)
    ref = oracle_for(w)
    outs = []
    for ns in (1, 2, 7, 1_000_000):
        got, plan = run_lib(w, num_splits=ns)
        err, worst = check(got, ref, "f16", "f32", f"splits={ns}")
        say(f"[multi] splits={ns}: rel L2 {err:.2e}, worst sequence {worst:.2e}")
        outs.append(host64(got))
    # P enters P.V as f16 relative to each split's running max, so split
    # counts differ by about one f16 rounding of P (~2e-4), not by fp32 noise.
    for o in outs[1:]:
        assert oracle.relative_l2(o, outs[0]) < 1e-3


def test_two_phase_run_to_run_and_page_permutation_are_bitwise(gpu):
    spec = spec_of(12, 4, 128, "bf16", "f32", 16, (12, 700, 2100), 0)
    w = wl.make_workload(spec, gpu)
    a, plan = run_lib(w, num_splits=4)
    assert plan.max_splits > 1
    b, _ = run_lib(w, num_splits=4, two_phase=True)
    assert torch.equal(a, b)
    for _ in range(2):
        c, _ = run_lib(w, num_splits=4)
        assert torch.equal(a, c)
    g = torch.Generator().manual_seed(3)
    perm = torch.randperm(w.num_pages, generator=g).to(gpu)
    kp = torch.empty_like(w.k_pool)
    vp = torch.empty_like(w.v_pool)
    kp[perm] = w.k_pool
    vp[perm] = w.v_pool
    table = perm.to(torch.int32)[w.page_table.long()].contiguous()
    d, _ = run_lib(w, num_splits=4, k_pool=kp, v_pool=vp, page_table=table)
    assert torch.equal(a, d)


# bf16 P enters P.V as a hi + lo pair (error ~1e-6); f16 P is rounded once
# to f16 (~2e-4), while the single-query kernels keep P in fp32.
@pytest.mark.parametrize("kv,tol", [("bf16", 5e-6), ("f16", 1e-3)])
def test_each_token_matches_decode_over_the_cut_cache(gpu, kv, tol):
    """Token t of the multi-token pass agrees (within tolerance; other
    kernel) with a single-query decode whose length stops at its position."""
    T = 8
    spec = spec_of(T, 4, 128, kv, "f32", 16, (8, 500, 2049), 0)
    w = wl.make_workload(spec, gpu)
    multi, _ = run_lib(w)
    for t in range(T):
        cut = (w.seq_lens_host - T + t + 1).to(torch.int32)
        one, _ = run_lib(w, q=w.q[:, t].contiguous(), seq_lens=cut.to(gpu), seq_lens_host=cut, out_dtype="f32")
        rel = ((multi[:, t] - one).norm() / one.norm()).item()
        assert rel < tol, f"token {t}: {rel:.3e}"


@pytest.mark.parametrize("kv", ["f16", "bf16"])
def test_window_one_returns_each_tokens_own_value_bitwise(gpu, kv):
    T = 16
    spec = spec_of(T, 4, 128, kv, kv, 16, (16, 40, 333), 1)
    w = wl.make_workload(spec, gpu)
    got, _ = run_lib(w)
    for b, L in enumerate(spec.lengths[1]):
        pos = torch.arange(L - T, L)
        pages = w.page_table[b, (pos // 16).to(gpu)].long()
        v = w.v_pool[pages, :, (pos % 16).to(gpu)]              # [T][H_kv][D]
        assert torch.equal(got[b], v.repeat_interleave(4, dim=1))


def sampled_decode_oracle(w, pairs):
    """Oracle values for sampled (sequence, token) pairs: decode over the
    cache cut at the token's position (equal to the multi-token oracle)."""
    out = {}
    T = w.spec.query_len
    for b, t in pairs:
        a = wl.to_numpy_inputs(w, [b])
        L = int(a["seq_lens"][0])
        out[(b, t)] = oracle.decode_attention(a["q"][:, t], a["k_pool"], a["v_pool"], a["page_table"],
                                              np.array([L - T + t + 1]), a["page_size"], a["scale"],
                                              a["window"])[0]
    return out


# A few long contexts among short ones: the split length capped at the
# balance limit (the fit-the-round split, or the limit itself with more than
# one round of work-groups); every sequence against the oracle.
BIMODAL = [
    # T, G, Hkv, D, kv, out, P, lens
    (4, 4, 2, 128, "f16", "f16", 16, (200,) * 15 + (20000,)),        # fit: 79 splits of 16 pages
    (128, 4, 2, 128, "f16", "f32", 16, (300,) * 7 + (9000,)),       # 128-row blocks, fit
    (2, 8, 8, 128, "bf16", "f32", 16, (100,) * 62 + (30000,) * 2),   # 512 blocks: the limit itself
    (4, 4, 2, 64, "bf16", "bf16", 32, (64,) * 20 + (40000,)),        # head_dim 64
]


@pytest.mark.parametrize("T,G,Hkv,D,kv,out,P,lens", BIMODAL)
def test_bimodal_batches_match_oracle(gpu, T, G, Hkv, D, kv, out, P, lens):
    spec = spec_of(T, G, D, kv, out, P, lens, 0, Hkv=Hkv, seed=77)
    say(f"[multi bimodal] {spec.name} B={len(lens)} longest {max(lens)}")
    w = wl.make_workload(spec, gpu)
    got, plan = run_lib(w)
    assert plan.info.split_kernel == 2 and plan.max_splits > 2
    say(f"  pages/split {plan.pages_per_split}, max splits {plan.max_splits}, active {plan.info.active_units}")
    err, worst = check(got, oracle_for(w), kv, out, spec.name)
    say(f"  rel L2 {err:.2e}, worst sequence {worst:.2e}")


@pytest.mark.parametrize("name", ["suffix_prefill", "verify_long"])
def test_full_size_workloads_sampled(gpu, name):
    spec = wl.NAMED[name]
    say(f"[multi] {spec.name} full size")
    w = wl.make_workload(spec, gpu)
    got, plan = run_lib(w)
    say(f"  pages/split {plan.pages_per_split}, max splits {plan.max_splits}, "
        f"work-groups {plan.info.split_work_groups}")
    T = spec.query_len
    pairs = [(0, 0), (0, T - 1), (1, T // 2), (spec.batch - 1, T - 1), (spec.batch // 2, 1)]
    ref = sampled_decode_oracle(w, pairs)
    g = np.stack([host64(got[b, t]) for b, t in pairs])
    g32 = np.stack([host64(got.f32_twin[b, t]) for b, t in pairs])
    r = np.stack([ref[p] for p in pairs])
    check(g[:, None], r[:, None], spec.kv_dtype, spec.out_dtype, name, twin=g32[:, None])
    assert torch.isfinite(got).all()


def test_whole_context_is_new(gpu):
    spec = spec_of(40, 2, 64, "bf16", "f32", 8, (40, 40, 40), 0)
    w = wl.make_workload(spec, gpu)
    got, _ = run_lib(w)
    check(got, oracle_for(w), "bf16", "f32", "L == T")


# Dtype combinations the multi-token kernels do not take (f32 K/V, q and K/V
# of different types) and a forced vector kernel run the single-query
# kernels once per token.
PER_TOKEN = [
    # T, G, D, q, kv, out, P, lens, W, kernel
    (4, 4, 128, "f32", "f32", "f32", 16, (4, 100, 3000), 0, "auto"),
    (3, 2, 64, "f32", "f16", "f32", 16, (3, 700), 0, "auto"),
    (5, 8, 256, "bf16", "f32", "f32", 8, (5, 50, 999), 7, "auto"),
    (8, 4, 128, "f16", "f16", "f16", 16, (8, 2000, 333), 0, "vector"),
    (6, 2, 128, "bf16", "bf16", "f32", 32, (6, 4100), 300, "vector"),
    # windows whose page count changes with the token's alignment (regression:
    # the splits must cover the largest count over the tokens)
    (40, 2, 128, "f16", "f16", "f32", 8, (2407,), 100, "vector"),
    (9, 4, 64, "f32", "f32", "f32", 16, (700, 9, 4000), 33, "auto"),
]


@pytest.mark.parametrize("T,G,D,qd,kv,out,P,lens,W,kernel", PER_TOKEN)
@pytest.mark.parametrize("splits", [0, 3])
def test_per_token_path_matches_oracle(gpu, T, G, D, qd, kv, out, P, lens, W, kernel, splits):
    spec = wl.WorkloadSpec(f"pt_T{T}_G{G}_D{D}_{qd}_{kv}", len(lens), 2 * G, 2, D, qd, kv, out, P,
                           ("list", tuple(lens)), seed=43, window=W, query_len=T)
    say(f"[per-token] {spec.name} lens={lens} kernel={kernel} splits={splits}")
    w = wl.make_workload(spec, gpu)
    got, plan = run_lib(w, num_splits=splits, kernel=kernel)
    assert plan.info.split_kernel == 0
    err, worst = check(got, oracle_for(w), kv, out, spec.name)
    say(f"  rel L2 {err:.2e}, worst sequence {worst:.2e}")
    two, _ = run_lib(w, num_splits=splits, kernel=kernel, two_phase=True)
    assert torch.equal(got, two)


# Zero and negative scales on the multi-token kernels: a negative scale is
# folded into q (a sign flip, exact), a zero scale makes every score 0 (the
# output is the mean of the attended V rows).
@pytest.mark.parametrize("scale", [0.0, -0.0625, -1.3])
@pytest.mark.parametrize("T,G,D,kv,P,W", [(16, 4, 128, "f16", 16, 0), (3, 4, 64, "bf16", 32, 0),
                                          (4, 4, 256, "f16", 16, 100), (40, 2, 128, "bf16", 16, 0),
                                          (8, 1, 128, "f16", 8, 7)])
def test_zero_and_negative_scale(gpu, scale, T, G, D, kv, P, W):
    spec = spec_of(T, G, D, kv, kv, P, (T, T + 5, 300, 2000), W).replace(scale=scale)
    say(f"[multi] {spec.name} scale={scale}")
    w = wl.make_workload(spec, gpu)
    ref = oracle_for(w)
    for ns in (0, 3):
        got, plan = run_lib(w, num_splits=ns)
        assert plan.info.split_kernel == 2
        err, worst = check(got, ref, kv, kv, f"{spec.name} scale {scale} splits {ns}")
        say(f"  splits {ns}: rel L2 {err:.2e}, worst sequence {worst:.2e}")
