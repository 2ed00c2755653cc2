"""Fixed-order mode on the GPU: the output is bitwise the same for every
split count (the pages' split-vs-unsplit bit-identity), within tolerance of
the oracle, and independent of workspace contents and of run order."""
import numpy as np
import pytest
import torch

from decode_attention_kv_04_amd import workloads as wl

from gpu_util import check, oracle_for, run_lib, say

pytestmark = pytest.mark.gpu

SPLITS = [1, 2, 3, 7, 0, 1_000_000]   # 0 = the planner decides


def all_split_counts_agree(w, chunk, splits=SPLITS, **kw):
    outs = []
    for ns in splits:
        out, plan = run_lib(w, num_splits=ns, fixed_chunk=chunk, **kw)
        assert plan.info.chunks_per_work_group >= 1
        say(f"  splits={ns}: chunks/group {plan.info.chunks_per_work_group}, "
            f"work-groups {plan.info.split_work_groups}, chunks {plan.max_splits}")
        outs.append(out)
    for ns, o in zip(splits[1:], outs[1:]):
        assert torch.equal(o, outs[0]), f"num_splits={ns} differs from num_splits={splits[0]}"
    return outs[0]


@pytest.mark.parametrize("kernel", ["auto", "vector"])
@pytest.mark.parametrize("name,chunk", [("tiny", 16), ("tiny", 64), ("llama8b_3060", 256),
                                        ("llama8b_3060", 1024), ("wide_gqa", 512)])
def test_named_workloads_bitwise_across_splits(gpu, name, chunk, kernel):
    spec = wl.NAMED[name]
    say(f"[fixed-order] {spec.name} chunk={chunk} kernel={kernel}")
    w = wl.make_workload(spec, gpu)
    out = all_split_counts_agree(w, chunk, kernel=kernel)
    check(out, oracle_for(w), spec.kv_dtype, spec.out_dtype, f"{name} fixed {chunk}")


# Where the decode kernels are weak (group width 8, or 3-4 query heads at
# head_dim 64 / 256 or 8-token pages) the mode runs on the multi-token kernel:
# one chunk per work-group, rows of one chunk written by the split pass.
MULTI_FIXED = [
    # B, H_q, H_kv, D, dtype, out, P, lengths, window, chunk
    (4, 64, 8, 128, "f16", "f16", 16, (3060, 100, 9000, 1), 0, 256),
    (3, 32, 8, 64, "bf16", "f32", 16, (5000, 17, 2049), 0, 1024),
    (3, 48, 8, 256, "f16", "f32", 16, (40, 3000, 700), 500, 128),
    (2, 16, 4, 128, "f16", "f32", 8, (6000, 333), 0, 64),
    (2, 64, 8, 128, "bf16", "bf16", 32, (70000, 12), 4096, 2048),
    (3, 128, 8, 128, "f16", "f16", 16, (3060, 0, 9000), 0, 512),            # G 16, an empty context
    (2, 48, 1, 64, "bf16", "f32", 16, (4000, 260), 1000, 256),            # G 48 (one KV head)
]


@pytest.mark.parametrize("i", range(len(MULTI_FIXED)))
def test_multi_token_kernel_bitwise_across_splits(gpu, i):
    B, HQ, HKV, D, dt, out, P, lens, W, chunk = MULTI_FIXED[i]
    spec = wl.WorkloadSpec(f"mqfixed{i}", B, HQ, HKV, D, dt, dt, out, P, ("list", lens), seed=7800 + i, window=W,
                           spike_frac=0.01)
    say(f"[fixed-order, multi-token kernel {i}] B={B} H={HQ}/{HKV} D={D} {dt} P={P} lens={lens} W={W} chunk={chunk}")
    w = wl.make_workload(spec, gpu)
    _, plan = run_lib(w, fixed_chunk=chunk, twin=False)
    assert plan.info.split_kernel == 2 and plan.info.chunks_per_work_group == 1
    got = all_split_counts_agree(w, chunk)
    check(got, oracle_for(w), dt, out, f"multi fixed {i}")
    # two-phase (split, then combine) equals run
    b, _ = run_lib(w, fixed_chunk=chunk, two_phase=True)
    assert torch.equal(b, got)


def test_mixed_window_full_size_bitwise_across_splits(gpu, mixed_window):
    w, ref = mixed_window
    say(f"[fixed-order] {w.spec.name} full size")
    out = all_split_counts_agree(w, 1024, splits=[1, 4, 0, 1_000_000])
    check(out, ref, w.spec.kv_dtype, w.spec.out_dtype, "mixed_window fixed")


@pytest.mark.parametrize("kernel", ["auto", "vector"])
def test_long_batch_full_size_bitwise_across_splits(gpu, long_batch, kernel):
    w, ref = long_batch
    say(f"[fixed-order] {w.spec.name} full size kernel={kernel}")
    out = all_split_counts_agree(w, 1024, splits=[0, 1, 5, 1_000_000], kernel=kernel)
    check(out, ref, w.spec.kv_dtype, w.spec.out_dtype, "long_batch fixed")


GRID = [
    # G, D, q, kv, out, P
    (1, 64, "f32", "f32", "f32", 16),
    (2, 256, "bf16", "bf16", "f32", 16),
    (4, 128, "f16", "f16", "f16", 16),
    (4, 128, "f32", "f16", "f32", 8),
    (8, 64, "bf16", "bf16", "bf16", 32),
    (8, 128, "f16", "f16", "f32", 24),
    (3, 128, "bf16", "bf16", "f32", 64),
]


@pytest.mark.parametrize("G,D,qd,kvd,od,P", GRID)
def test_grid_bitwise_across_splits(gpu, G, D, qd, kvd, od, P):
    lens = (0, 1, P - 1, P, 3 * P + 1, 2000, 4099)
    spec = wl.WorkloadSpec(f"fx_g{G}_d{D}_{kvd}", len(lens), 2 * G, 2, D, qd, kvd, od, P, ("list", lens), seed=31)
    say(f"[fixed-order] {spec.name} P={P}")
    w = wl.make_workload(spec, gpu)
    out = all_split_counts_agree(w, 8 * P)
    check(out, oracle_for(w), kvd, od, spec.name)
    assert torch.all(out[0] == 0)   # an empty sequence gives a zero row


@pytest.mark.parametrize("kernel", ["auto", "vector"])
@pytest.mark.parametrize("W", [1, 100, 1000, 4096])
def test_window_bitwise_across_splits(gpu, W, kernel):
    spec = wl.LLAMA8B_3060.replace(batch=3, lengths=("list", (3060, 777, 5000)), window=W)
    say(f"[fixed-order] window {W} kernel={kernel}")
    w = wl.make_workload(spec, gpu)
    out = all_split_counts_agree(w, 256, kernel=kernel)
    check(out, oracle_for(w), "f16", "f16", f"window {W}")


def test_one_page_chunks_and_one_chunk(gpu):
    spec = wl.WIDE_GQA.replace(head_dim=128)
    w = wl.make_workload(spec, gpu)
    ref = oracle_for(w)
    for chunk in (16, 1 << 16):                  # one page per chunk; every sequence in one chunk
        say(f"[fixed-order] chunk {chunk}")
        out = all_split_counts_agree(w, chunk, splits=[1, 3, 1_000_000])
        check(out, ref, spec.kv_dtype, spec.out_dtype, f"chunk {chunk}")


def test_matrix_and_vector_kernels_agree_within_tolerance(gpu):
    w = wl.make_workload(wl.LLAMA8B_3060.replace(batch=2, lengths=("list", (3060, 1200)), out_dtype="f32"), gpu)
    a, pa = run_lib(w, fixed_chunk=512)
    b, pb = run_lib(w, fixed_chunk=512, kernel="vector")
    assert pa.info.split_kernel == 1 and pb.info.split_kernel == 0
    assert ((a - b).norm() / b.norm()).item() < 2e-6


def test_two_phase_equals_run_and_workspace_contents_do_not_matter(gpu):
    w = wl.make_workload(wl.LLAMA8B_3060.replace(batch=2, lengths=("list", (3060, 1200))), gpu)
    a, _ = run_lib(w, fixed_chunk=256, num_splits=3)
    b, _ = run_lib(w, fixed_chunk=256, num_splits=3, two_phase=True)
    assert torch.equal(a, b)
    # run_lib fills the workspace with NaN bit patterns before each call
    for _ in range(3):
        c, _ = run_lib(w, fixed_chunk=256, num_splits=2)
        assert torch.equal(a, c)


def test_long_context_f32(gpu):
    spec = wl.WorkloadSpec("fx_long_f32", 1, 8, 2, 128, "f32", "f32", "f32", 16, ("list", (65536,)), seed=32)
    w = wl.make_workload(spec, gpu)
    out = all_split_counts_agree(w, 2048, splits=[1, 2, 0, 1_000_000])
    check(out, oracle_for(w), "f32", "f32", "65536 f32")
