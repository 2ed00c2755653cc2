"""Decode steps on the multi-token kernel: one new token per sequence, with 5
to 8 query heads per KV head (3 or 4 at head_dim 64 and 256, pages not a
multiple of 16, or fewer (sequence, KV head) streams than compute units; 2 at
head_dim 64) on
16-bit q and K/V, run as one 16-row block per KV head with both products on
the matrix cores, merged by the decode combine. Against the oracle at several
head dims, page sizes, windows and split counts, ragged, bimodal (one long
context among short ones: the split that fits one round of work-groups) and
single-key contexts; an empty context in the batch keeps the decode kernels;
the full long-context batch at 64 query heads in the planner's launch
configuration, sampled sequences against the oracle."""
import numpy as np
import pytest
import torch

from decode_attention_kv_04_amd import workloads as wl

from gpu_util import check, host64, oracle_for, run_lib, say

pytestmark = pytest.mark.gpu

CASES = [
    # B, H_q, H_kv, D, q/kv dtype, out, page, lengths, window
    (4, 64, 8, 128, "f16", "f16", 16, (1, 17, 3060, 5000), 0),
    (5, 40, 8, 128, "bf16", "f32", 32, (300, 4097, 2, 64, 1000), 700),     # G 5, window
    (2, 48, 8, 256, "f16", "f32", 16, (3000, 129), 0),                      # G 6, head_dim 256
    (4, 56, 8, 64, "bf16", "bf16", 8, (1, 8, 9, 2500), 100),               # G 7, head_dim 64, 8-token pages
    (3, 24, 8, 64, "f16", "f16", 24, (23, 24, 3001), 0),                    # G 3, head_dim 64, 24-token pages
    (2, 32, 8, 256, "bf16", "f32", 16, (2049, 700), 1000),                  # G 4, head_dim 256
    (3, 16, 4, 128, "f16", "f32", 8, (7, 1500, 260), 0),                    # G 4, 8-token pages
    (6, 16, 2, 128, "f16", "f32", 16, (1, 1, 1, 1, 1, 1), 0),               # one key each: the output is v
    (2, 64, 8, 128, "f16", "f32", 16, (257, 256), 1),                       # window 1: the new token's own v
    (16, 64, 8, 128, "f16", "f16", 16, (200,) * 15 + (20000,), 0),          # bimodal: 49 splits of 26 pages
    (16, 32, 8, 64, "bf16", "f32", 32, (300,) * 15 + (30000,), 0),         # bimodal at head_dim 64
    (3, 32, 8, 128, "bf16", "f32", 16, (3060, 100, 2049), 0),              # G 4, head_dim 128, 24 streams
    (3, 24, 8, 128, "f16", "f16", 16, (4097, 1, 640), 2000),               # G 3, head_dim 128, window
    (4, 16, 8, 64, "bf16", "f32", 16, (3000, 1, 257, 9000), 0),             # G 2, head_dim 64
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_decode_on_multi_kernel_matches_oracle(gpu, i):
    B, HQ, HKV, D, dt, out, P, lens, W = CASES[i]
    spec = wl.WorkloadSpec(f"mqdec{i}", B, HQ, HKV, D, dt, dt, out, P, ("list", lens), seed=7600 + i, window=W,
                           spike_frac=0.01)
    say(f"[decode on multi {i}] B={B} H={HQ}/{HKV} D={D} {dt}->{out} P={P} lens={lens} W={W}")
    w = wl.make_workload(spec, gpu)
    ref = oracle_for(w)
    # G 3-4 at head_dim 128 take it only with the planner's own split choice
    g34_d128 = HQ // HKV <= 4 and D == 128 and P % 16 == 0
    for ns in (0, 1, 3):
        got, plan = run_lib(w, num_splits=ns)
        assert plan.info.split_kernel == (1 if (g34_d128 and ns > 0) else 2)
        err, worst = check(got, ref, dt, out, f"decode on multi {i} splits={ns}")
        say(f"  splits {ns} -> {plan.max_splits} x {plan.pages_per_split} pages: rel L2 {err:.2e}, "
            f"worst sequence {worst:.2e}")
    # split + combine as two calls: the same bits as one run
    a, _ = run_lib(w, twin=False)
    b, _ = run_lib(w, two_phase=True, twin=False)
    assert torch.equal(a, b)


def test_single_key_returns_v(gpu):
    """One key per sequence: softmax weight 1, so the output is that key's V
    row (through f16 P = 1 exactly and fp32 accumulation)."""
    spec = wl.WorkloadSpec("mqdec_single", 3, 64, 8, 128, "f16", "f16", "f32", 16, ("list", (1, 1, 1)),
                           seed=7650)
    w = wl.make_workload(spec, gpu)
    got, plan = run_lib(w)
    assert plan.info.split_kernel == 2
    a = wl.to_numpy_inputs(w)
    for b in range(3):
        page = int(a["page_table"][b, 0])
        v = a["v_pool"][page, :, 0, :]                      # [H_kv][D] of key 0
        want = np.repeat(v, 8, axis=0)                      # every query head of a group
        np.testing.assert_array_equal(host64(got)[b], want.astype(np.float64))


def test_empty_context_keeps_the_decode_kernels(gpu):
    lens = (0, 3060, 1, 0)
    spec = wl.WorkloadSpec("mqdec_empty", len(lens), 64, 8, 128, "f16", "f16", "f16", 16, ("list", lens),
                           seed=7660)
    w = wl.make_workload(spec, gpu)
    got, plan = run_lib(w)
    assert plan.info.split_kernel == 1
    g = host64(got)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(g[b], np.zeros_like(g[b]))
    check(got, oracle_for(w), "f16", "f16", "empty context")


def test_long_batch_64_query_heads_full_size(gpu):
    """Batch 32, 64/8 heads, head_dim 128, fp16, 16k-32k tokens with spiky
    keys: the whole batch in the planner's launch configuration (one round of
    16-row work-groups), five sequences checked against the oracle; and
    against the matrix-core decode kernel on every sequence."""
    spec = wl.LONG_BATCH.replace(name="long_batch_g8", num_q_heads=64)
    w = wl.make_workload(spec, gpu)
    got, plan = run_lib(w)
    assert plan.info.split_kernel == 2
    say(f"  plan: pages/split {plan.pages_per_split} max splits {plan.max_splits} "
        f"work-groups {plan.info.split_work_groups}")
    rows = [0, 5, 13, 22, 31]
    idx = torch.tensor(rows, device=gpu)
    sub = got[idx]
    sub.f32_twin = got.f32_twin[idx]
    err, worst = check(sub, oracle_for(w, rows), "f16", "f16", "long batch, 64 query heads")
    say(f"  sampled sequences: rel L2 {err:.2e}, worst {worst:.2e}")
    other, oplan = run_lib(w, kernel="matrix")
    assert oplan.info.split_kernel == 1
    a, b = got.f32_twin.double(), other.f32_twin.double()
    per_seq = ((a - b).flatten(1).norm(dim=1) / b.flatten(1).norm(dim=1)).max().item()
    say(f"  against the decode kernel: worst per-sequence relative L2 {per_seq:.2e}")
    assert per_seq <= 1e-3
