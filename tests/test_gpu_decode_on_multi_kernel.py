"""Decode steps on the multi-token kernel: one new token per sequence, with 5
to 8 query heads per KV head (3 or 4 at head_dim 64 and 256, pages not a
multiple of 16, or fewer (sequence, KV head) streams than compute units; 2 at
head_dim 64), and every group wider than 8 (16 query heads per KV head as in
a 128-over-8 model, 32 to 64 over one KV head), on 16-bit q and K/V: one
16-row block per KV head (more rows: blocks of 64 or 128) with both products
on the matrix cores, merged by the decode combine. Against the oracle at
several head dims, page sizes, windows, split counts and forced block sizes,
ragged, bimodal (one long context among short ones: the split that fits one
round of work-groups), single-key and empty contexts (rows of zeros); the
full long-context batch at 64 and 128 query heads in the planner's launch
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
    (3, 128, 8, 128, "f16", "f16", 16, (3060, 1, 9000), 0),                # G 16
    (2, 96, 8, 128, "bf16", "f32", 32, (5000, 700), 1000),                 # G 12, window
    (2, 48, 1, 128, "f16", "f32", 16, (4097, 300), 0),                     # G 48, one KV head
    (2, 64, 2, 64, "bf16", "bf16", 8, (2, 6000), 0),                       # G 32, head_dim 64
    (2, 32, 2, 256, "f16", "f32", 16, (1500, 333), 200),                   # G 16, head_dim 256
    (2, 64, 1, 256, "bf16", "f32", 16, (2500, 17), 0),                     # G 64 at head_dim 256: 64-row block
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


@pytest.mark.parametrize("HQ,chunk", [(64, 0), (64, 256), (128, 0), (128, 512)])
def test_empty_context_rows_are_zero(gpu, HQ, chunk):
    """An empty context has no keys: its block reads no page and its rows are
    written as zeros, also in a batch that splits and in the fixed order."""
    lens = (0, 3060, 1, 0, 20000)
    spec = wl.WorkloadSpec(f"mqdec_empty{HQ}", len(lens), HQ, 8, 128, "f16", "f16", "f16", 16, ("list", lens),
                           seed=7660 + HQ + chunk)
    w = wl.make_workload(spec, gpu)
    say(f"[empty contexts on the multi-token kernel] H={HQ}/8 lens={lens} chunk={chunk}")
    got, plan = run_lib(w, fixed_chunk=chunk)
    assert plan.info.split_kernel == 2 and plan.max_splits > 1
    g = host64(got)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(g[b], np.zeros_like(g[b]))
    check(got, oracle_for(w), "f16", "f16", "empty context")


@pytest.mark.parametrize("rows", [16, 64, 128])
def test_wide_group_block_sizes_agree(gpu, rows):
    """48 query heads over one KV head in 16-, 64- and 128-row blocks (three
    blocks reading the same keys, one with 16 empty rows, one with 80): each
    against the oracle, and all within fp32 rounding of the planner's own."""
    spec = wl.WorkloadSpec("mqdec_rows", 3, 48, 1, 128, "bf16", "bf16", "f32", 16, ("list", (3000, 40, 12000)),
                           seed=7670, spike_frac=0.01)
    w = wl.make_workload(spec, gpu)
    say(f"[wide group, {rows}-row blocks]")
    ref = oracle_for(w)
    got, plan = run_lib(w, rows_per_block=rows)
    assert plan.info.split_kernel == 2
    assert plan.info.split_work_groups == 3 * -(-48 // rows) * plan.max_splits  # B x row blocks x splits
    check(got, ref, "bf16", "f32", f"{rows}-row blocks")
    auto, _ = run_lib(w)
    a, b = host64(got), host64(auto)
    assert np.linalg.norm(a - b) <= 2e-6 * np.linalg.norm(b)


@pytest.mark.parametrize("HQ", [64, 128])
def test_long_batch_wide_groups_full_size(gpu, HQ):
    """Batch 32, 64/8 and 128/8 heads, head_dim 128, fp16, 16k-32k tokens with
    spiky keys: the whole batch in the planner's launch configuration (one
    round of 16-row work-groups), five sequences checked against the oracle;
    at 64 heads also against the matrix-core decode kernel on every
    sequence."""
    spec = wl.LONG_BATCH.replace(name=f"long_batch_h{HQ}", num_q_heads=HQ)
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
    if HQ != 64:
        return
    other, oplan = run_lib(w, kernel="matrix")
    assert oplan.info.split_kernel == 1
    a, b = got.f32_twin.double(), other.f32_twin.double()
    per_seq = ((a - b).flatten(1).norm(dim=1) / b.flatten(1).norm(dim=1)).max().item()
    say(f"  against the decode kernel: worst per-sequence relative L2 {per_seq:.2e}")
    assert per_seq <= 1e-3


SMALL_GROUPS = [
    # B, H_q, H_kv, D, q/kv dtype, out, page, lengths, window, kernel with the planner's split, forced 3 splits
    (4, 8, 8, 128, "f16", "f16", 16, (3060, 1, 700, 0), 0, 2, 0),           # G 1, head_dim 128
    (2, 16, 8, 128, "bf16", "f32", 8, (5000, 17), 0, 2, 0),                 # G 2, 8-token pages
    (3, 16, 8, 128, "f16", "f32", 16, (2049, 300, 4096), 1000, 2, 1),       # G 2, window
    (2, 16, 8, 256, "bf16", "f32", 16, (9000, 300), 0, 2, 0),               # G 2, head_dim 256, 9000 tokens
    (1, 8, 8, 256, "f16", "f32", 32, (12000,), 0, 2, 0),                    # G 1, head_dim 256
    (2, 16, 8, 256, "f16", "f32", 16, (4000, 100), 0, 0, 0),                # G 2, head_dim 256, short: vector
    (2, 8, 8, 64, "bf16", "f32", 16, (20000, 5), 0, 0, 0),                  # G 1, head_dim 64: vector
]


@pytest.mark.parametrize("i", range(len(SMALL_GROUPS)))
def test_small_groups_few_streams_match_oracle(gpu, i):
    """One or two query heads per KV head in batches of fewer streams than
    compute units: the multi-token kernel at head_dim 128, and at head_dim
    256 from 8192 attended tokens, with the planner's split choice; the
    decode kernels otherwise and with a forced split count."""
    B, HQ, HKV, D, dt, out, P, lens, W, want_auto, want_forced = SMALL_GROUPS[i]
    spec = wl.WorkloadSpec(f"smallg{i}", B, HQ, HKV, D, dt, dt, out, P, ("list", lens), seed=7700 + i, window=W,
                           spike_frac=0.01)
    say(f"[small groups {i}] B={B} H={HQ}/{HKV} D={D} {dt}->{out} P={P} lens={lens} W={W}")
    w = wl.make_workload(spec, gpu)
    ref = oracle_for(w)
    for ns, want in ((0, want_auto), (3, want_forced)):
        got, plan = run_lib(w, num_splits=ns)
        assert plan.info.split_kernel == want
        err, worst = check(got, ref, dt, out, f"small groups {i} splits={ns}")
        say(f"  splits {ns}: kernel {plan.info.split_kernel}, rel L2 {err:.2e}, worst sequence {worst:.2e}")


def test_all_contexts_empty_wide_group(gpu):
    """Every context empty at 128/8 heads: one unsplit block per KV head that
    reads nothing, and every row of the output is zero."""
    spec = wl.WorkloadSpec("mqdec_all_empty", 3, 128, 8, 128, "bf16", "bf16", "f32", 16, ("list", (0, 0, 0)),
                           seed=7690)
    w = wl.make_workload(spec, gpu)
    got, plan = run_lib(w)
    assert plan.info.split_kernel == 2 and plan.max_splits == 1 and plan.workspace_bytes == 0
    assert torch.count_nonzero(got).item() == 0
