"""Whole streams: a batch with at least one (sequence, KV head) stream per
compute unit and about equal attended lengths runs unsplit (one work-group per
stream, no combine, no workspace). Such batches on both decode kernels and on
the multi-token kernel (head_dim 128, 8 and 16 query heads per KV head, and
4 tokens x 4 heads in one 16-row block), with
windows, ragged lengths within the equal-length band and several new tokens
per sequence, against the oracle, and against a forced split count of the same
kernel within fp32 rounding."""
import numpy as np
import pytest

from decode_attention_kv_04_amd import workloads as wl

from gpu_util import check, host64, oracle_for, run_lib, say

pytestmark = pytest.mark.gpu

CASES = [
    # B, H_q, H_kv, D, q/kv dtype, out, page, lengths, window, query_len
    (32, 32, 8, 128, "f16", "f16", 16, ("fixed", 2048), 0, 1),
    (32, 32, 8, 128, "bf16", "f32", 32, ("uniform", 1900, 2050), 1000, 1),
    (64, 8, 4, 256, "f16", "f32", 16, ("fixed", 777), 0, 1),         # G 2, head_dim 256: vector kernel
    (32, 8, 8, 128, "f16", "f16", 16, ("fixed", 1500), 0, 1),        # one head per group: vector kernel
    (32, 32, 8, 128, "f32", "f32", 16, ("fixed", 1024), 0, 1),       # fp32 K/V: vector kernel
    (256, 32, 8, 128, "f16", "f16", 16, ("uniform", 300, 320), 0, 1),
    (32, 32, 8, 128, "f32", "f32", 16, ("fixed", 600), 200, 3),      # three new tokens, once per token
    (32, 64, 8, 128, "f16", "f32", 16, ("fixed", 2048), 0, 1),       # G 8: the multi-token kernel, unsplit
    (32, 128, 8, 128, "bf16", "f32", 24, ("uniform", 1900, 2050), 500, 1),  # G 16, 24-token pages, window
    (32, 32, 8, 128, "f16", "f32", 16, ("fixed", 2048), 0, 4),       # a 4-token check: one 16-row block
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_whole_streams_match_oracle(gpu, i):
    B, HQ, HKV, D, dt, out, P, lens, W, T = CASES[i]
    spec = wl.WorkloadSpec(f"whole{i}", B, HQ, HKV, D, dt, dt, out, P, lens, seed=7400 + i, window=W,
                           spike_frac=0.01, query_len=T)
    say(f"[whole streams {i}] B={B} H={HQ}/{HKV} D={D} {dt}->{out} P={P} lens={lens} W={W} T={T}")
    w = wl.make_workload(spec, gpu)
    got, plan = run_lib(w)
    assert plan.max_splits == 1 and plan.workspace_bytes == 0 and plan.info.balanced == 0
    say(f"  split kernel {plan.info.split_kernel}, work-groups {plan.info.split_work_groups}")
    err, worst = check(got, oracle_for(w), dt, out, f"whole streams {i}")
    say(f"  rel L2 {err:.2e}, worst sequence {worst:.2e}")
    split, splan = run_lib(w, num_splits=3, twin=False)
    assert splan.max_splits > 1
    a = host64(got.f32_twin if hasattr(got, "f32_twin") else got)
    b = host64(split)
    if out == "f32":
        # The decode kernels keep P in fp32: the split changes only the fp32
        # summation order. The multi-token kernel rounds P to f16 (or a bf16
        # pair) relative to each split's running maximum, so a split changes
        # that rounding: bounded by the f16 unit roundoff 2^-11.
        tol = 2.0 ** -11 if plan.info.split_kernel == 2 else 2e-6
        assert np.linalg.norm(a - b) <= tol * np.linalg.norm(b)
