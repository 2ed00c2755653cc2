"""The balanced schedule of the matrix-core decode kernel (taken when the
split-length heuristic would need more than one round of resident
work-groups): batches large enough to select it, with empty, one-token,
page-boundary and long sequences, windows, every compiled group width, page
sizes 16-64 and both 16-bit types, against the oracle, and against the grid
schedule of the same kernel (forced split count) within fp32 rounding."""
import numpy as np
import pytest
import torch

from decode_attention_kv_04_amd import workloads as wl

from gpu_util import check, host64, oracle_for, run_lib, say

pytestmark = pytest.mark.gpu


def lengths(rng, B, P, long_frac, long_max):
    out = []
    for _ in range(B):
        u = rng.random()
        if u < 0.1:
            out.append(0)
        elif u < 0.2:
            out.append(int(rng.integers(1, 3)) * P + int(rng.integers(-1, 2)))
        elif u < 1 - long_frac:
            out.append(int(rng.integers(1, 700)))
        else:
            out.append(int(rng.integers(2000, long_max)))
    return out


CASES = [
    # B, G, P, kv/q dtype, out, window, long fraction, longest
    (96, 4, 16, "f16", "f16", 0, 0.5, 9000),
    (64, 4, 32, "bf16", "f32", 1000, 0.5, 20000),
    (200, 2, 16, "bf16", "bf16", 0, 0.3, 6000),
    (48, 8, 64, "f16", "f32", 0, 0.7, 12000),     # G 8 on the forced matrix-core kernel
    (128, 1, 16, "f16", "f16", 300, 0.6, 8000),    # G 1 on the forced matrix-core kernel
    (40, 3, 16, "f16", "f32", 0, 1.0, 16000),
    (700, 4, 16, "f16", "f16", 0, 0.05, 30000),
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_balanced_schedule_matches_oracle(gpu, i):
    B, G, P, dt, out, W, frac, lmax = CASES[i]
    rng = np.random.default_rng(7000 + i)
    lens = lengths(rng, B, P, frac, lmax)
    spec = wl.WorkloadSpec(f"bal{i}", B, 8 * G, 8, 128, dt, dt, out, P, ("list", tuple(lens)), seed=7100 + i,
                           window=W, spike_frac=0.01)
    say(f"[balanced {i}] B={B} G={G} P={P} {dt}->{out} W={W} keys={sum(lens)}")
    w = wl.make_workload(spec, gpu)
    # G 1 and G 5-8 reach the matrix-core decode kernel only when it is asked for
    kernel = "matrix" if G == 1 or G >= 5 else None
    got, plan = run_lib(w, kernel=kernel)
    assert plan.info.balanced == 1 and plan.info.split_kernel == 1
    say(f"  work-groups {plan.info.split_work_groups}, pages each {plan.pages_per_split}, "
        f"max pieces {plan.max_splits}")
    err, worst = check(got, oracle_for(w), dt, out, f"balanced {i}")
    say(f"  rel L2 {err:.2e}, worst sequence {worst:.2e}")
    # the grid schedule of the same kernel (forced split count): fp32 rounding apart
    grid, gplan = run_lib(w, kernel=kernel, num_splits=plan.max_splits + 1, twin=False)
    assert gplan.info.balanced == 0
    a = host64(got.f32_twin if hasattr(got, "f32_twin") else got)
    b = host64(grid)
    if out == "f32":
        assert np.linalg.norm(a - b) <= 2e-6 * np.linalg.norm(b)


def test_balanced_two_phase_and_repeat_bitwise(gpu):
    lens = [0, 1, 17, 5000, 900, 31, 8000, 2] * 12
    spec = wl.LLAMA8B_3060.replace(batch=len(lens), lengths=("list", tuple(lens)), seed=7200)
    w = wl.make_workload(spec, gpu)
    a, plan = run_lib(w)
    assert plan.info.balanced == 1 and plan.max_splits > 1
    b, _ = run_lib(w, two_phase=True)
    c, _ = run_lib(w)
    assert torch.equal(a, b) and torch.equal(a, c)
    for bb, L in enumerate(lens):
        if L == 0:
            assert torch.all(a[bb] == 0)
