"""GPU invariants: properties the HIP path must satisfy exactly (bitwise) or
within tolerance, independent of the oracle."""
import numpy as np
import pytest
import torch

from decode_attention_kv_04_amd import workloads as wl

from gpu_util import check, host64, oracle_for, run_lib, say

pytestmark = pytest.mark.gpu


def make(spec, gpu, **kw):
    say(f"[workload] {spec.name} {kw or ''}")
    return wl.make_workload(spec.replace(**kw) if kw else spec, gpu)


KERNELS = ["auto", "vector"]


@pytest.mark.parametrize("kernel", KERNELS)
def test_run_to_run_bitwise_determinism(gpu, kernel):
    w = make(wl.LLAMA8B_3060, gpu)
    a, _ = run_lib(w, kernel=kernel)
    for _ in range(3):
        b, _ = run_lib(w, kernel=kernel)
        assert torch.equal(a, b)


@pytest.mark.parametrize("kernel", KERNELS)
def test_page_permutation_is_bitwise(gpu, kernel):
    w = make(wl.WIDE_GQA.replace(head_dim=128), gpu)
    a, _ = run_lib(w, num_splits=3, kernel=kernel)
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(w.num_pages, generator=g).to(gpu)  # page p moves to perm[p]
    kp = torch.empty_like(w.k_pool)
    vp = torch.empty_like(w.v_pool)
    kp[perm] = w.k_pool
    vp[perm] = w.v_pool
    table = perm.to(torch.int32)[w.page_table.long()]
    b, _ = run_lib(w, num_splits=3, k_pool=kp, v_pool=vp, page_table=table.contiguous(), kernel=kernel)
    assert torch.equal(a, b)


@pytest.mark.parametrize("kernel", KERNELS)
def test_unattended_contents_do_not_matter(gpu, kernel):
    spec = wl.MIXED_WINDOW.replace(batch=4, lengths=("list", (100, 5000, 33, 4097)), window=1000, page_size=32)
    w = make(spec, gpu)
    a, _ = run_lib(w, kernel=kernel)
    kp = torch.where(torch.isnan(w.k_pool), torch.full_like(w.k_pool, 1000.0), w.k_pool)
    vp = torch.where(torch.isnan(w.v_pool), torch.full_like(w.v_pool, -7.0), w.v_pool)
    b, _ = run_lib(w, k_pool=kp, v_pool=vp, kernel=kernel)
    assert torch.isfinite(a).all()
    assert torch.equal(a, b)


@pytest.mark.parametrize("kernel", KERNELS)
def test_single_key_returns_value_bitwise(gpu, kernel):
    for kv in ("f32", "f16", "bf16"):
        spec = wl.WorkloadSpec(f"one_{kv}", 3, 8, 2, 128, kv, kv, kv, 16, ("list", (1, 1, 1)), seed=3)
        w = make(spec, gpu)
        out, _ = run_lib(w, kernel=kernel)
        v = w.v_pool[w.page_table[:, 0].long(), :, 0, :]            # [B][Hkv][D]
        expect = v.repeat_interleave(4, dim=1)
        assert torch.equal(out, expect)
    # window 1 keeps only the newest key
    spec = wl.WorkloadSpec("w1", 2, 4, 1, 64, "f32", "f32", "f32", 16, ("list", (37, 16)), seed=4, window=1)
    w = make(spec, gpu)
    out, _ = run_lib(w)
    for b, L in enumerate((37, 16)):
        t = L - 1
        v = w.v_pool[w.page_table[b, t // 16].long(), 0, t % 16]
        assert torch.equal(out[b], v.expand(4, -1))


@pytest.mark.parametrize("kernel", KERNELS)
def test_doubling_values_doubles_output_bitwise(gpu, kernel):
    w = make(wl.WIDE_GQA.replace(head_dim=128), gpu)
    a, _ = run_lib(w, out_dtype="f32", kernel=kernel)
    b, _ = run_lib(w, out_dtype="f32", v_pool=w.v_pool * 2, kernel=kernel)
    assert torch.equal(b, 2 * a)


@pytest.mark.parametrize("kernel", KERNELS)
def test_window_at_least_length_is_bitwise_no_window(gpu, kernel):
    spec = wl.LLAMA8B_3060.replace(batch=2, lengths=("list", (3060, 700)))
    w = make(spec, gpu)
    a, _ = run_lib(w, window=0, num_splits=4, kernel=kernel)
    b, _ = run_lib(w, window=3060, num_splits=4, kernel=kernel)
    assert torch.equal(a, b)


def test_window_equals_truncation(gpu):
    """A window over the last W keys equals a no-window run over those W keys
    re-paged into a fresh pool (different page alignment)."""
    W, P = 1000, 16
    spec = wl.LLAMA8B_3060.replace(batch=2, lengths=("list", (3060, 1501)), window=W)
    w = make(spec, gpu)
    a, _ = run_lib(w)
    host = wl.to_numpy_inputs(w)
    for b, L in enumerate((3060, 1501)):
        keep = np.arange(L - W, L)
        pages = host["page_table"][b, keep // P]
        K = torch.from_numpy(host["k_pool"][pages, :, keep % P]).to(torch.float16)   # [W][Hkv][D]
        V = torch.from_numpy(host["v_pool"][pages, :, keep % P]).to(torch.float16)
        npg = (W + P - 1) // P
        kp = torch.full((npg, 8, P, 128), float("nan"), dtype=torch.float16)
        vp = torch.full_like(kp, float("nan"))
        idx = torch.arange(W)
        kp[idx // P, :, idx % P] = K
        vp[idx // P, :, idx % P] = V
        table = torch.arange(npg, dtype=torch.int32)[None, :].to(gpu)
        lens = torch.tensor([W], dtype=torch.int32)
        out, _ = run_lib(w, q=w.q[b:b + 1].contiguous(), k_pool=kp.to(gpu), v_pool=vp.to(gpu), page_table=table,
                         window=0, seq_lens=lens.to(gpu), seq_lens_host=lens)
        rel = (out.float() - a[b:b + 1].float()).norm() / a[b:b + 1].float().norm()
        assert rel.item() < 1e-3


def test_gqa_equals_mha_with_repeated_kv(gpu):
    spec = wl.WorkloadSpec("gqa", 2, 8, 2, 128, "f32", "f32", "f32", 16, ("list", (500, 3000)), seed=11)
    w = make(spec, gpu)
    a, _ = run_lib(w)
    kp = w.k_pool.repeat_interleave(4, dim=1).contiguous()
    vp = w.v_pool.repeat_interleave(4, dim=1).contiguous()
    b, _ = run_lib(w, k_pool=kp, v_pool=vp)
    rel = ((a - b).norm() / a.norm()).item()
    assert rel < 1e-6


def test_split_count_changes_within_tolerance(gpu):
    spec = wl.WorkloadSpec("splits", 2, 8, 2, 128, "f32", "f32", "f32", 16, ("list", (5000, 3333)), seed=12)
    w = make(spec, gpu)
    ref = oracle_for(w)
    outs = []
    for ns in (1, 2, 3, 7, 10_000):
        out, _ = run_lib(w, num_splits=ns)
        check(out, ref, "f32", "f32", f"splits={ns}")
        outs.append(host64(out))
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 1e-5


@pytest.mark.parametrize("kernel", KERNELS)
def test_batch_independence_bitwise(gpu, kernel):
    spec = wl.LLAMA8B_3060.replace(batch=3, lengths=("list", (3000, 3000, 3000)))
    w = make(spec, gpu)
    a, _ = run_lib(w, num_splits=1, kernel=kernel)
    for b in range(3):
        lens = w.seq_lens_host[b:b + 1].clone()
        out, _ = run_lib(w, num_splits=1, q=w.q[b:b + 1].contiguous(), page_table=w.page_table[b:b + 1].contiguous(),
                         seq_lens=lens.to(gpu), seq_lens_host=lens, kernel=kernel)
        assert torch.equal(out[0], a[b])
