"""K/V append on the GPU through the C-ABI: bit-exact against the append
oracle (pools compared as integer bit patterns, NaN payloads included), and
end to end with decode attention over the grown cache."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_kv_04_amd import binding
from decode_attention_kv_04_amd import workloads as wl

from gpu_util import check, oracle_for, run_lib, say

pytestmark = pytest.mark.gpu

INT_VIEW = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}


def bits(t):
    return t.contiguous().view(INT_VIEW[t.dtype]).cpu().numpy()


def grown_workload(spec, lens_before, T, gpu, max_pages=None):
    """A workload whose page table already maps room for T more keys per
    sequence (capped by max_pages); the current lengths are lens_before."""
    cap = (max_pages or 1 << 30) * spec.page_size
    spec = spec.replace(batch=len(lens_before))
    w = wl.make_workload(spec, gpu, lengths=[min(L + T, cap) for L in lens_before], max_pages_per_seq=max_pages)
    before = torch.tensor(lens_before, dtype=torch.int32)
    return w, before


def append_lib(w, lens_before, k_new, v_new, k_pool=None, v_pool=None):
    k_pool = w.k_pool.clone() if k_pool is None else k_pool
    v_pool = w.v_pool.clone() if v_pool is None else v_pool
    params = binding.params_for(w.q, k_pool, w.page_table, scale=w.scale)
    binding.decode_attn_append_kv(params, k_new, v_new, w.page_table, lens_before.to(k_pool.device), k_pool, v_pool)
    torch.cuda.synchronize()
    return k_pool, v_pool


def append_oracle_bits(w, lens_before, k_new, v_new):
    return oracle.append_kv(bits(w.k_pool), bits(w.v_pool), w.page_table.cpu().numpy(), lens_before.numpy(),
                            bits(k_new), bits(v_new), w.spec.page_size)


SHAPES = [
    # kv dtype, D, P, H_kv, T
    ("f32", 64, 16, 1, 1),
    ("f16", 128, 16, 8, 1),
    ("bf16", 128, 16, 8, 5),
    ("f16", 256, 8, 4, 37),
    ("bf16", 64, 32, 2, 40),
    ("f32", 256, 24, 3, 9),
    ("f16", 128, 64, 8, 130),
]


@pytest.mark.parametrize("kv,D,P,Hkv,T", SHAPES)
def test_append_is_bit_exact(gpu, kv, D, P, Hkv, T):
    spec = wl.WorkloadSpec(f"append_{kv}_{D}_{P}", 5, Hkv * 2, Hkv, D, kv, kv, kv, P, ("list", (0,) * 5), seed=21)
    lens = [0, 1, P - 1, P, 3 * P + 5]
    say(f"[append] kv={kv} D={D} P={P} Hkv={Hkv} T={T} lens={lens}")
    w, before = grown_workload(spec, lens, T, gpu)
    k_new, v_new = wl.make_new_rows(w.spec, T, gpu)
    kp, vp = append_lib(w, before, k_new, v_new)
    ek, ev = append_oracle_bits(w, before, k_new, v_new)
    np.testing.assert_array_equal(bits(kp), ek)
    np.testing.assert_array_equal(bits(vp), ev)


def test_rows_past_the_page_table_are_skipped(gpu):
    P = 16
    spec = wl.WorkloadSpec("append_cap", 3, 8, 2, 128, "f16", "f16", "f16", P, ("list", (0,) * 3), seed=22)
    lens = [4 * P - 2, 4 * P, 10]          # capacity 4 pages: 2, 0 and 5 of the 5 new rows fit
    w, before = grown_workload(spec, lens, 5, gpu, max_pages=4)
    k_new, v_new = wl.make_new_rows(w.spec, 5, gpu)
    kp, vp = append_lib(w, before, k_new, v_new)
    ek, ev = append_oracle_bits(w, before, k_new, v_new)
    np.testing.assert_array_equal(bits(kp), ek)
    np.testing.assert_array_equal(bits(vp), ev)


def test_zero_tokens_and_empty_batch_change_nothing(gpu):
    spec = wl.LLAMA8B_3060.replace(batch=2, lengths=("list", (100, 50)))
    w = wl.make_workload(spec, gpu)
    kp, vp = append_lib(w, w.seq_lens_host, w.k_pool.new_empty((2, 0, 8, 128)), w.v_pool.new_empty((2, 0, 8, 128)))
    assert np.array_equal(bits(kp), bits(w.k_pool)) and np.array_equal(bits(vp), bits(w.v_pool))


@pytest.mark.parametrize("kernel", ["auto", "vector"])
def test_decode_loop_over_a_growing_cache(gpu, kernel):
    """Four decode steps: append one token, attend over L + 1 keys; each
    step's output is checked against the oracle on the oracle-appended cache."""
    spec = wl.LLAMA8B_3060.replace(batch=3)
    lens = [3060, 17, 511]
    steps = 4
    w, lens_t = grown_workload(spec, lens, steps, gpu)
    host_k, host_v = w.k_pool.float().cpu().numpy(), w.v_pool.float().cpu().numpy()
    table = w.page_table.cpu().numpy()
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    for s in range(steps):
        k_new, v_new = wl.make_new_rows(w.spec, 1, gpu, salt=10 + s)
        say(f"[decode-loop] step {s} kernel={kernel}")
        append_lib(w, lens_t, k_new, v_new, k_pool=kp, v_pool=vp)
        host_k, host_v = oracle.append_kv(host_k, host_v, table, lens_t.numpy(), k_new.float().cpu().numpy(),
                                          v_new.float().cpu().numpy(), spec.page_size)
        lens_t = lens_t + 1
        out, _ = run_lib(w, k_pool=kp, v_pool=vp, seq_lens=lens_t.to(gpu), seq_lens_host=lens_t, kernel=kernel)
        ref = oracle.decode_attention(w.q.float().cpu().numpy(), host_k, host_v, table, lens_t.numpy(),
                                      spec.page_size, w.scale)
        check(out, ref, "f16", "f16", f"step {s}")


def test_full_size_append_changes_exactly_the_new_rows(gpu):
    """Batched long-context shape, one new token per sequence written at each
    sequence's end (the page table has room): the written rows equal the new
    rows and every other byte of the pools is unchanged."""
    spec = wl.LONG_BATCH
    lens = wl.draw_lengths(spec, torch.Generator().manual_seed(spec.seed))
    lens_before = [L - 1 for L in lens]                    # the last resident row is the append target
    say(f"[append-full] {spec.name} B={spec.batch}")
    w, before = grown_workload(spec, lens_before, 1, gpu, max_pages=spec.max_pages_per_seq)
    k_new, v_new = wl.make_new_rows(w.spec, 1, gpu)
    kp, vp = append_lib(w, before, k_new, v_new)
    P = spec.page_size
    pos = before.long().to(gpu)
    pages = w.page_table.long().gather(1, (pos // P)[:, None])[:, 0]
    slots = pos % P
    for got, orig, new in ((kp, w.k_pool, k_new), (vp, w.v_pool, v_new)):
        assert torch.equal(got[pages, :, slots].view(INT_VIEW[got.dtype]), new[:, 0].view(INT_VIEW[got.dtype]))
        got[pages, :, slots] = orig[pages, :, slots]
        assert torch.equal(got.view(INT_VIEW[got.dtype]), orig.view(INT_VIEW[orig.dtype]))


def test_append_then_attend_full_size(gpu):
    """Mixed-window shape after a one-token append: every sequence against
    the oracle on the appended cache."""
    spec = wl.MIXED_WINDOW
    lens = wl.draw_lengths(spec, torch.Generator().manual_seed(spec.seed))
    w, before = grown_workload(spec, lens, 1, gpu)
    k_new, v_new = wl.make_new_rows(w.spec, 1, gpu)
    kp, vp = append_lib(w, before, k_new, v_new)
    after = before + 1
    out, _ = run_lib(w, k_pool=kp, v_pool=vp, seq_lens=after.to(gpu), seq_lens_host=after)
    w2 = wl.Workload(spec=w.spec, q=w.q, k_pool=kp, v_pool=vp, page_table=w.page_table, seq_lens=after.to(gpu),
                     seq_lens_host=after, scale=w.scale, window=w.window, num_pages=w.num_pages,
                     poison_page=w.poison_page)
    ref = oracle_for(w2, attended_only=True)
    check(out, ref, spec.kv_dtype, spec.out_dtype, "mixed_window+append")
