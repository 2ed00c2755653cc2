"""Helpers shared by the GPU tests: run the library on a workload and compare
with the oracle."""
import contextlib
import os
import sys

import numpy as np
import torch

import oracle
from decode_attention_kv_04_amd import binding, workloads

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
KV_TOL = {"f32": 1e-5, "f16": 1e-3, "bf16": 1e-3}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@contextlib.contextmanager
def split_kernel(kind):
    """kind: None / "auto" (the planner chooses) or "vector" / "matrix"."""
    old = os.environ.get("DECODE_ATTN_KERNEL")
    if kind and kind != "auto":
        os.environ["DECODE_ATTN_KERNEL"] = kind
    else:
        os.environ.pop("DECODE_ATTN_KERNEL", None)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("DECODE_ATTN_KERNEL", None)
        else:
            os.environ["DECODE_ATTN_KERNEL"] = old


@contextlib.contextmanager
def mq_rows(rows):
    """Rows per block of the head_dim-128 multi-token kernel ("64" / "128"; None = default)."""
    old = os.environ.get("DECODE_ATTN_MQ_ROWS")
    if rows:
        os.environ["DECODE_ATTN_MQ_ROWS"] = str(rows)
    else:
        os.environ.pop("DECODE_ATTN_MQ_ROWS", None)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("DECODE_ATTN_MQ_ROWS", None)
        else:
            os.environ["DECODE_ATTN_MQ_ROWS"] = old


def run_lib(w, *, num_splits=0, out_dtype=None, q=None, k_pool=None, v_pool=None, page_table=None,
            window=None, seq_lens=None, seq_lens_host=None, two_phase=False, kernel=None, fixed_chunk=0):
    """One decode_attn_run (or split + combine) on the workload's tensors;
    returns (out tensor, plan). The output starts as NaN so unwritten rows show.
    `kernel` = "vector" forces the vector split kernel; default: automatic.
    `fixed_chunk` > 0 selects the fixed-order mode with chunks of that many tokens."""
    q = w.q if q is None else q
    k_pool = w.k_pool if k_pool is None else k_pool
    v_pool = w.v_pool if v_pool is None else v_pool
    page_table = w.page_table if page_table is None else page_table
    seq_lens = w.seq_lens if seq_lens is None else seq_lens
    seq_lens_host = w.seq_lens_host if seq_lens_host is None else seq_lens_host
    window = w.window if window is None else window
    out_dtype = out_dtype or w.spec.out_dtype
    params = binding.params_for(q, k_pool, page_table, window=window, scale=w.scale, out_dtype=out_dtype,
                                num_splits=num_splits, fixed_chunk=fixed_chunk)
    with split_kernel(kernel):
        plan = binding.decode_attn_plan(params, seq_lens_host, device=q.device.index)
    out = torch.full(q.shape, float("nan"), dtype=TORCH_DT[out_dtype], device=q.device)
    ws = binding.alloc_workspace(plan, q.device)
    if ws is not None:
        ws.fill_(0xFF)  # NaN bit patterns: stale state would show
    if two_phase:
        binding.decode_attn_split(plan, q, k_pool, v_pool, page_table, seq_lens, out, ws)
        binding.decode_attn_combine(plan, seq_lens, out, ws)
    else:
        binding.decode_attn_run(plan, q, k_pool, v_pool, page_table, seq_lens, out, ws)
    torch.cuda.synchronize()
    return out, plan


def host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_for(w, rows=None):
    a = workloads.to_numpy_inputs(w, rows)
    fn = oracle.prefill_attention if a["q"].ndim == 4 else oracle.decode_attention
    return fn(a["q"], a["k_pool"], a["v_pool"], a["page_table"], a["seq_lens"], a["page_size"], a["scale"],
              a["window"])


BF16_ROUNDING = 2.0 ** -8  # largest relative error of rounding to bf16 (half a step at 8 significant bits)


def check(got, ref, kv_dtype, out_dtype, label=""):
    """Relative L2 over the whole output and per sequence, within the bound
    for the KV dtype (1e-5 fp32, 1e-3 fp16/bf16, fp32 accumulation).

    A bf16 output cannot meet that bar (its own rounding is ~1.6e-3 relative
    L2), and against the bf16-rounded oracle any tiny difference next to a
    rounding boundary becomes a whole bf16 step (near-zero elements included).
    It is held to the bound that follows from the arithmetic: the rounding
    adds at most 2^-8 of each element, so the relative L2 against the exact
    oracle is at most the KV bound plus 2^-8. (The same computation at fp32
    output, in the same suites, is held to the KV bound itself.)"""
    got = host64(got) if isinstance(got, torch.Tensor) else got
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    tol = KV_TOL[kv_dtype]
    if out_dtype == "f16" and kv_dtype == "f32":
        tol = 1e-3  # fp16 output rounding alone is ~2e-4
    if out_dtype == "bf16":
        tol = tol + BF16_ROUNDING
    err = oracle.relative_l2(got, ref)
    rows = oracle.relative_l2_per_row(got, ref)
    worst = max(rows) if rows else 0.0
    assert err <= tol, f"{label}: relative L2 {err:.3e} > {tol:g}"
    assert worst <= tol, f"{label}: worst per-sequence relative L2 {worst:.3e} > {tol:g}"
    return err, worst
