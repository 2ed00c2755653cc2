"""Decode-attention benchmark on one MI355X.

A step is one decode_attn_run (split pass + combine pass) over one batch of
the batched long-context workload: batch 32, 32 query / 8 KV heads (GQA 4),
head_dim 128, fp16 q/K/V, per-sequence context uniform in [16384, 32768],
1 % of keys x8, 16-token pages in a shuffled pool. Inputs are resident in HBM
before timing starts. Prints one JSON line.

value   = algorithmic KV bytes per step / step time (GB/s), where the
          algorithmic bytes are every attended K and V row read once per KV
          head: sum_b L_b * H_kv * D * 2 bytes * 2.
roofline: the split kernel alone, timed with HIP events on the stream it is
          launched on, against the 8 TB/s HBM peak.
cpu_baseline: the f64 CPU oracle on a bounded sample of the same batch.
configs: the five named configurations (tiny, the Llama-3.1-8B shape at 3060
          tokens, wide-head GQA, this batch, the mixed sliding-window batch):
          step and split-pass µs as median / p10 / p90 over alternating
          repeats, GB/s, fractions of the peak and of the measured gather
          ceiling, cold-cache µs where the inputs fit the last-level cache,
          the oracle's wall time on each, and each output checked against
          the oracle (the run exits 1 if any check fails).
--sweep: only a context-length sweep on the Llama shape (L 256..65536,
          batch 1 and 32), the same shape at 3060 tokens with head_dim
          64, 128 and 256, and with 1, 2, 4, 8 and 16 query heads per KV
          head (batch 1 x 3060 and 32 x 4096 tokens).
Also reported, each timed the same way: the fixed-order mode on the same
batch (fixed_order), several new tokens per sequence on their own workloads
(multi_token: a 4-token check over the long-context batch and a 128-token
suffix prefill, each against its HBM or matrix-core roofline), one whole
decode step (32 layers, 32 KV pools) of the Llama-3.1-8B shape at 3060 tokens
issued eagerly and as a replayed HIP graph (layer_step), and the K/V append
of 1 and 256 tokens per sequence (append_kv).
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention µs/step + achieved HBM GB/s (% of peak), Llama-8B shape"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "split_kernel_long_batch_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "decode_attention_kv_04_amd", "csrc", f)
                  for f in ("decode_split.hip", "decode_split_mfma.hip", "device_common.h", "kernels.h")]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per split-kernel launch from the committed counter summary,
    or None if there is none or the kernel source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash():
        return None
    return float(m_bytes.group(1))


def time_on_stream(fn, iters, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters  # ms


CALIBRATION_BYTES = 1 << 30


def _probe():
    lib = ctypes.CDLL(os.path.join(ROOT, "decode_attention_kv_04_amd", "libda_probe.so"))
    vp = ctypes.c_void_p
    lib.da_probe_read_stream.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_int, vp]
    lib.da_probe_read_blocks.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp, vp]
    lib.da_probe_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
    return lib


def measure_ceilings(dev, sptr, stream):
    """HBM read ceilings measured on this GPU over a 4 GiB buffer:
    'stream' = each work-group reads one contiguous chunk (nontemporal
    16-byte loads); 'gather4k' = 4 KiB blocks in a random order, the access
    pattern of a shuffled page pool."""
    import torch
    probe = _probe()
    nbytes = 4 << 30
    nblk = nbytes // 4096
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    perm = torch.randperm(nblk, generator=g, device=dev).to(torch.int32)
    per_wg = 128
    sink = torch.empty(max(1024, -(-nblk // per_wg)) * 256, dtype=torch.int32, device=dev)
    runs = {
        "stream": lambda: probe.da_probe_read_stream(buf.data_ptr(), nbytes, sink.data_ptr(), 1024, sptr),
        "gather4k": lambda: probe.da_probe_read_blocks(buf.data_ptr(), perm.data_ptr(), nblk, per_wg,
                                                       sink.data_ptr(), sptr),
    }
    out = {}
    for name, fn in runs.items():
        for _ in range(2):
            fn()
        ms = time_on_stream(fn, 5, stream)
        out[name] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del buf, sink, perm
    return out


def calibration_copy(dev, sptr):
    import torch
    probe = _probe()
    src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    probe.da_probe_copy(dst.data_ptr(), src.data_ptr(), CALIBRATION_BYTES, sptr)
    torch.cuda.synchronize()


def cpu_baseline(w, budget_s=12.0, max_passes=8):
    """Time the oracle on whole sequences of the batch, cycling over the batch,
    until ~budget_s of CPU work (at most max_passes passes); GB/s of
    algorithmic KV bytes processed."""
    import numpy as np

    import oracle
    from decode_attention_kv_04_amd import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    spec = w.spec
    elt = workloads.ELT_BYTES[spec.kv_dtype]
    done_bytes = 0
    spent = 0.0
    rows = []
    for i in range(spec.batch * max_passes):
        b = i % spec.batch
        a = workloads.to_numpy_inputs(w, [b])
        t = time.perf_counter()
        fn = oracle.prefill_attention if a["q"].ndim == 4 else oracle.decode_attention
        fn(a["q"], a["k_pool"], a["v_pool"], a["page_table"], a["seq_lens"], a["page_size"], a["scale"], a["window"])
        spent += time.perf_counter() - t
        t0, t1 = w.attended()[b]
        done_bytes += (t1 - t0) * spec.num_kv_heads * spec.head_dim * elt * 2
        rows.append(b)
        if spent >= budget_s:
            break
    return {
        "value": round(done_bytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(rows)} sequence runs over the {spec.batch} sequences of the batch, in order "
                  f"(all {spec.num_q_heads} query heads, "
                  f"{sum(e - s for s, e in (w.attended()[b] for b in rows))} keys), f64 numpy, "
                  f"{spent:.1f} s; host has {os.cpu_count()} logical CPUs",
        "seconds": round(spent, 2),
    }


FIXED_CHUNK = 1024


def measure_fixed_order(w, binding, lib, dev, stream, iters):
    """Time decode_attn_run in the fixed-order mode (planner-chosen chunks per
    work-group) on the workload; {chunk_tokens, us, GB_s, chunks_per_work_group}."""
    import torch
    spec = w.spec
    params = binding.params_for(w.q, w.k_pool, w.page_table, window=w.window, scale=w.scale,
                                out_dtype=spec.out_dtype, fixed_chunk=FIXED_CHUNK)
    plan = binding.decode_attn_plan(params, w.seq_lens_host, device=dev.index or 0)
    out = torch.empty(w.q.shape, dtype={"f32": torch.float32, "f16": torch.float16,
                                        "bf16": torch.bfloat16}[spec.out_dtype], device=dev)
    ws = binding.alloc_workspace(plan, dev)
    ptrs = [w.q.data_ptr(), w.k_pool.data_ptr(), w.v_pool.data_ptr(), w.page_table.data_ptr(),
            w.seq_lens.data_ptr(), out.data_ptr(), ws.data_ptr(), plan.workspace_bytes, stream.cuda_stream]

    def run():
        st = lib.decode_attn_run(plan.handle, *ptrs)
        if st != 0:
            raise binding.DecodeAttnError(st, "decode_attn_run (fixed order)")

    for _ in range(3):
        run()
    ms = time_on_stream(run, iters, stream)
    return {"chunk_tokens": FIXED_CHUNK, "us": round(ms * 1e3, 2),
            "GB_s": round(w.kv_bytes() / (ms * 1e-3) / 1e9, 1),
            "chunks_per_work_group": plan.info.chunks_per_work_group,
            "work_groups": plan.info.split_work_groups}


MFMA_PEAK_TFLOPS_16BIT = 2500.0  # dense f16/bf16 matrix-core peak
MULTI_TOKEN_WORKLOADS = ("verify_long", "suffix_prefill")


def attention_flops(w):
    """2 FLOPs per multiply-add of q.k and of p.v: 4*D per (query head, key)."""
    T = w.spec.query_len
    keys = 0
    for L in w.seq_lens_host.tolist():
        for t in range(T):
            p = L - T + t
            keys += min(p + 1, w.window) if w.window > 0 else p + 1
    return keys * w.spec.num_q_heads * w.spec.head_dim * 4


def measure_multi_token(binding, workloads, lib, dev, stream, rounds):
    """Several new tokens per sequence: time decode_attn_run and the split
    pass alone on each multi-token workload, and place them against their
    roofline (HBM when the FLOPs per algorithmic byte are below the 16-bit
    matrix-core ridge, matrix cores otherwise). The workloads are timed like
    the named configurations: after ~30 ms of warm-up launches (the clocks
    rise over the first blocks of a compute-bound kernel: 109 -> 93 us per
    step over six 50-launch blocks of the 128-token suffix), in `rounds`
    alternating rounds of ~2 ms blocks; the median is reported with p10 and
    p90."""
    import torch
    ridge = MFMA_PEAK_TFLOPS_16BIT * 1e12 / (HBM_PEAK_GBPS * 1e9)
    runners = {}
    for name in MULTI_TOKEN_WORKLOADS:
        w = workloads.make_workload(workloads.NAMED[name], dev)
        runners[name] = Runner(binding, lib, w, dev, stream)
    for r in runners.values():
        n = int(max(10, 30000.0 // max(1.0, block_us(r.run, 5, stream))))
        block_us(r.run, n, stream)
    t = time_alternating(runners, rounds, stream)
    res = []
    for name, r in runners.items():
        w, spec = r.w, r.w.spec
        step, split = quantiles(t[name]["run"]), quantiles(t[name]["split"])
        by, fl = w.kv_bytes(), attention_flops(w)
        hbm = fl / by < ridge

        def frac(t_us):
            return round(by / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBPS if hbm
                         else fl / (t_us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS_16BIT, 4)

        us, us_split = step["median"], split["median"]
        # "frac" places the dominant kernel (the split pass) against its
        # roofline, as the headline does; "step_frac" the whole step (with
        # the combine).
        res.append({"workload": spec.name, "query_len": spec.query_len, "us": us, "us_quantiles": step,
                    "split_us": us_split, "split_us_quantiles": split,
                    "GB_s": round(by / (us * 1e-6) / 1e9, 1), "TFLOP_s": round(fl / (us * 1e-6) / 1e12, 1),
                    "split_TFLOP_s": round(fl / (us_split * 1e-6) / 1e12, 1), "bound": "hbm" if hbm else "mfma",
                    "frac": frac(us_split), "step_frac": frac(us),
                    "algorithmic_bytes": by, "flops": fl, "work_groups": r.plan.info.split_work_groups})
        print(f"[bench] {name}: {us:.1f} us (split pass {us_split:.1f} us)", file=sys.stderr, flush=True)
    del runners
    torch.cuda.empty_cache()
    return res


COLD_BYTES = 1 << 30
LLC_BYTES = 256 << 20  # MI355X last-level (Infinity) cache


def measure_cold(w, plan, lib, out, ws, stream, cycles=3):
    """The step over inputs the last-level cache cannot hold: k copies of the
    K/V pool side by side (k * KV bytes >= 1 GiB), copy c addressed through
    the page table offset by c * num_pages, the steps cycling through the
    copies in order so every step reads pages that ~1 GiB of other steps
    has touched since. {sets, us, GB_s} per step (mean over whole cycles)."""
    import torch
    kvb = w.kv_bytes()
    k = max(2, -(-COLD_BYTES // max(1, kvb)))
    n = w.num_pages
    kp = w.k_pool.repeat(k, 1, 1, 1)
    vp = w.v_pool.repeat(k, 1, 1, 1)
    tables = torch.stack([w.page_table + c * n for c in range(k)]).contiguous()
    row = tables[0].numel() * tables.element_size()
    sptr = stream.cuda_stream
    base = [w.q.data_ptr(), kp.data_ptr(), vp.data_ptr()]
    tail = [w.seq_lens.data_ptr(), out.data_ptr(), ws.data_ptr() if ws is not None else None, plan.workspace_bytes,
            sptr]
    args = [base + [tables.data_ptr() + c * row] + tail for c in range(k)]

    def cycle():
        for a in args:
            st = lib.decode_attn_run(plan.handle, *a)
            if st != 0:
                raise RuntimeError(f"decode_attn_run (cold): status {st}")

    cycle()
    ms = time_on_stream(cycle, cycles, stream) / k
    del kp, vp, tables
    torch.cuda.empty_cache()
    return {"sets": k, "us": round(ms * 1e3, 2), "GB_s": round(kvb / (ms * 1e-3) / 1e9, 1)}


LAYERS = 32


def measure_layer_step(binding, workloads, dev, stream, iters, layers=LAYERS):
    """Attention of one whole decode step of the Llama-3.1-8B shape at 3060
    tokens: `layers` independent KV pools (one per layer, 401 MB for 32, more
    than the last-level cache holds), one decode_attn_run each, back to back,
    issued eagerly and replayed from a captured HIP graph (the replay must
    equal the eager outputs bitwise). {layers, eager_us, graph_us, GB_s}."""
    import torch
    spec = workloads.LLAMA8B_3060
    ws_ = [workloads.make_workload(spec.replace(seed=spec.seed * 1000 + i), dev) for i in range(layers)]
    params = binding.params_for(ws_[0].q, ws_[0].k_pool, ws_[0].page_table, window=ws_[0].window,
                                scale=ws_[0].scale, out_dtype=spec.out_dtype)
    plan = binding.decode_attn_plan(params, ws_[0].seq_lens_host, device=dev.index or 0)
    scratch = binding.alloc_workspace(plan, dev)
    outs = [torch.empty(w.q.shape, dtype=workloads.DTYPES[spec.out_dtype], device=dev) for w in ws_]

    def step(s=None):
        for w, o in zip(ws_, outs):
            binding.decode_attn_run(plan, w.q, w.k_pool, w.v_pool, w.page_table, w.seq_lens, o, scratch, stream=s)

    for _ in range(3):
        step()
    eager_ms = time_on_stream(step, iters, stream)
    eager_out = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(side)
    torch.cuda.synchronize()
    for o in outs:
        o.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    if not all(torch.equal(a, b) for a, b in zip(outs, eager_out)):
        raise RuntimeError("graph replay of the layer step differs from the eager step")
    graph_ms = time_on_stream(graph.replay, iters, stream)
    total = sum(w.kv_bytes() for w in ws_)
    del graph, ws_, outs, eager_out, scratch
    torch.cuda.empty_cache()
    return {"workload": f"{spec.name} x {layers} layers", "layers": layers, "eager_us": round(eager_ms * 1e3, 1),
            "graph_us": round(graph_ms * 1e3, 1), "GB_s": round(total / (graph_ms * 1e-3) / 1e9, 1),
            "bytes": total}


def measure_append(w, lib, params, stream, tokens, iters):
    """Time decode_attn_append_kv writing `tokens` rows per sequence at the
    end of each sequence's context (positions L-T .. L-1), with new rows equal
    to the rows already there, so the pools keep their contents. Returns
    {tokens, us, GB_s} where the bytes are the rows read plus the rows written."""
    import ctypes as C

    import torch
    P = w.spec.page_size
    dev = w.q.device
    L = w.seq_lens.long()
    pos = L[:, None] - tokens + torch.arange(tokens, device=dev)[None, :]          # [B][T]
    valid = pos >= 0
    posc = pos.clamp(min=0)
    pages = w.page_table.long().gather(1, posc // P)
    slots = posc % P
    k_new = w.k_pool[pages, :, slots].contiguous()                                  # [B][T][H_kv][D]
    v_new = w.v_pool[pages, :, slots].contiguous()
    before = (L - tokens).to(torch.int32).contiguous()
    rows = int(valid.sum().item())
    row_bytes = w.spec.num_kv_heads * w.spec.head_dim * w.k_pool.element_size()
    sptr = stream.cuda_stream
    args = (C.byref(params), tokens, k_new.data_ptr(), v_new.data_ptr(), w.page_table.data_ptr(),
            before.data_ptr(), w.k_pool.data_ptr(), w.v_pool.data_ptr(), sptr)

    def append():
        st = lib.decode_attn_append_kv(*args)
        if st != 0:
            raise RuntimeError(f"decode_attn_append_kv: status {st}")

    append()
    ms = time_on_stream(append, iters, stream)
    moved = rows * row_bytes * 2 * 2
    return {"tokens": tokens, "us": round(ms * 1e3, 2), "GB_s": round(moved / (ms * 1e-3) / 1e9, 1),
            "bytes": moved}


# ---------------------------------------------------------------------------
# The five named configurations, each timed over alternating repeats, and the
# oracle's wall time on each (the CPU-baseline leg).
# ---------------------------------------------------------------------------

CONFIGS = (("C1", "tiny"), ("C2", "llama8b_3060"), ("C3", "wide_gqa"), ("C4", "long_batch"),
           ("C5", "mixed_window"))
BLOCK_US = 2000.0   # each timed block holds about this much GPU time
KV_TOL = {"f32": 1e-5, "f16": 1e-3, "bf16": 1e-3}


class Runner:
    """One planned decode_attn_run on a workload's resident inputs."""

    def __init__(self, binding, lib, w, dev, stream, **plan_kw):
        import torch
        self.w = w
        spec = w.spec
        params = binding.params_for(w.q, w.k_pool, w.page_table, window=w.window, scale=w.scale,
                                    out_dtype=spec.out_dtype, **plan_kw)
        self.plan = binding.decode_attn_plan(params, w.seq_lens_host, device=dev.index or 0)
        from decode_attention_kv_04_amd import workloads
        self.out = torch.empty(w.q.shape, dtype=workloads.DTYPES[spec.out_dtype], device=dev)
        self.ws = binding.alloc_workspace(self.plan, dev)
        self.ptrs = [w.q.data_ptr(), w.k_pool.data_ptr(), w.v_pool.data_ptr(), w.page_table.data_ptr(),
                     w.seq_lens.data_ptr(), self.out.data_ptr(), self.ws.data_ptr() if self.ws is not None else None,
                     self.plan.workspace_bytes, stream.cuda_stream]
        self.lib, self.binding, self.stream = lib, binding, stream

    def run(self):
        st = self.lib.decode_attn_run(self.plan.handle, *self.ptrs)
        if st != 0:
            raise self.binding.DecodeAttnError(st, f"decode_attn_run ({self.w.spec.name})")

    def split(self):
        st = self.lib.decode_attn_split(self.plan.handle, *self.ptrs)
        if st != 0:
            raise self.binding.DecodeAttnError(st, f"decode_attn_split ({self.w.spec.name})")


def block_us(fn, n, stream):
    """Mean µs per launch over one block of n back-to-back launches."""
    return time_on_stream(fn, n, stream) * 1e3


def quantiles(xs):
    xs = sorted(xs)

    def q(f):
        i = f * (len(xs) - 1)
        lo = int(i)
        hi = min(lo + 1, len(xs) - 1)
        return xs[lo] + (xs[hi] - xs[lo]) * (i - lo)
    return {"median": round(q(0.5), 2), "p10": round(q(0.1), 2), "p90": round(q(0.9), 2), "n": len(xs)}


def time_alternating(runners, rounds, stream):
    """Time every runner's step (and split pass) in `rounds` rounds that visit
    the runners in turn, so drifts of clock or temperature fall on all of them
    alike; each sample is the mean over a block of about BLOCK_US of launches.
    Returns {key: {"run": [...], "split": [...], "block": n}} in µs per launch."""
    res = {}
    for key, r in runners.items():
        for _ in range(3):
            r.run()
        est = max(1.0, block_us(r.run, 5, stream))
        res[key] = {"run": [], "split": [], "block": int(min(2000, max(10, BLOCK_US // est)))}
    for _ in range(rounds):
        for key, r in runners.items():
            n = res[key]["block"]
            res[key]["run"].append(block_us(r.run, n, stream))
            res[key]["split"].append(block_us(r.split, n, stream))
    return res


def host_cpu():
    """The host's CPU model and the threads numpy's BLAS uses (the oracle's)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    return {"model": model, "logical_cpus": os.cpu_count(), "oracle_threads": int(threads)}


def cpu_baseline_configs(runners):
    """CPU-baseline leg over the named configurations: the f64 oracle's wall
    time on each whole batch (median of 3 for the three small ones, one run
    for the two large ones), excluding input copies to the host. Returns
    {key: (seconds, oracle output)}; the outputs also check the GPU's."""
    import oracle
    from decode_attention_kv_04_amd import workloads
    res = {}
    for key, r in runners.items():
        w = r.w
        a = workloads.to_numpy_inputs(w, attended_only=w.window > 0)
        fn = oracle.prefill_attention if a["q"].ndim == 4 else oracle.decode_attention
        times, ref = [], None
        for _ in range(1 if w.kv_bytes() > (1 << 30) or w.window > 0 else 3):
            t = time.perf_counter()
            ref = fn(a["q"], a["k_pool"], a["v_pool"], a["page_table"], a["seq_lens"], a["page_size"], a["scale"],
                     a["window"])
            times.append(time.perf_counter() - t)
        res[key] = (sorted(times)[len(times) // 2], ref)
        print(f"[bench] oracle {key}: {res[key][0]:.2f} s", file=sys.stderr, flush=True)
    return res


def output_check(r, ref):
    """Relative L2 of the runner's last output against the oracle's, over the
    whole output and per (sequence, query head) row, against the bound the
    tests use: the KV-dtype bound, 1e-3 for an fp16 output of fp32 K/V, plus
    2^-8 for a bf16 output (its own rounding)."""
    import numpy as np
    got = r.out.float().cpu().numpy().astype(np.float64)
    spec = r.w.spec
    finite = bool(np.isfinite(got).all())
    res = {"finite": finite}
    if ref is None:
        res["ok"] = finite
        return res
    tol = KV_TOL[spec.kv_dtype]
    if spec.out_dtype == "f16" and spec.kv_dtype == "f32":
        tol = 1e-3
    if spec.out_dtype == "bf16":
        tol += 2.0 ** -8
    D = ref.shape[-1]
    g, f = got.reshape(-1, D), ref.reshape(-1, D)
    den = np.sqrt((f * f).sum(axis=1))
    num = np.sqrt(((g - f) ** 2).sum(axis=1))
    heads = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    whole = float(np.sqrt(((got - ref) ** 2).sum()) / max(np.sqrt((ref * ref).sum()), 1e-300))
    res.update({"rel_l2": float(f"{whole:.3e}"), "worst_head_rel_l2": float(f"{heads.max():.3e}"),
                "tol": tol, "rows_checked": int(heads.size)})
    res["ok"] = finite and whole <= tol and float(heads.max()) <= tol
    return res


def measure_configs(binding, workloads, lib, dev, stream, rounds, headline, ceilings, with_oracle):
    """Every named configuration: step and split-pass µs (median, p10, p90
    over `rounds` alternating repeats), GB/s of algorithmic KV bytes,
    fractions of the 8 TB/s peak and of the measured 4 KiB-gather ceiling,
    cold-cache µs for inputs the last-level cache could hold, the oracle's
    wall time and the check of the timed output against it."""
    import torch
    runners = {}
    for key, name in CONFIGS:
        if headline is not None and workloads.NAMED[name] == headline.w.spec:
            runners[key] = headline
        else:
            w = workloads.make_workload(workloads.NAMED[name], dev)
            runners[key] = Runner(binding, lib, w, dev, stream)
    torch.cuda.synchronize()
    times = time_alternating(runners, rounds, stream)
    refs = cpu_baseline_configs(runners) if with_oracle else {}
    gather = ceilings.get("gather4k")
    out = []
    for key, name in CONFIGS:
        r = runners[key]
        w, spec, t = r.w, r.w.spec, times[key]
        r.out.fill_(float("nan"))
        r.run()
        torch.cuda.synchronize()
        kvb = w.kv_bytes()
        run_q, split_q = quantiles(t["run"]), quantiles(t["split"])
        gbs = kvb / (run_q["median"] * 1e-6) / 1e9
        split_gbs = kvb / (split_q["median"] * 1e-6) / 1e9
        check = output_check(r, refs[key][1] if key in refs else None)
        cold = measure_cold(w, r.plan, lib, r.out, r.ws, stream) if kvb < LLC_BYTES else None
        entry = {
            "config": key, "workload": spec.name, "batch": spec.batch, "heads": [spec.num_q_heads, spec.num_kv_heads],
            "head_dim": spec.head_dim, "dtypes": [spec.q_dtype, spec.kv_dtype, spec.out_dtype],
            "page_size": spec.page_size, "window": spec.window, "attended_keys": int(r.plan.info.attended_keys),
            "algorithmic_bytes": kvb, "split_kernel": int(r.plan.info.split_kernel),
            "max_splits": r.plan.max_splits, "block_launches": t["block"],
            "us": run_q, "split_us": split_q,
            "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBPS, 4),
            "frac_gather4k": round(gbs / gather, 4) if gather else None,
            "split_GB_s": round(split_gbs, 1), "split_frac_hbm_peak": round(split_gbs / HBM_PEAK_GBPS, 4),
            "cold": cold,
        }
        if key in refs:
            entry["oracle_s"] = round(refs[key][0], 3)
        entry["output_check"] = check
        out.append(entry)
        print(f"[bench] {key} {spec.name}: {run_q['median']:.1f} us (p10 {run_q['p10']:.1f}, p90 {run_q['p90']:.1f}), "
              f"{gbs:.0f} GB/s, check {entry['output_check']}", file=sys.stderr, flush=True)
    for key, r in runners.items():
        if r is not headline:
            del r.w, r.out, r.ws
    torch.cuda.empty_cache()
    return out


SWEEP_LENGTHS = tuple(256 << i for i in range(9))   # 256 .. 65536
SWEEP_BATCHES = (1, 32)


def measure_sweep(binding, workloads, lib, dev, stream, rounds):
    """Context-length sweep on the Llama-3.1-8B decode shape (32/8 heads, D
    128, fp16, 16-token pages): every sequence of the batch at context L, for
    L = 256 .. 65536 and batch 1 and 32; step and split µs (median, p10, p90
    over alternating repeats within each batch size) and GB/s."""
    import torch
    res = []
    for B in SWEEP_BATCHES:
        runners = {}
        for L in SWEEP_LENGTHS:
            spec = workloads.LLAMA8B_3060.replace(name=f"llama8b_b{B}_l{L}_f16", batch=B, lengths=("fixed", L),
                                                  seed=100 + L % 97 + B, max_pages_per_seq=L // 16)
            runners[L] = Runner(binding, lib, workloads.make_workload(spec, dev), dev, stream)
        torch.cuda.synchronize()
        times = time_alternating(runners, rounds, stream)
        for L, r in runners.items():
            kvb = r.w.kv_bytes()
            run_q, split_q = quantiles(times[L]["run"]), quantiles(times[L]["split"])
            gbs = kvb / (run_q["median"] * 1e-6) / 1e9
            res.append({"batch": B, "context": L, "us": run_q, "split_us": split_q, "GB_s": round(gbs, 1),
                        "frac_hbm_peak": round(gbs / HBM_PEAK_GBPS, 4), "max_splits": r.plan.max_splits,
                        "split_kernel": int(r.plan.info.split_kernel), "algorithmic_bytes": kvb})
            print(f"[bench] sweep B {B} L {L}: {run_q['median']:.1f} us, {gbs:.0f} GB/s", file=sys.stderr,
                  flush=True)
        del runners
        torch.cuda.empty_cache()
    return res


def measure_head_dims(binding, workloads, lib, dev, stream, rounds):
    """The Llama-3.1-8B decode shape at 3060 tokens with head_dim 64, 128 and
    256 (32/8 heads, fp16, 16-token pages), batch 1 and 32: step and split
    µs over alternating repeats, GB/s, and the split kernel the plan picks."""
    import torch
    res = []
    for B in SWEEP_BATCHES:
        runners = {}
        for D in (64, 128, 256):
            spec = workloads.LLAMA8B_3060.replace(name=f"llama8b_b{B}_l3060_d{D}_f16", batch=B, head_dim=D,
                                                  seed=300 + D + B)
            runners[D] = Runner(binding, lib, workloads.make_workload(spec, dev), dev, stream)
        torch.cuda.synchronize()
        times = time_alternating(runners, rounds, stream)
        for D, r in runners.items():
            kvb = r.w.kv_bytes()
            run_q, split_q = quantiles(times[D]["run"]), quantiles(times[D]["split"])
            gbs = kvb / (run_q["median"] * 1e-6) / 1e9
            res.append({"batch": B, "context": 3060, "head_dim": D, "us": run_q, "split_us": split_q,
                        "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBPS, 4),
                        "max_splits": r.plan.max_splits, "split_kernel": int(r.plan.info.split_kernel),
                        "algorithmic_bytes": kvb})
            print(f"[bench] head_dim {D} B {B} L 3060: {run_q['median']:.1f} us, {gbs:.0f} GB/s", file=sys.stderr,
                  flush=True)
        del runners
        torch.cuda.empty_cache()
    return res


def measure_groups(binding, workloads, lib, dev, stream, rounds):
    """Query heads per KV head 1, 2, 4, 8 and 16 (8 KV heads, head_dim 128,
    fp16, 16-token pages) at batch 1 x 3060 and batch 32 x 4096 tokens: step
    and split µs over alternating repeats, GB/s of K/V, and the split kernel
    the plan picks (G 16 has only the multi-token kernel)."""
    import torch
    res = []
    for B, L in ((1, 3060), (32, 4096)):
        runners = {}
        for G in (1, 2, 4, 8, 16):
            spec = workloads.LLAMA8B_3060.replace(name=f"g{G}_b{B}_l{L}_f16", batch=B, num_q_heads=8 * G,
                                                  lengths=("fixed", L), seed=500 + G + B)
            runners[G] = Runner(binding, lib, workloads.make_workload(spec, dev), dev, stream)
        torch.cuda.synchronize()
        times = time_alternating(runners, rounds, stream)
        for G, r in runners.items():
            kvb = r.w.kv_bytes()
            run_q, split_q = quantiles(times[G]["run"]), quantiles(times[G]["split"])
            gbs = kvb / (run_q["median"] * 1e-6) / 1e9
            res.append({"batch": B, "context": L, "group": G, "heads": [8 * G, 8], "us": run_q, "split_us": split_q,
                        "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBPS, 4),
                        "max_splits": r.plan.max_splits, "split_kernel": int(r.plan.info.split_kernel),
                        "algorithmic_bytes": kvb})
            print(f"[bench] G {G} B {B} L {L}: {run_q['median']:.1f} us, {gbs:.0f} GB/s", file=sys.stderr,
                  flush=True)
        del runners
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long_batch", help="one of: long_batch, llama8b_3060, wide_gqa, "
                    "mixed_window, tiny")
    ap.add_argument("--num-splits", type=int, default=0, help="0 = the planner decides")
    ap.add_argument("--rounds", type=int, default=7, help="alternating repeats per configuration")
    ap.add_argument("--no-configs", action="store_true", help="skip the five named configurations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-multi-token", action="store_true", help="skip the multi-token workloads")
    ap.add_argument("--layer-step-only", action="store_true",
                    help="only the 32-layer decode step of the Llama-3.1-8B shape at 3060 tokens (for traces)")
    ap.add_argument("--sweep", action="store_true",
                    help="only the context-length sweep (Llama shape, L 256..65536, batch 1 and 32) and "
                    "the head_dim sweep at 3060 tokens, and query heads per KV head 1..16")
    ap.add_argument("--calibrate", action="store_true",
                    help="after timing, copy a buffer of known size once (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from decode_attention_kv_04_amd import binding, workloads
    if not os.path.exists(binding.library_path()):
        from decode_attention_kv_04_amd import build as _build
        _build.build_library()

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    lib = binding.load()
    sptr = stream.cuda_stream

    if args.layer_step_only:
        ls = measure_layer_step(binding, workloads, dev, stream, args.steps)
        print(json.dumps({"metric": METRIC, "layer_step": ls, "n_gpus": 1, "data": "synthetic",
                          "kernel_source_sha256_16": kernel_hash()}), flush=True)
        return

    if args.sweep:
        sweep = measure_sweep(binding, workloads, lib, dev, stream, args.rounds)
        head_dims = measure_head_dims(binding, workloads, lib, dev, stream, args.rounds)
        groups = measure_groups(binding, workloads, lib, dev, stream, args.rounds)
        print(json.dumps({"metric": METRIC, "sweep": sweep, "head_dims": head_dims, "groups": groups,
                          "unit": "GB/s", "n_gpus": 1,
                          "data": "synthetic", "kernel_source_sha256_16": kernel_hash()}), flush=True)
        return

    spec = workloads.NAMED[args.workload]
    print(f"[bench] generating {spec.name} on {dev}", file=sys.stderr, flush=True)
    w = workloads.make_workload(spec, dev)
    torch.cuda.synchronize()
    kv_bytes = w.kv_bytes()

    params = binding.params_for(w.q, w.k_pool, w.page_table, window=w.window, scale=w.scale,
                                out_dtype=spec.out_dtype, num_splits=args.num_splits)
    # The first plan also reads the device's CU count; the host cost of a
    # plan is the median of later calls.
    head = Runner(binding, lib, w, dev, stream, num_splits=args.num_splits)
    plan = head.plan
    plan_times = []
    for _ in range(21):
        t = time.perf_counter()
        again = binding.decode_attn_plan(params, w.seq_lens_host, device=0)
        plan_times.append((time.perf_counter() - t) * 1e6)
        del again
    plan_us = sorted(plan_times)[len(plan_times) // 2]
    out, ws, ptrs = head.out, head.ws, head.ptrs

    def combine_only():
        st = lib.decode_attn_combine(plan.handle, ptrs[4], ptrs[5], ptrs[6], ptrs[7], sptr)
        if st != 0:
            raise binding.DecodeAttnError(st, "decode_attn_combine")

    print(f"[bench] plan: pages/split {plan.pages_per_split}, max splits {plan.max_splits}, "
          f"work-groups {plan.info.split_work_groups}; warmup {args.warmup}", file=sys.stderr, flush=True)
    out.fill_(float("nan"))
    for _ in range(args.warmup):
        head.run()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps, synchronized on both sides.
    torch.cuda.synchronize()
    ms_per_step = time_on_stream(head.run, args.steps, stream)
    print(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    timed_out = out.clone()   # the output the timed steps left, checked against the oracle below

    # The dominant kernel alone (split pass), then the combine pass alone.
    split_ms = time_on_stream(head.split, args.steps, stream)
    combine_ms = time_on_stream(combine_only, args.steps, stream) if plan.max_splits > 1 else 0.0

    ceilings = {}
    if not args.no_ceiling:
        ceilings = measure_ceilings(dev, sptr, stream)

    # The five named configurations (the headline batch among them, reusing
    # its inputs), over alternating repeats, with the oracle's time on each.
    configs = None
    if not args.no_configs and args.num_splits == 0:
        configs = measure_configs(binding, workloads, lib, dev, stream, args.rounds,
                                  head if args.workload in dict(CONFIGS).values() else None, ceilings,
                                  not args.no_cpu_baseline)

    # The headline's timed output against the oracle: the configuration list
    # re-ran the same plan on the same inputs and checked that output, which
    # must be bitwise the timed one (the step is deterministic).
    head_check = {"finite": bool(torch.isfinite(timed_out.float()).all().item())}
    for c in configs or []:
        if c["workload"] == spec.name:
            same = bool(torch.equal(out, timed_out))
            head_check = dict(c["output_check"], timed_output_identical=same)
            head_check["ok"] = head_check["ok"] and same
    head_check.setdefault("ok", head_check["finite"])

    # The fixed-order mode (output bitwise independent of the split count) on
    # the same batch: whole step, chunks of FIXED_CHUNK tokens.
    fixed = measure_fixed_order(w, binding, lib, dev, stream, args.steps) if spec.query_len == 1 else None

    # Several new tokens per sequence (drafted-token check, suffix prefill).
    multi = [] if args.no_multi_token else measure_multi_token(binding, workloads, lib, dev, stream, args.rounds)

    # One whole decode step (32 layers) of the Llama-3.1-8B shape at 3060
    # tokens, eager and as a replayed HIP graph.
    layer_step = None if args.no_multi_token else measure_layer_step(binding, workloads, dev, stream, args.steps)

    # K/V append (the step before the path): one token per sequence, and a
    # 256-token suffix; written rows equal the resident rows.
    append_stats = [measure_append(w, lib, params, stream, t, args.steps) for t in (1, 256)]

    # Workloads the last-level cache could hold are also timed cold.
    cold = measure_cold(w, plan, lib, out, ws, stream) if kv_bytes < 2 * LLC_BYTES else None

    if args.calibrate:
        calibration_copy(dev, sptr)

    achieved = kv_bytes / (split_ms * 1e-3) / 1e9
    traffic = recorded_traffic()
    cpu = None if args.no_cpu_baseline else cpu_baseline(w)
    if cpu is not None:
        cpu["host"] = host_cpu()

    step_gbps = kv_bytes / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(step_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * step_gbps / HBM_PEAK_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.kv_dtype,
        "data": "synthetic (seeded torch generator on the GPU, shapes and distributions of the workload)",
        "config": {
            "workload": spec.name,
            "batch": spec.batch, "num_q_heads": spec.num_q_heads, "num_kv_heads": spec.num_kv_heads,
            "head_dim": spec.head_dim, "page_size": spec.page_size, "window": spec.window,
            "context": list(spec.lengths), "attended_keys": int(plan.info.attended_keys),
            "kv_dtype": spec.kv_dtype, "out_dtype": spec.out_dtype,
            "pages_per_split": plan.pages_per_split, "max_splits": plan.max_splits,
            "parallelism": "single GPU",
        },
        "output_check": head_check,
        "roofline": {
            "bound": "hbm",
            "kernel": {0: "split pass, vector q.K (da::split_kernel)",
                       1: "split pass, q.K on the matrix cores (da::split_kernel_mfma)",
                       2: "multi-token split pass (da::multi_dma_kernel)"}[plan.info.split_kernel],
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_source": ("FETCH_SIZE + WRITE_SIZE per launch from the committed counter summary "
                               "(profiles/split_kernel_long_batch_traffic.md), valid while the kernel sources "
                               "keep its hash; null otherwise") if traffic is not None else None,
            "algorithmic_bytes_per_launch": kv_bytes,
            "avg_launch_us": round(split_ms * 1e3, 2),
        },
        "configs": configs,
        "configs_oracle_host": host_cpu() if configs and not args.no_cpu_baseline else None,
        "cold": cold,
        "combine_us": round(combine_ms * 1e3, 2),
        "fixed_order": fixed,
        "multi_token": multi,
        "layer_step": layer_step,
        "append_kv": append_stats,
        "plan_host_us": round(plan_us, 1),
        "hbm_read_ceiling_GBps": ceilings.get("stream"),
        "gather4k_read_ceiling_GBps": ceilings.get("gather4k"),
        "split_frac_of_gather4k_ceiling": (round(achieved / ceilings["gather4k"], 4)
                                           if ceilings.get("gather4k") else None),
        "calibration_copy_bytes": CALIBRATION_BYTES if args.calibrate else None,
        "cpu_baseline": cpu,
        "kernel_source_sha256_16": kernel_hash(),
    }
    print(json.dumps(result), flush=True)
    if not head_check["ok"] or any(not c["output_check"]["ok"] for c in configs or []):
        print("[bench] an output check against the oracle FAILED (see output_check)", file=sys.stderr, flush=True)
        sys.exit(1)


if __name__ == "__main__":
    main()
