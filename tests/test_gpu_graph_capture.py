"""The library makes no allocation, host synchronisation or memset inside a
step, so a caller can capture decode_attn_run (split + combine launches) in a
HIP graph and replay it: every replay must equal the eager result bitwise,
with eager work and synchronisations between the replays."""
import pytest
import torch

from decode_attention_kv_04_amd import binding
from decode_attention_kv_04_amd import workloads as wl

from gpu_util import TORCH_DT, say

pytestmark = pytest.mark.gpu


CASES = [
    # (workload, overrides, fixed_chunk)
    ("llama8b_3060", {}, 0),                                                          # one token, multi-token kernel
    ("long_batch", {"batch": 4, "num_q_heads": 64, "lengths": ("list", (20000, 3060, 100, 9000))}, 0),  # GQA 8
    ("mixed_window", {"batch": 4, "lengths": ("list", (100, 40000, 7, 33000))}, 0),
    ("llama8b_3060", {"batch": 3, "lengths": ("list", (3060, 9000, 1))}, 256),      # fixed-order mode
    ("verify_long", {"batch": 3, "lengths": ("list", (20000, 4, 900))}, 0),          # multi-token kernel
    ("verify_long", {"batch": 2, "lengths": ("list", (5000, 77)), "q_dtype": "bf16",
                     "out_dtype": "f32"}, 0),                                          # per-token launches
]


@pytest.mark.parametrize("name,kw,fixed_chunk", CASES)
def test_captured_step_replays_bitwise(gpu, name, kw, fixed_chunk):
    spec = wl.NAMED[name].replace(**kw) if kw else wl.NAMED[name]
    say(f"[graph] {spec.name} {kw} fixed_chunk={fixed_chunk}")
    w = wl.make_workload(spec, gpu)
    params = binding.params_for(w.q, w.k_pool, w.page_table, window=w.window, scale=w.scale,
                                out_dtype=spec.out_dtype, fixed_chunk=fixed_chunk)
    plan = binding.decode_attn_plan(params, w.seq_lens_host, device=gpu.index or 0)
    ws = binding.alloc_workspace(plan, gpu)
    eager = torch.empty(w.q.shape, dtype=TORCH_DT[spec.out_dtype], device=gpu)
    binding.decode_attn_run(plan, w.q, w.k_pool, w.v_pool, w.page_table, w.seq_lens, eager, ws)
    torch.cuda.synchronize()

    out = torch.full_like(eager, float("nan"))
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            binding.decode_attn_run(plan, w.q, w.k_pool, w.v_pool, w.page_table, w.seq_lens, out, ws, stream=stream)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        if ws is not None:
            ws.fill_(0xFF)                       # stale states must not matter
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager step"
        # eager work between replays
        again = torch.empty_like(eager)
        binding.decode_attn_run(plan, w.q, w.k_pool, w.v_pool, w.page_table, w.seq_lens, again, ws)
        torch.cuda.synchronize()
        assert torch.equal(again, eager)
