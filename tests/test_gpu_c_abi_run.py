"""A C program (tests/c_abi_run.c, C99, built here with gcc against
include/decode_attn.h, the library and the HIP runtime) allocates every
device buffer with hipMalloc and runs decode attention through the C ABI:
decode_attn_run, decode_attn_split + decode_attn_combine and
decode_attn_run_noalloc on the same inputs. Its outputs must agree with each
other bit for bit and with the oracle."""
import os
import subprocess

import numpy as np
import pytest
import torch

from decode_attention_kv_04_amd import binding
from decode_attention_kv_04_amd import workloads as wl

from gpu_util import check, oracle_for, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
NP_DT = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


@pytest.fixture(scope="module")
def c_program(tmp_path_factory, lib):
    exe = str(tmp_path_factory.mktemp("c_abi_run") / "c_abi_run")
    pkg = os.path.dirname(binding.library_path())
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_abi_run.c"), "-o", exe,
           "-L", pkg, "-ldecode_attn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{pkg}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def raw(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.numpy().tobytes()


def run_c(exe, w, out_dtype, d, num_splits=0):
    s = w.spec
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "params.txt"), "w") as f:
        f.write(" ".join(str(x) for x in (
            s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim, s.page_size, w.page_table.shape[1], w.window,
            repr(w.scale), binding.DTYPE_CODES[s.q_dtype], binding.DTYPE_CODES[s.kv_dtype],
            binding.DTYPE_CODES[out_dtype], num_splits, w.num_pages)) + "\n")
    for name, t in (("q.bin", w.q), ("k.bin", w.k_pool), ("v.bin", w.v_pool), ("table.bin", w.page_table),
                    ("lens.bin", w.seq_lens)):
        with open(os.path.join(d, name), "wb") as f:
            f.write(raw(t))
    r = subprocess.run([exe, d], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip(), r.stderr.strip())
    assert r.returncode == 0, r.stderr
    outs = []
    for name in ("out_run.bin", "out_two.bin", "out_noalloc.bin"):
        a = np.fromfile(os.path.join(d, name), dtype=NP_DT[out_dtype]).reshape(tuple(w.q.shape))
        if out_dtype == "bf16":
            a = (a.astype(np.uint32) << 16).view(np.float32)
        outs.append(a.astype(np.float64))
    return outs


CASES = [
    ("llama8b", wl.LLAMA8B_3060.replace(batch=3, lengths=("list", (3060, 17, 0))), 0),
    ("llama8b-splits", wl.LLAMA8B_3060.replace(batch=2, lengths=("list", (3060, 700))), 7),
    ("wide-gqa-bf16", wl.WIDE_GQA, 0),
    ("mixed-window-bf16", wl.MIXED_WINDOW.replace(batch=3, lengths=("list", (9000, 40, 5000)),
                                                  out_dtype="bf16"), 0),
    ("tiny-f32", wl.TINY, 0),
]


@pytest.mark.parametrize("name,spec,ns", CASES, ids=[c[0] for c in CASES])
def test_c_program_runs_the_step(gpu, c_program, tmp_path, name, spec, ns):
    say(f"[c-abi-run] {name}")
    w = wl.make_workload(spec, "cpu")           # host inputs, handed to the C program as files
    ref = oracle_for(w)
    outs = run_c(c_program, w, spec.out_dtype, str(tmp_path / "out"), ns)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])       # split + combine and the no-alloc call equal run
    twin = None
    if spec.out_dtype in ("f16", "bf16"):
        twin = run_c(c_program, w, "f32", str(tmp_path / "f32"), ns)[0]
    err, worst = check(outs[0], ref, spec.kv_dtype, spec.out_dtype, f"C program {name}", twin=twin)
    say(f"  rel L2 {err:.2e}, worst sequence {worst:.2e}")
