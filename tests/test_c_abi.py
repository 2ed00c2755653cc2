"""The C ABI from a C99 program (no Python in between): tests/c_abi_plan.c is
compiled with gcc against include/decode_attn.h and the built library, run on
the CPU (planning makes no HIP call), and its plan must equal the one the
ctypes binding gets for the same parameters."""
import math
import os
import re
import shutil
import subprocess

import pytest

from decode_attention_kv_04_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_plans_like_the_binding(lib, tmp_path):
    exe = str(tmp_path / "c_abi_plan")
    libdir = os.path.dirname(B.library_path())
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_plan.c"), "-o", exe, "-L", libdir, "-ldecode_attn",
                    f"-Wl,-rpath,{libdir}"], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    out = r.stdout
    got = dict((k, int(v)) for k, v in re.findall(r"(\w+) (\d+)", out.splitlines()[0]))
    lens = [16384 + (b * 523) % 16384 for b in range(32)]
    params = B.make_params(32, 32, 8, 128, 16, 2048, scale=128 ** -0.5)
    pl = B.decode_attn_plan_for_cus(params, lens, 256)
    assert got["pages_per_split"] == pl.pages_per_split
    assert got["max_splits"] == pl.max_splits
    assert got["split_work_groups"] == pl.info.split_work_groups
    assert got["split_kernel"] == pl.info.split_kernel == 1
    assert got["balanced"] == pl.info.balanced == 1
    assert got["attended_keys"] == sum(lens)
    assert got["workspace"] == pl.workspace_bytes
    # balanced schedule: units (sequence, KV head, page) dealt q at a time
    q = pl.pages_per_split
    ov = 65536 // (2 * 16 * 128 * 2)      # start weight of a stream, in units
    start = 0
    for b in range(3):
        n = math.ceil(lens[b] / 16)
        pieces = []
        for _ in range(8):
            pieces.append((start + ov + n - 1) // q - (start + ov) // q + 1)
            start += ov + n
        assert f"splits[{b}] {pl.splits(b)}" in out
        assert pl.splits(b) == max(pieces)
    assert "invalid: DA_ERR_INVALID" in out
