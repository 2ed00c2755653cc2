"""Build the HIP library in-tree: ``libdecode_attn.so`` (split and combine
kernels, planner, C ABI) and ``libda_probe.so`` (the bandwidth probe the
benchmark uses to calibrate counters), both for gfx950.

Host-only sources are compiled with g++, kernel sources with hipcc; hipcc
links. Packed fp32 VALU instructions are switched off for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))
ARCH = "gfx950"

LIB = os.path.join(PKG, "libdecode_attn.so")
PROBE_LIB = os.path.join(PKG, "libda_probe.so")

HIP_FLAGS = [
    "-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]

HOST_SOURCES = ["plan.cpp", "api.cpp"]
KERNEL_SOURCES = ["decode_split.hip", "decode_split_mfma.hip", "decode_combine.hip", "append_kv.hip",
                  "decode_multi.hip", "scratch.hip"]
PROBE_SOURCES = ["probe.hip"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    inc = ["-I", INCLUDE, "-I", CSRC]
    if src.endswith(".hip"):
        cmd = [HIPCC, *HIP_FLAGS, *inc, "-c", path, "-o", obj]
    else:
        cmd = ["g++", *CXX_FLAGS, "-D__HIP_PLATFORM_AMD__", *inc, "-I", os.path.join(ROCM, "include"),
               "-c", path, "-o", obj]
    _run(cmd)
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)


def build_library(verbose: bool = False) -> str:
    """Compile every source and link both libraries; returns the main library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = HOST_SOURCES + KERNEL_SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in HOST_SOURCES + KERNEL_SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
