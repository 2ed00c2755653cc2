"""ctypes binding of ``libdecode_attn.so`` (``include/decode_attn.h``).

Argument marshalling only: torch tensors are passed as device pointers and the
current torch stream as the HIP stream; every step of the computation runs in
the library's HIP kernels. A missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libdecode_attn.so"

DA_OK, DA_ERR_INVALID, DA_ERR_UNSUPPORTED, DA_ERR_WORKSPACE, DA_ERR_HIP = range(5)
DA_F32, DA_F16, DA_BF16 = 0, 1, 2
DTYPE_CODES = {"f32": DA_F32, "f16": DA_F16, "bf16": DA_BF16}
DA_KERNEL_AUTO, DA_KERNEL_VECTOR, DA_KERNEL_MATRIX = range(3)
KERNEL_CODES = {None: DA_KERNEL_AUTO, "auto": DA_KERNEL_AUTO, "vector": DA_KERNEL_VECTOR,
                "matrix": DA_KERNEL_MATRIX}

# Every symbol include/decode_attn.h declares.
EXPORTS = (
    "decode_attn_plan", "decode_attn_plan_for_cus", "decode_attn_plan_info", "decode_attn_plan_splits",
    "decode_attn_run", "decode_attn_split", "decode_attn_combine", "decode_attn_append_kv",
    "decode_attn_run_noalloc", "decode_attn_plan_destroy", "decode_attn_status_str",
)
SCRATCH_BYTES = 64 * 1024 * 1024  # DECODE_ATTN_SCRATCH_BYTES


class DecodeAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


class Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("window", ctypes.c_int32), ("scale", ctypes.c_float),
        ("q_dtype", ctypes.c_int), ("kv_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("num_splits", ctypes.c_int32), ("fixed_chunk", ctypes.c_int32), ("query_len", ctypes.c_int32),
        ("kernel", ctypes.c_int32), ("rows_per_block", ctypes.c_int32),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("pages_per_split", ctypes.c_int32), ("max_splits", ctypes.c_int32), ("num_cus", ctypes.c_int32),
        ("split_work_groups", ctypes.c_int32), ("active_units", ctypes.c_int64),
        ("attended_keys", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
        ("split_kernel", ctypes.c_int32), ("chunks_per_work_group", ctypes.c_int32),
        ("balanced", ctypes.c_int32),
    ]


_lib = None


def library_path() -> str:
    return os.path.join(PKG, _LIB_NAME)


def load() -> ctypes.CDLL:
    """Load the library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(python -m decode_attention_kv_04_amd.build)")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    plan_p = ctypes.POINTER(ctypes.c_void_p)
    lens_p = ctypes.POINTER(ctypes.c_int32)
    lib.decode_attn_plan.argtypes = [ctypes.POINTER(Params), lens_p, ctypes.c_int, plan_p, ctypes.POINTER(sz)]
    lib.decode_attn_plan_for_cus.argtypes = [ctypes.POINTER(Params), lens_p, i32, plan_p, ctypes.POINTER(sz)]
    lib.decode_attn_plan_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    lib.decode_attn_plan_splits.argtypes = [vp, i32]
    lib.decode_attn_plan_splits.restype = i32
    run_args = [vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.decode_attn_run.argtypes = run_args
    lib.decode_attn_split.argtypes = run_args
    lib.decode_attn_combine.argtypes = [vp, vp, vp, vp, sz, vp]
    lib.decode_attn_append_kv.argtypes = [ctypes.POINTER(Params), i32, vp, vp, vp, vp, vp, vp, vp]
    lib.decode_attn_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
    lib.decode_attn_plan_destroy.argtypes = [vp]
    lib.decode_attn_plan_destroy.restype = None
    lib.decode_attn_status_str.argtypes = [ctypes.c_int]
    lib.decode_attn_status_str.restype = ctypes.c_char_p
    for name in ("decode_attn_plan", "decode_attn_plan_for_cus", "decode_attn_plan_info", "decode_attn_run",
                 "decode_attn_split", "decode_attn_combine", "decode_attn_append_kv", "decode_attn_run_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().decode_attn_status_str(int(status)).decode()


decode_attn_status_str = status_str


def make_params(batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_seq, *, window=0,
                scale=None, q_dtype="f16", kv_dtype="f16", out_dtype="f16", num_splits=0,
                fixed_chunk=0, query_len=1, kernel=None, rows_per_block=0) -> Params:
    """da_params; `kernel` is None / "auto", "vector", "matrix" or a da_kernel code."""
    def code(t):
        return DTYPE_CODES[t] if isinstance(t, str) else int(t)
    kern = KERNEL_CODES[kernel] if kernel is None or isinstance(kernel, str) else int(kernel)
    return Params(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim), int(page_size),
                  int(max_pages_per_seq), int(window),
                  float(scale if scale is not None else (head_dim ** -0.5 if head_dim > 0 else 1.0)),
                  code(q_dtype), code(kv_dtype), code(out_dtype), int(num_splits), int(fixed_chunk),
                  int(query_len), kern, int(rows_per_block))


class Plan:
    """Owns a da_plan_t; freed when garbage-collected or on close()."""

    def __init__(self, handle: int, params: Params):
        self.handle = ctypes.c_void_p(handle)
        self.params = params
        self._lib = load()  # the library that made the plan also frees it
        info = PlanInfo()
        st = load().decode_attn_plan_info(self.handle, ctypes.byref(info))
        if st != DA_OK:
            raise DecodeAttnError(st, "decode_attn_plan_info")
        self.info = info

    @property
    def workspace_bytes(self) -> int:
        return int(self.info.workspace_bytes)

    @property
    def max_splits(self) -> int:
        return int(self.info.max_splits)

    @property
    def pages_per_split(self) -> int:
        return int(self.info.pages_per_split)

    def splits(self, b: int) -> int:
        return int(load().decode_attn_plan_splits(self.handle, int(b)))

    def close(self):
        if self.handle:
            self._lib.decode_attn_plan_destroy(self.handle)
            self.handle = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _lens_array(seq_lens_host: Sequence[int]):
    vals = [int(x) for x in (seq_lens_host.tolist() if hasattr(seq_lens_host, "tolist") else seq_lens_host)]
    arr = (ctypes.c_int32 * max(1, len(vals)))(*vals)
    return arr, len(vals)


def decode_attn_plan(params: Params, seq_lens_host, device: Optional[int] = None) -> Plan:
    """Plan for the host-side lengths on HIP device `device` (default: torch's current device)."""
    if device is None:
        import torch
        device = torch.cuda.current_device()
    arr, n = _lens_array(seq_lens_host)
    h = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    st = load().decode_attn_plan(ctypes.byref(params), arr if n else None, int(device), ctypes.byref(h),
                                 ctypes.byref(ws))
    if st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_plan")
    return Plan(h.value, params)


def decode_attn_plan_for_cus(params: Params, seq_lens_host, num_cus: int) -> Plan:
    """Plan for an explicit compute-unit count (no HIP call; works without a GPU)."""
    arr, n = _lens_array(seq_lens_host)
    h = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    st = load().decode_attn_plan_for_cus(ctypes.byref(params), arr if n else None, int(num_cus),
                                         ctypes.byref(h), ctypes.byref(ws))
    if st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_plan_for_cus")
    return Plan(h.value, params)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("decode_attn: tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("decode_attn: tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    if t is None:
        return 0
    return t.numel() * t.element_size()


def decode_attn_run(plan: Plan, q, k_pool, v_pool, page_table, seq_lens, out, workspace=None, stream=None):
    st = load().decode_attn_run(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table), _ptr(seq_lens),
                                _ptr(out), _ptr(workspace), _nbytes(workspace), _stream(stream))
    if st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_run")


def decode_attn_run_noalloc(plan: Plan, q, k_pool, v_pool, page_table, seq_lens, out, stream=None):
    """decode_attn_run with the split states in the library's static scratch (no workspace)."""
    st = load().decode_attn_run_noalloc(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
                                        _ptr(seq_lens), _ptr(out), _stream(stream))
    if st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_run_noalloc")


def decode_attn_split(plan: Plan, q, k_pool, v_pool, page_table, seq_lens, out, workspace=None, stream=None):
    st = load().decode_attn_split(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
                                  _ptr(seq_lens), _ptr(out), _ptr(workspace), _nbytes(workspace), _stream(stream))
    if st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_split")


def decode_attn_combine(plan: Plan, seq_lens, out, workspace=None, stream=None):
    st = load().decode_attn_combine(plan.handle, _ptr(seq_lens), _ptr(out), _ptr(workspace), _nbytes(workspace),
                                    _stream(stream))
    if st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_combine")


def decode_attn_append_kv(params: Params, k_new, v_new, page_table, seq_lens, k_pool, v_pool, stream=None):
    """Write k_new / v_new ([B][T][H_kv][D]) after each sequence's seq_lens keys."""
    tokens = int(k_new.shape[1]) if k_new is not None else 0
    st = load().decode_attn_append_kv(ctypes.byref(params), tokens, _ptr(k_new), _ptr(v_new), _ptr(page_table),
                                      _ptr(seq_lens), _ptr(k_pool), _ptr(v_pool), _stream(stream))
    if st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_append_kv")


def params_for(q, k_pool, page_table, *, window=0, scale=None, out_dtype=None, num_splits=0,
               fixed_chunk=0, kernel=None, rows_per_block=0) -> Params:
    """da_params from tensor shapes and dtypes; q is [B][H_q][D] (one query
    token per sequence) or [B][T][H_q][D] (T new tokens per sequence)."""
    import torch
    names = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}
    if q.dim() == 4:
        B, T, Hq, D = q.shape
    else:
        (B, Hq, D), T = q.shape, 1
    _, Hkv, P, D2 = k_pool.shape
    assert D == D2, "q and the pools disagree on head_dim"
    return make_params(B, Hq, Hkv, D, P, page_table.shape[1], window=window, scale=scale,
                       q_dtype=names[q.dtype], kv_dtype=names[k_pool.dtype],
                       out_dtype=out_dtype or names[q.dtype], num_splits=num_splits, fixed_chunk=fixed_chunk,
                       query_len=T, kernel=kernel, rows_per_block=rows_per_block)


def alloc_workspace(plan: Plan, device):
    """Device workspace of the size `plan` needs (None if it needs none)."""
    import torch
    if plan.workspace_bytes == 0:
        return None
    return torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=device)


def decode_attention(q, k_pool, v_pool, page_table, seq_lens, seq_lens_host=None, *, window=0, scale=None,
                     out_dtype=None, num_splits=0, fixed_chunk=0, out=None, workspace=None, stream=None):
    """Plan, allocate (output and workspace, through torch) and run one step."""
    import torch
    params = params_for(q, k_pool, page_table, window=window, scale=scale, out_dtype=out_dtype,
                        num_splits=num_splits, fixed_chunk=fixed_chunk)
    host = seq_lens_host if seq_lens_host is not None else seq_lens.cpu()
    plan = decode_attn_plan(params, host, device=q.device.index)
    dt = {DA_F32: torch.float32, DA_F16: torch.float16, DA_BF16: torch.bfloat16}[params.out_dtype]
    if out is None:
        out = torch.empty(q.shape, dtype=dt, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(plan, q.device)
    decode_attn_run(plan, q, k_pool, v_pool, page_table, seq_lens, out, workspace, stream)
    return out
