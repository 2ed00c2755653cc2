"""Paged single-query decode attention for MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``csrc/``, header ``include/decode_attn.h``); ``binding`` is a thin ctypes
layer over it that passes torch tensors' device pointers and the current
stream. ``workloads`` draws seeded synthetic inputs.
"""
