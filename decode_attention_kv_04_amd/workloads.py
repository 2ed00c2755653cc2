"""Seeded synthetic inputs for paged single-query decode attention.

This module only *draws and lays out* inputs: lengths, a shuffled page pool,
a page table, q, K and V. It holds none of the attention arithmetic, so both
the HIP path and the CPU oracle can be fed from it without sharing any of the
method's code.

Layouts (the library's contract):

* ``q``          [B][H_q][D]                 in ``q_dtype``
* ``k_pool``     [num_pages][H_kv][P][D]     in ``kv_dtype`` (one contiguous
  P x D block per (page, KV head))
* ``v_pool``     same shape as ``k_pool``
* ``page_table`` [B][max_pages_per_seq]      int32, logical page -> physical page
* ``seq_lens``   [B]                         int32, keys in the cache for each
  sequence (the newest token's K/V included)

Every slot that the attention must not read is NaN: the tail of the last page,
the keys before a sliding window, the pages wholly before the window, and one
extra "poison" page that unused page-table entries point at. A masking bug that
lets any of them in turns the output into NaN.

Draw order for a seed: lengths, short/long assignment, page permutation (all
from a CPU generator, so the structure does not depend on the device), then q,
K with its spike mask, V (from a generator on the target device; pass
``device="cpu"`` for values that are identical on every machine).

The five named workloads are the shapes the paged decode-attention pages
measure or imply (TVM pull 20426, commit message of the sharded nest: the
Llama-3.1-8B shape at 3060 tokens, head_dim 64/128/256, sliding windows),
sized for one MI355X.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    """Shape and value recipe of one synthetic decode-attention batch.

    ``lengths`` is one of
      ("fixed", L)                          every sequence has L keys
      ("uniform", lo, hi)                   integers uniform in [lo, hi]
      ("mixed", (lo1, hi1), (lo2, hi2))     exactly B//2 sequences from the
                                            first range, the rest from the
                                            second, order shuffled by the seed
      ("list", (L0, L1, ...))               explicit lengths
    """

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str
    kv_dtype: str
    out_dtype: str
    page_size: int
    lengths: tuple
    seed: int
    window: int = 0
    spike_frac: float = 0.0
    spike_scale: float = 8.0
    shuffle: bool = True
    max_pages_per_seq: Optional[int] = None
    scale: Optional[float] = None  # default 1/sqrt(head_dim)
    query_len: int = 1             # T new tokens per sequence (the last T keys); q is [B][T][H_q][D] if T > 1

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def replace(self, **kw) -> "WorkloadSpec":
        return dataclasses.replace(self, **kw)


# The five configurations, in order: tiny, Llama-3.1-8B decode shape at 3060
# tokens, wide-head GQA, batched long context (the throughput workload) and a
# mixed sliding-window batch.
TINY = WorkloadSpec("tiny_b1_h1_d64_f32_l256", 1, 1, 1, 64, "f32", "f32", "f32", 16,
                    ("fixed", 256), seed=1, shuffle=False, scale=0.125)
LLAMA8B_3060 = WorkloadSpec("llama8b_b1_l3060_f16", 1, 32, 8, 128, "f16", "f16", "f16", 16,
                            ("fixed", 3060), seed=2)
WIDE_GQA = WorkloadSpec("widehead_b4_h8kv4_d256_bf16_l1-4096", 4, 8, 4, 256, "bf16", "bf16", "f32",
                        16, ("uniform", 1, 4096), seed=3)
LONG_BATCH = WorkloadSpec("llama8b_b32_l16k-32k_f16_spiky", 32, 32, 8, 128, "f16", "f16", "f16", 16,
                          ("uniform", 16384, 32768), seed=4, spike_frac=0.01,
                          max_pages_per_seq=2048)
MIXED_WINDOW = WorkloadSpec("llama8b_b64_window4096_mixed_bf16", 64, 32, 8, 128, "bf16", "bf16", "f32",
                            32, ("mixed", (1, 256), (32768, 65536)), seed=5, window=4096)

# Several new tokens per sequence: a suffix prefill of 128 tokens behind a
# cached prefix, and checking 4 drafted tokens on the batched long-context
# shape.
SUFFIX_PREFILL = WorkloadSpec("llama8b_b4_suffix128_l2k-8k_f16", 4, 32, 8, 128, "f16", "f16", "f16", 16,
                              ("uniform", 2048, 8192), seed=6, query_len=128)
VERIFY_LONG = WorkloadSpec("llama8b_b32_verify4_l16k-32k_f16", 32, 32, 8, 128, "f16", "f16", "f16", 16,
                           ("uniform", 16384, 32768), seed=7, query_len=4, max_pages_per_seq=2048)

NAMED = {"tiny": TINY, "llama8b_3060": LLAMA8B_3060, "wide_gqa": WIDE_GQA,
         "long_batch": LONG_BATCH, "mixed_window": MIXED_WINDOW,
         "suffix_prefill": SUFFIX_PREFILL, "verify_long": VERIFY_LONG}


@dataclasses.dataclass
class Workload:
    spec: WorkloadSpec
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    page_table: torch.Tensor     # int32 on the workload's device
    seq_lens: torch.Tensor       # int32 on the workload's device
    seq_lens_host: torch.Tensor  # int32 on the CPU (what the planner reads)
    scale: float                 # the float32 value the kernels use
    window: int
    num_pages: int               # pool pages, poison page included
    poison_page: int

    @property
    def page_size(self) -> int:
        return self.spec.page_size

    def attended(self) -> list:
        """(first key, end key) of the keys any query of each sequence
        attends (with T new tokens, from the first one's window start)."""
        return [(first_attended(L, self.spec.query_len, self.window), L) for L in self.seq_lens_host.tolist()]

    def kv_bytes(self) -> int:
        """Bytes of K and V that the method must read: each attended key row
        once per KV head (once per GQA group), K and V."""
        s = self.spec
        keys = sum(e - b for b, e in self.attended())
        return keys * s.num_kv_heads * s.head_dim * ELT_BYTES[s.kv_dtype] * 2


def first_attended(L: int, T: int, window: int) -> int:
    """First key any of the T newest tokens of a sequence of L keys attends."""
    return max(0, L - T + 1 - window) if window > 0 else 0


def draw_lengths(spec: WorkloadSpec, gen: torch.Generator) -> list:
    kind = spec.lengths[0]
    B = spec.batch
    if kind == "fixed":
        return [int(spec.lengths[1])] * B
    if kind == "list":
        lens = [int(x) for x in spec.lengths[1]]
        assert len(lens) == B
        return lens
    if kind == "uniform":
        lo, hi = spec.lengths[1], spec.lengths[2]
        return torch.randint(lo, hi + 1, (B,), generator=gen).tolist()
    if kind == "mixed":
        (lo1, hi1), (lo2, hi2) = spec.lengths[1], spec.lengths[2]
        n1 = B // 2
        a = torch.randint(lo1, hi1 + 1, (n1,), generator=gen)
        b = torch.randint(lo2, hi2 + 1, (B - n1,), generator=gen)
        order = torch.randperm(B, generator=gen)
        lens = torch.empty(B, dtype=torch.int64)
        lens[order[:n1]] = a
        lens[order[n1:]] = b
        return lens.tolist()
    raise ValueError(f"unknown length recipe {spec.lengths!r}")


def _value_generator(device: torch.device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + 17)
    return g


def make_workload(spec: WorkloadSpec, device="cpu", lengths: Optional[Sequence[int]] = None,
                  max_pages_per_seq: Optional[int] = None) -> Workload:
    """Draw one batch for ``spec`` on ``device``."""
    device = torch.device(device)
    B, Hq, Hkv, D, P = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size
    assert Hq % Hkv == 0
    cpu_gen = torch.Generator().manual_seed(spec.seed)
    lens = list(lengths) if lengths is not None else draw_lengths(spec, cpu_gen)
    T = spec.query_len
    assert len(lens) == B and all(L >= 0 for L in lens)
    assert T == 1 or all(L >= T for L in lens), "every sequence must hold its T new tokens"
    npages = [(L + P - 1) // P for L in lens]
    total = sum(npages)
    num_pages = total + 1
    poison = total
    if spec.shuffle:
        perm = torch.randperm(total, generator=cpu_gen)
    else:
        perm = torch.arange(total)
    maxp = max_pages_per_seq or spec.max_pages_per_seq or max(1, max(npages))
    assert maxp >= max(npages, default=0)
    table = torch.full((B, maxp), poison, dtype=torch.int32)
    offs = []
    off = 0
    for b in range(B):
        table[b, :npages[b]] = perm[off:off + npages[b]].to(torch.int32)
        offs.append(off)
        off += npages[b]

    window = int(spec.window)
    scale = float(torch.tensor(spec.scale if spec.scale is not None else 1.0 / math.sqrt(D),
                               dtype=torch.float32))
    kv_t = DTYPES[spec.kv_dtype]
    vg = _value_generator(device, spec.seed)
    q_shape = (B, Hq, D) if T == 1 else (B, T, Hq, D)
    q = torch.randn(q_shape, generator=vg, device=device, dtype=torch.float32).to(DTYPES[spec.q_dtype])

    pools = []
    table_dev = table.to(device)
    for which in ("k", "v"):
        pool = torch.full((num_pages, Hkv, P, D), float("nan"), dtype=kv_t, device=device)
        for b in range(B):
            L = lens[b]
            if L == 0:
                continue
            t0 = first_attended(L, T, window)
            p_first = t0 // P
            npw = npages[b] - p_first
            vals = torch.randn((npw, Hkv, P, D), generator=vg, device=device, dtype=torch.float32)
            if which == "k" and spec.spike_frac > 0:
                spikes = torch.rand((npw, Hkv, P), generator=vg, device=device) < spec.spike_frac
                vals = torch.where(spikes[..., None], vals * spec.spike_scale, vals)
            vals = vals.to(kv_t)
            tok = (torch.arange(npw, device=device)[:, None] + p_first) * P + torch.arange(P, device=device)[None, :]
            dead = (tok < t0) | (tok >= L)
            vals.masked_fill_(dead[:, None, :, None], float("nan"))
            phys = table_dev[b, p_first:npages[b]].long()
            pool[phys] = vals
        pools.append(pool)

    lens_host = torch.tensor(lens, dtype=torch.int32)
    return Workload(spec=spec, q=q, k_pool=pools[0], v_pool=pools[1], page_table=table_dev,
                    seq_lens=lens_host.to(device), seq_lens_host=lens_host, scale=scale,
                    window=window, num_pages=num_pages, poison_page=poison)


def to_numpy_inputs(w: Workload, rows: Optional[Sequence[int]] = None, attended_only: bool = False) -> dict:
    """Host copies of a workload (or of the sequences in ``rows``) as numpy
    arrays holding the stored values exactly (bf16 is widened to float32,
    which is exact). For a subset, only the pages those rows reference are
    copied and the page table is renumbered to the compact pool; the poison
    page is kept and unused entries point at it.

    ``attended_only``: copy only the pages that hold keys some query attends
    (from each sequence's first attended page on); table entries before
    them point at the poison page (NaN, like the pages they replace). Only
    a layout choice: the values of every attended key are the same."""
    if attended_only and rows is None:
        rows = range(w.spec.batch)
    import numpy as np

    def host(t: torch.Tensor) -> "np.ndarray":
        t = t.detach()
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.cpu().numpy()

    P = w.spec.page_size
    lens = w.seq_lens_host.tolist()
    if rows is None:
        return dict(q=host(w.q), k_pool=host(w.k_pool), v_pool=host(w.v_pool),
                    page_table=host(w.page_table).astype(np.int64), seq_lens=np.array(lens, dtype=np.int64),
                    page_size=P, scale=w.scale, window=w.window)
    rows = list(rows)
    table = w.page_table.cpu()
    T = w.spec.query_len

    def first_page(b):
        return first_attended(lens[b], T, w.window) // P if attended_only and lens[b] > 0 else 0

    used = []
    for b in rows:
        used.extend(table[b, first_page(b):(lens[b] + P - 1) // P].tolist())
    used.append(w.poison_page)
    idx = torch.tensor(used, dtype=torch.long, device=w.k_pool.device)
    remap = {p: i for i, p in enumerate(used)}
    poison_new = remap[w.poison_page]
    new_table = np.full((len(rows), table.shape[1]), poison_new, dtype=np.int64)
    for r, b in enumerate(rows):
        n = (lens[b] + P - 1) // P
        f = first_page(b)
        new_table[r, f:n] = [remap[p] for p in table[b, f:n].tolist()]
    return dict(q=host(w.q[torch.tensor(rows, device=w.q.device)]),
                k_pool=host(w.k_pool[idx]), v_pool=host(w.v_pool[idx]),
                page_table=new_table, seq_lens=np.array([lens[b] for b in rows], dtype=np.int64),
                page_size=P, scale=w.scale, window=w.window)


def make_new_rows(spec: WorkloadSpec, tokens: int, device="cpu", salt: int = 1):
    """K and V rows for ``tokens`` new tokens per sequence, [B][T][H_kv][D] in
    the KV dtype, N(0,1) drawn on ``device`` from a generator seeded by the
    spec's seed and ``salt``."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(spec.seed * 1_000_003 + 7919 * salt + 5)
    shape = (spec.batch, tokens, spec.num_kv_heads, spec.head_dim)
    kv_t = DTYPES[spec.kv_dtype]
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(kv_t)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(kv_t)
    return k, v

