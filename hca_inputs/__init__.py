"""Seeded synthetic inputs for HCA attention.

This module is shared by the tests, the benchmark and the smoke check.  It
draws random tensors and document lengths and nothing else: it holds none of
the method's arithmetic (no masking rule, no attention), so the oracle and the
HIP path receive identical inputs without sharing any of the computation.

Workloads (the five standard problem sizes; every one is synthetic, with the
shapes, value distributions and document structure the method's pages and the
problem statement give):

  tiny_fp32    B=1 S=489 H=4  D=64  r=16  Sc=30   W=64  fp32, one document
  packed_bf16  B=2 S=4096 H=16 D=128 r=128 Sc=32  W=128 bf16, documents with
               lengths uniform on the integers 256..2048
  mid_bf16     B=1 S=16384 H=64 D=512 r=128 Sc=128 W=128 bf16, one document,
               q / kv / kv_comp scaled by 0.5
  long_bf16    B=1 S=65536 H=64 D=512 r=128 Sc=512 W=128 bf16, one document
  max_bf16     B=1 S=131063 H=64 D=512 r=128 Sc=1023 W=128 bf16, documents
               with lengths log-uniform on [1024, 65536)

Draw recipe: a torch generator seeded with the workload number draws q, kv,
kv_comp and dout, in that order, as float32 N(0, 1) (times the workload's value
scale for q / kv / kv_comp), then rounds to the workload dtype
(round-to-nearest-even for bf16).  Document lengths come from
numpy.random.default_rng(seed): per batch row, lengths are drawn until they
cover S, and the last one is cut at S.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    H: int
    D: int
    r: int
    Sc: int
    W: int
    dtype: str  # "f32" or "bf16"
    docs: Optional[str] = None  # None, "uniform", "loguniform"
    doc_lo: int = 0
    doc_hi: int = 0
    value_scale: float = 1.0
    seed: int = 0


WORKLOADS = {
    1: Workload("tiny_fp32", 1, 489, 4, 64, 16, 30, 64, "f32", seed=1),
    2: Workload("packed_bf16", 2, 4096, 16, 128, 128, 32, 128, "bf16", docs="uniform",
                doc_lo=256, doc_hi=2048, seed=2),
    3: Workload("mid_bf16", 1, 16384, 64, 512, 128, 128, 128, "bf16", value_scale=0.5,
                seed=3),
    4: Workload("long_bf16", 1, 65536, 64, 512, 128, 512, 128, "bf16", seed=4),
    5: Workload("max_bf16", 1, 131063, 64, 512, 128, 1023, 128, "bf16", docs="loguniform",
                doc_lo=1024, doc_hi=65536, seed=5),
}


# The CSA form of the compressed path (compress ratio 4, a top-k selection of
# compressed entries per query, shared by its heads), at the mid-length shape.
# The pages give the ratio but not k; 512 entries per query is used.  The
# selection is drawn here (seeded), not computed by an indexer.
CSA_TOPK = Workload("csa_topk_bf16", 1, 16384, 64, 512, 4, 4096, 128, "bf16", seed=6)
CSA_TOPK_K = 512


def topk_indices(wl: Workload, K: int) -> np.ndarray:
    """Per-query selections [B, S, K] int32 for the top-k workload: query i picks
    min(K, n_i) distinct entries uniformly among the n_i = (i + 1) // r entries
    whose windows end at or before it (-1 fills the rest), from
    numpy.random.default_rng(seed)."""
    rng = np.random.default_rng(wl.seed)
    out = np.full((wl.B, wl.S, K), -1, np.int32)
    for b in range(wl.B):
        for i0 in range(0, wl.S, 1024):
            i1 = min(wl.S, i0 + 1024)
            done = (np.arange(i0, i1) + 1) // wl.r
            key = rng.random((i1 - i0, wl.Sc))
            key[np.arange(wl.Sc)[None, :] >= done[:, None]] = np.inf
            pick = np.argpartition(key, min(K, wl.Sc) - 1, axis=1)[:, :K].astype(np.int32)
            pick[np.take_along_axis(key, pick, 1) == np.inf] = -1
            out[b, i0:i1, :pick.shape[1]] = pick
    return out


def doc_lengths(wl: Workload) -> Optional[List[List[int]]]:
    """Per batch row, the list of document lengths (None: one document)."""
    if wl.docs is None:
        return None
    rng = np.random.default_rng(wl.seed)
    out = []
    for _ in range(wl.B):
        lens, total = [], 0
        while total < wl.S:
            if wl.docs == "uniform":
                L = int(rng.integers(wl.doc_lo, wl.doc_hi + 1))
            else:
                L = int(math.floor(math.exp(rng.uniform(math.log(wl.doc_lo),
                                                        math.log(wl.doc_hi)))))
            L = min(L, wl.S - total)
            lens.append(L)
            total += L
        out.append(lens)
    return out


def starts_csr(lengths: Optional[List[List[int]]], B: int):
    """Document start positions, concatenated over the batch, plus per-row counts."""
    if lengths is None:
        return None, None
    starts, counts = [], []
    for lens in lengths:
        pos = 0
        for L in lens:
            starts.append(pos)
            pos += L
        counts.append(len(lens))
    assert len(counts) == B
    return np.asarray(starts, dtype=np.int32), np.asarray(counts, dtype=np.int32)


def segment_ids(lengths: Optional[List[List[int]]], B: int, S: int) -> np.ndarray:
    """Per-token document index [B, S] int32."""
    seg = np.zeros((B, S), dtype=np.int32)
    if lengths is None:
        return seg
    for b, lens in enumerate(lengths):
        pos = 0
        for j, L in enumerate(lens):
            seg[b, pos:pos + L] = j
            pos += L
        assert pos == S
    return seg


def draw(B, S, H, D, Sc, dtype="bf16", seed=0, value_scale=1.0, device="cpu", kv_heads=1):
    """Draws q [B,H,S,D], kv [B,S,D], kv_comp [B,Sc,D], dout [B,H,S,D] (torch); with
    kv_heads = G > 1, kv [B,G,S,D] and kv_comp [B,G,Sc,D]."""
    import torch

    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def one(shape, scale):
        t = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
        if scale != 1.0:
            t.mul_(scale)
        return t.to(tdt)

    q = one((B, H, S, D), value_scale)
    g = () if kv_heads == 1 else (kv_heads,)
    kv = one((B,) + g + (S, D), value_scale)
    kvc = one((B,) + g + (Sc, D), value_scale)
    dout = one((B, H, S, D), 1.0)
    return q, kv, kvc, dout


def draw_workload(wl: Workload, device="cpu"):
    return draw(wl.B, wl.S, wl.H, wl.D, wl.Sc, wl.dtype, wl.seed, wl.value_scale, device)


def random_lengths(rng: np.random.Generator, S: int, lo: int, hi: int) -> List[int]:
    """Lengths drawn uniformly from lo..hi until they cover S (last one cut)."""
    lens, total = [], 0
    while total < S:
        L = min(int(rng.integers(lo, hi + 1)), S - total)
        lens.append(L)
        total += L
    return lens


def to_host_bits(t):
    """Host numpy view of a torch tensor for the oracle: float32, or bf16 bits as uint16."""
    import torch

    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.to(torch.float32).numpy()
