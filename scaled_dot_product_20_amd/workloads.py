"""Seeded synthetic inputs shaped like the workloads the AOTriton pages time.

This module holds input generation only (random draws, sequence-length draws
and their prefix sums); it contains none of the attention arithmetic, and it
is the one module that both the GPU path's callers and the CPU oracle's
callers use.

Shapes come from the pages' own workloads: the BERT-family and gpt2 training
rows of the gfx950 table and the LTX diffusion rows of the gfx1100 forward
table (AOTriton 0.15b release notes, "gfx950, BERT-family and gpt2
Workloads" and "gfx1100, Forward"), plus a packed variable-length case with a
bottom-right numeric window ("Bottom-Right Aligned Sliding Windows").  The
pages time model shapes, not datasets: activations are i.i.d. N(0, 1).

Recipe: Q, K, V, dO are drawn in that order as float32 N(0, 1) from
``torch.Generator('cpu').manual_seed(seed)`` and then cast to the working
dtype with round-to-nearest-even (torch's ``.to``).  Packed sequence lengths
come from ``numpy.random.default_rng(seed)``: first every seqlen_q, then
every extra KV length, inclusive bounds.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

WINDOW_INF = 2147483647


def draw(shapes: Sequence[Sequence[int]], seed: int, dtype: torch.dtype) -> List[torch.Tensor]:
    """float32 N(0,1) draws in order, cast (RNE) to ``dtype``; CPU tensors."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    out = []
    for s in shapes:
        t = torch.randn(tuple(int(x) for x in s), generator=g, dtype=torch.float32)
        out.append(t.to(dtype))
    return out


def varlen_lengths(seed: int, n: int, q_lo: int, q_hi: int, extra_hi: int) -> Tuple[np.ndarray, np.ndarray]:
    """seqlen_q ~ U{q_lo..q_hi}, seqlen_k = seqlen_q + U{0..extra_hi}."""
    rng = np.random.default_rng(int(seed))
    sq = rng.integers(q_lo, q_hi + 1, size=n)
    extra = rng.integers(0, extra_hi + 1, size=n)
    return sq.astype(np.int64), (sq + extra).astype(np.int64)


def prefix(lengths: Sequence[int]) -> np.ndarray:
    """cu_seqlens: int32 [n+1], leading zero."""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    if out[-1] >= 2**31:
        raise ValueError("packed length overflows int32")
    return out.astype(np.int32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layout: str                 # "bhsd" or "thd"
    batch: int                  # bhsd: batch; thd: number of sequences
    heads: int
    head_dim: int
    seqlen_q: int               # bhsd: exact; thd: max over sequences
    seqlen_k: int
    dtypes: Tuple[torch.dtype, ...]
    window: Tuple[int, int] = (WINDOW_INF, WINDOW_INF)
    diag: str = "top_left"
    passes: Tuple[str, ...] = ("fwd", "bwd")
    seed: int = 1
    lens_q: Optional[Tuple[int, ...]] = None   # thd only
    lens_k: Optional[Tuple[int, ...]] = None

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def shapes(self):
        """(q_shape, k_shape): [B,H,S,D] or [T,H,D]."""
        if self.layout == "bhsd":
            return ((self.batch, self.heads, self.seqlen_q, self.head_dim),
                    (self.batch, self.heads, self.seqlen_k, self.head_dim))
        tq, tk = int(sum(self.lens_q)), int(sum(self.lens_k))
        return (tq, self.heads, self.head_dim), (tk, self.heads, self.head_dim)

    def cu_seqlens(self):
        if self.layout != "thd":
            return None, None
        return prefix(self.lens_q), prefix(self.lens_k)

    def inputs(self, dtype: torch.dtype, with_dout: bool = True):
        """(q, k, v[, dout]) CPU tensors for this workload."""
        qs, ks = self.shapes()
        shapes = [qs, ks, ks] + ([qs] if with_dout else [])
        return draw(shapes, self.seed, dtype)


def _varlen(name: str, head_dim: int) -> Workload:
    sq, sk = varlen_lengths(5, 24, 64, 2048, 1024)
    return Workload(name=name, layout="thd", batch=24, heads=16, head_dim=head_dim,
                    seqlen_q=int(sq.max()), seqlen_k=int(sk.max()),
                    dtypes=(torch.bfloat16,), window=(256, 0), diag="bottom_right",
                    seed=5, lens_q=tuple(int(x) for x in sq), lens_k=tuple(int(x) for x in sk))


def workloads() -> dict:
    """The tiny check, the pages' model shapes, and a long-sequence bwd cell at each built head dim."""
    ws = [
        Workload("tiny_f32", "bhsd", 1, 2, 64, 128, 128, (torch.float32,), seed=1),
        Workload("bert_like", "bhsd", 192, 16, 64, 512, 512, (torch.float16, torch.bfloat16), seed=2),
        Workload("gpt2_like_causal", "bhsd", 72, 12, 64, 1024, 1024, (torch.bfloat16,),
                 window=(WINDOW_INF, 0), seed=3),
        Workload("long_6630", "bhsd", 1, 32, 128, 6630, 6630, (torch.bfloat16,), passes=("fwd",), seed=4),
        Workload("long_15300", "bhsd", 1, 32, 128, 15300, 15300, (torch.bfloat16,), passes=("fwd",), seed=4),
        _varlen("varlen_window_d80", 80),
        _varlen("varlen_window_d128", 128),
        Workload("long_4096_bwd", "bhsd", 1, 32, 128, 4096, 4096, (torch.bfloat16,), seed=6),
        # The same cell at the other head dims the kernels are built for.
        Workload("long_4096_d32", "bhsd", 1, 32, 32, 4096, 4096, (torch.bfloat16,), seed=7),
        Workload("long_4096_d48", "bhsd", 1, 32, 48, 4096, 4096, (torch.bfloat16,), seed=8),
        Workload("long_4096_d96", "bhsd", 1, 32, 96, 4096, 4096, (torch.bfloat16,), seed=9),
    ]
    return {w.name: w for w in ws}
