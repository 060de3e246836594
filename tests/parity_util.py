"""Shared helpers of the GPU parity tests: seeded inputs, the HIP path through
the C ABI, the oracle on the same inputs, and the max-abs comparison at the
tolerances the attention path is held to (O and LSE: fp32 1e-5, fp16 5e-3,
bf16 2e-2; dQ/dK/dV twice those)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import oracle as orc
from scaled_dot_product_20_amd import binding as bd
from scaled_dot_product_20_amd import workloads as wl

INF = wl.WINDOW_INF
TOL = {torch.float32: 1e-5, torch.float16: 5e-3, torch.bfloat16: 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# Significand bits (with the implicit one) of each output type.
_SIG_BITS = {torch.float32: 24, torch.float16: 11, torch.bfloat16: 8}


def ulp(x, dtype):
    """Spacing of `dtype` values at |x| (normal range; a value of 0 gives the
    spacing at the smallest normal, far below any bound used here)."""
    _, e = np.frexp(np.maximum(np.abs(x), np.finfo(np.float32).tiny))  # |x| = m * 2^e, m in [0.5, 1)
    return np.ldexp(1.0, e - _SIG_BITS[dtype])


def half_ulp_bound(got, ref, tol, dtype):
    """Per-element bound on |got - ref|: tol, plus half the output type's
    spacing wherever that spacing exceeds tol.  A result computed within tol
    of ref and then rounded to the output type lies within tol + 1/2 ulp of
    ref; below that spacing the absolute bound alone decides.  The spacing is
    taken at the larger of |got| and |ref|, so a value rounded across a power
    of two is held to the coarser side's spacing."""
    if dtype not in _SIG_BITS:
        return np.full(np.shape(ref), tol, dtype=np.float64)
    u = ulp(np.maximum(np.abs(got), np.abs(ref)), dtype)
    return np.where(u > tol, tol + 0.5 * u, tol)


# Elements (per comparison name) that exceeded the absolute bound and were
# admitted only by the output type's half ulp; printed by every comparison
# and summed here for a test run.
HALF_ULP_ADMITTED = {}


def max_err(name, got, ref, tol, inf_exact=False):
    """Max |got - ref| over all elements; +inf in ref must be matched
    exactly, and any NaN fails.  Each element is held to half_ulp_bound:
    where the output type's spacing exceeds the absolute bound (bf16 values
    of magnitude 8 and up against the 4e-2 gradient bound, e.g. dV of one key
    summed over a hundred queries) the bound is the output's own rounding
    plus tol.  The elements admitted only by that half ulp are counted and
    printed."""
    dtype = got.dtype if isinstance(got, torch.Tensor) else torch.float64
    g = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert not np.isnan(g).any(), f"{name}: NaN in GPU output"
    if inf_exact:
        inf = np.isinf(r)
        assert np.array_equal(g[inf], r[inf]), f"{name}: +inf rows differ"
        assert np.isfinite(g[~inf]).all(), f"{name}: unexpected inf"
        g, r = g[~inf], r[~inf]
    d = np.abs(g - r)
    err = float(d.max()) if g.size else 0.0
    bound = half_ulp_bound(g, r, tol, dtype)
    if g.size and not np.all(d <= bound):
        i = int(np.argmax(d - bound))
        raise AssertionError(f"{name}: abs err {d.flat[i]:.3e} > {bound.flat[i]:.3e} at ref {r.flat[i]:.4g} "
                             f"(max abs err {err:.3e}, tol {tol:.1e})")
    admitted = int(np.count_nonzero(d > tol))
    if admitted:
        HALF_ULP_ADMITTED[name] = HALF_ULP_ADMITTED.get(name, 0) + admitted
        say(f"  {name}: {admitted} of {g.size} elements beyond {tol:.1e}, within tol + 1/2 ulp of the output type")
    return err


class Case:
    """A small problem run end to end on the GPU and on the oracle."""

    def __init__(self, *, layout="bhsd", B=1, H=2, Sq=64, Sk=None, D=64, dtype=torch.bfloat16,
                 window=(INF, INF), diag="top_left", scale=None, seed=0, lens_q=None, lens_k=None,
                 bshd=False, split=True):
        self.layout, self.B, self.H, self.D, self.dtype = layout, B, H, D, dtype
        self.Sq, self.Sk = Sq, (Sq if Sk is None else Sk)
        self.window, self.diag = window, diag
        self.scale = 1.0 / math.sqrt(D) if scale is None else scale
        self.seed, self.bshd, self.split = seed, bshd, split
        if layout == "thd":
            self.lens_q, self.lens_k = list(lens_q), list(lens_k)
            self.cu_q, self.cu_k = wl.prefix(self.lens_q), wl.prefix(self.lens_k)
            tq, tk = int(self.cu_q[-1]), int(self.cu_k[-1])
            shapes = [(tq, H, D), (tk, H, D), (tk, H, D), (tq, H, D)]
        elif bshd:  # drawn as [B, S, H, D] and viewed as [B, H, S, D]
            shapes = [(B, self.Sq, H, D), (B, self.Sk, H, D), (B, self.Sk, H, D), (B, self.Sq, H, D)]
        else:
            shapes = [(B, H, self.Sq, D), (B, H, self.Sk, D), (B, H, self.Sk, D), (B, H, self.Sq, D)]
        q, k, v, do = wl.draw(shapes, seed, dtype)
        if bshd:
            q, k, v, do = (t.permute(0, 2, 1, 3) for t in (q, k, v, do))
        self.cpu = (q, k, v, do)

    def tol_factor(self):
        """Factor on the bounds of LSE and the gradients (and of O in fp32):
        1 at the configs' scale 1/sqrt(D).  Off that scale the logits grow
        with |scale| * sqrt(D) (the logit standard deviation for N(0,1)
        inputs), and with them the absolute error of LSE (a logit plus a
        log), of dS = P (dP - Delta) times scale in dQ and dK, and of the
        fp32-rounded exponents c * s, whose relative error carries into every
        P.  That last error is what bounds O in fp32; in fp16 / bf16 the
        rounding of P to the 16-bit type (a relative 2^-11 / 2^-8, whatever
        the logits) dominates, and O's bound there stays unscaled."""
        return max(1.0, abs(self.scale) * math.sqrt(self.D))

    def o_tol(self):
        base = TOL[self.dtype]
        return base * self.tol_factor() if self.dtype == torch.float32 else base

    def kw_oracle(self):
        kw = dict(scale=self.scale, window=self.window, diag=self.diag)
        if self.layout == "thd":
            kw.update(cu_seqlens_q=self.cu_q, cu_seqlens_k=self.cu_k)
        return kw

    def kw_gpu(self, dev):
        kw = dict(scale=self.scale, window=self.window, diag=self.diag, split=self.split)
        if self.layout == "thd":
            kw.update(cu_seqlens_q=torch.from_numpy(self.cu_q).to(dev),
                      cu_seqlens_k=torch.from_numpy(self.cu_k).to(dev),
                      max_seqlen_q=max(self.lens_q + [0]), max_seqlen_k=max(self.lens_k + [0]))
        return kw

    def gpu(self, dev="cuda", bwd=True):
        q, k, v, do = (t.to(dev) for t in self.cpu)  # strides kept (bshd views stay views)
        if self.bshd:
            q, k, v, do = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v, do))
        kw = self.kw_gpu(dev)
        o, lse = bd.attn_fwd(q, k, v, **kw)
        out = {"o": o, "lse": lse}
        if bwd:
            dq, dk, dv = bd.attn_bwd(do, q, k, v, o, lse, **kw)
            out.update(dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        return out

    def oracle(self, bwd=True):
        q, k, v, do = (t.contiguous() for t in self.cpu)
        if bwd:
            o, lse, dq, dk, dv = orc.bwd(q, k, v, do, **self.kw_oracle())
            return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
        o, lse = orc.fwd(q, k, v, **self.kw_oracle())
        return {"o": o, "lse": lse}

    def check(self, bwd=True, dev="cuda"):
        say(f"case layout={self.layout} B={self.B} H={self.H} Sq={self.Sq} Sk={self.Sk} D={self.D} "
            f"dtype={self.dtype} window={self.window} diag={self.diag} scale={self.scale} seed={self.seed} "
            f"split={self.split}")
        got = self.gpu(dev, bwd)
        ref = self.oracle(bwd)
        base = TOL[self.dtype]
        tol = base * self.tol_factor()
        errs = {"o": max_err("O", got["o"], ref["o"], self.o_tol()),
                "lse": max_err("LSE", got["lse"], ref["lse"], tol, inf_exact=True)}
        if bwd:
            for n in ("dq", "dk", "dv"):
                errs[n] = max_err(n, got[n], ref[n], 2 * tol)
        say("  errs", {k: f"{v:.2e}" for k, v in errs.items()})
        return got, ref, errs
