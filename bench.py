#!/usr/bin/env python3
"""Throughput of the fused attention forward + backward on one MI355X.

One step = the whole path over one batch of synthetic input: attn_fwd (O,
LSE), then the backward's two calls (attn_bwd_preprocess for Delta, then
attn_bwd_dkdv_dq for dK, dV and dQ), all through the C ABI on torch's
current stream.  Inputs are resident in HBM before the timed region starts;
K steps are timed between a synchronize on each side, and every call is also
bracketed by HIP events on the launch stream so its own average duration is
known.

FLOPs are counted on visible (query, key) pairs only: forward 4*D per pair
(Q K^T and P V), backward 10*D per pair (S recomputed once, dV, dP, dK, dQ).
The roofline object reports the call with the largest time share against
that algorithmic work and the bf16/fp16 dense MFMA peak of 2516.6 TFLOP/s
(256 CUs x 2.4 GHz x 4096 FLOP/clk/CU); the backward call's executed work
(S and dP are computed both for dK/dV and for dQ: 14*D per pair) is reported
beside it as executed_tflops.  The kernels each call launches are the
library's own plan (attn_fwd_plan / attn_bwd_plan).

Algorithmic HBM bytes: forward reads Q and the K/V rows some query sees and
writes O and the fp32 LSE; backward reads Q, K, V, O, dO and LSE, writes dQ,
dK and dV, and writes and reads the fp32 Delta.

Besides the headline workload, the line carries `cells`: every workload of
the pages' shapes, each pass timed as a run of back-to-back calls (the
backward's two calls together) between two events, behind a short spin
kernel that lets the host enqueue the run first.  For calls of tens of
microseconds this keeps per-call events (a few microseconds of device time
each) and the host's launch rate out of the numbers; for the rest it equals
the per-call timing.

The CPU baseline is the fp64 oracle timed on this host on (sequence, head)
slices of the headline workload, scaled to the same unit.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd/bwd TFLOP/s (unmasked FLOPs) + % bf16 MFMA peak, hdim 128"
PEAK_MFMA_16 = 2516.6   # TFLOP/s, bf16 and fp16 dense
PEAK_MFMA_32 = 157.3    # TFLOP/s, fp32
PEAK_HBM = 8000.0       # GB/s
WINDOW_INF = 2147483647  # unbounded window side
DEFAULT_WORKLOAD = "long_6630"
# The timed cells besides the headline: every workload of the pages' shapes
# (tiny fp32, BERT-like in fp16 and bf16, gpt2-like causal, both long
# sequences, packed windowed at head_dim 80 and 128, the 4096-row cell).
CELLS = [("tiny_f32", "fp32"), ("bert_like", "fp16"), ("bert_like", "bf16"), ("gpt2_like_causal", "bf16"),
         ("long_6630", "bf16"), ("long_15300", "bf16"), ("varlen_window_d80", "bf16"),
         ("varlen_window_d128", "bf16"), ("long_4096_bwd", "bf16")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dkdv_traffic_long_6630.txt")
KERNEL_SOURCES = ["scaled_dot_product_20_amd/csrc/attn_bwd_kernels.hpp",
                  "scaled_dot_product_20_amd/csrc/attn_device.hpp",
                  "scaled_dot_product_20_amd/csrc/attn_launch.hpp"]
ENTRY = {"fwd": "attn_fwd", "bwd_preprocess": "attn_bwd_preprocess", "bwd_dkdv_dq": "attn_bwd_dkdv_dq"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def row_ranges(sq: int, sk: int, window, diag: str):
    """Per query row i, the visible keys [lo_i, hi_i] of one sequence (empty
    when hi < lo): key j is visible to query i iff i - L <= j <= i + R, (L, R)
    shifted by d = sk - sq under the bottom-right diagonal when both sides
    are finite."""
    import numpy as np
    inf = 2147483647
    wl, wr = window
    L, R = wl, wr
    if diag == "bottom_right" and wl != inf and wr != inf:
        L, R = wl - (sk - sq), wr + (sk - sq)
    i = np.arange(sq, dtype=np.int64)
    lo = np.zeros(sq, np.int64) if L == inf else np.maximum(0, i - L)
    hi = np.full(sq, sk - 1, np.int64) if R == inf else np.minimum(sk - 1, i + R)
    return lo, hi


def visible_pairs(sq: int, sk: int, window, diag: str) -> int:
    import numpy as np
    lo, hi = row_ranges(sq, sk, window, diag)
    return int(np.maximum(0, hi - lo + 1).sum())


def visible_keys(sq: int, sk: int, window, diag: str) -> int:
    """Keys of one sequence that at least one query sees."""
    import numpy as np
    lo, hi = row_ranges(sq, sk, window, diag)
    ok = hi >= lo
    cover = np.zeros(sk + 1, np.int64)
    np.add.at(cover, lo[ok], 1)
    np.add.at(cover, hi[ok] + 1, -1)
    return int((np.cumsum(cover[:sk]) > 0).sum())


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the backward call from the committed counter
    summary, or None when there is none for this workload and kernel or the
    kernel's sources changed since."""
    if workload != DEFAULT_WORKLOAD or not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_hash() or vals.get("kernel") != kernel:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w, dtype, min_seconds=10.0, max_slices=32):
    """The fp64 oracle timed on (sequence, head) slices of the workload's
    shape, slice after slice until at least `min_seconds` have run; TFLOP/s
    on the same visible-pair count as the GPU figure.  Slice s is drawn with
    seed 1000 * workload seed + s (same shape and distribution)."""
    from oracle import oracle as orc
    from scaled_dot_product_20_amd import workloads as wls

    if w.layout == "thd":
        sq, sk = int(w.lens_q[0]), int(w.lens_k[0])
        cu_q, cu_k = wls.prefix([sq]), wls.prefix([sk])
        shapes = [(sq, 1, w.head_dim), (sk, 1, w.head_dim), (sk, 1, w.head_dim), (sq, 1, w.head_dim)]
        kw = dict(cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
        what = f"sequence 0 (Sq={sq}, Sk={sk}) of {w.name}, one head per slice"
    else:
        sq, sk = w.seqlen_q, w.seqlen_k
        shapes = [(1, 1, sq, w.head_dim), (1, 1, sk, w.head_dim), (1, 1, sk, w.head_dim),
                  (1, 1, sq, w.head_dim)]
        kw = {}
        what = f"one (batch, head) slice {sq}x{sk}x{w.head_dim} of {w.name} per slice"
    pairs = visible_pairs(sq, sk, w.window, w.diag)
    flop_slice = (4 + (10 if "bwd" in w.passes else 0)) * w.head_dim * pairs
    spent, n = 0.0, 0
    while n < max_slices and spent < min_seconds:
        q, k, v, do = wls.draw(shapes, 1000 * w.seed + n, dtype)
        t0 = time.perf_counter()
        if "bwd" in w.passes:
            orc.bwd(q, k, v, do, scale=w.scale, window=w.window, diag=w.diag, **kw)
        else:
            orc.fwd(q, k, v, scale=w.scale, window=w.window, diag=w.diag, **kw)
        spent += time.perf_counter() - t0
        n += 1
    return {"value": round(n * flop_slice / spent / 1e12, 6), "unit": "TFLOP/s",
            "cores": orc.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"fp64 {'+'.join(w.passes)} of {n} slices: {what}; {spent:.1f} s",
            "seconds": round(spent, 2)}


def copy_probe(mib: int, steps: int) -> None:
    """A plain copy of `mib` MiB between two device buffers, `steps` times:
    each launch reads and writes exactly mib MiB, so what an HBM byte
    counter reports per launch, divided by that, is the counter's scale."""
    import torch
    n = mib * 2**20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_probe_bytes": n, "launches": steps, "ms": round(dt * 1e3, 4),
                      "gb_s_read_plus_write": round(2 * n / dt / 1e9, 1)}), flush=True)


def mfma_probe(n: int, steps: int) -> None:
    """A plain bf16 GEMM (torch.matmul, n x n x n), `steps` times: a matrix-
    core-bound library kernel whose FLOP rate is known from its time, the
    reference against which an MFMA-busy counter's reading is scaled."""
    import torch
    g = torch.Generator(device="cuda:0").manual_seed(0)
    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    c = torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        c = torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    print(json.dumps({"mfma_probe_n": n, "launches": steps + 1, "ms": round(ms, 4), "tflops": round(tf, 1),
                      "frac_of_bf16_peak": round(tf / PEAK_MFMA_16, 4)}), flush=True)


# Small problems the backward's split mode is for: (dtype, B, H, S, D), no
# mask, scale 1/sqrt(D).
SPLIT_SHAPES = [("fp32", 1, 2, 128, 64), ("fp32", 1, 4, 512, 64), ("fp16", 2, 3, 300, 80),
                ("bf16", 1, 2, 512, 64), ("bf16", 1, 8, 512, 64), ("bf16", 1, 1, 256, 128),
                ("bf16", 1, 2, 1000, 128), ("bf16", 1, 4, 1000, 128), ("bf16", 1, 1, 4000, 64),
                ("bf16", 1, 8, 2048, 128), ("bf16", 4, 8, 1024, 128)]


def split_probe(steps: int) -> None:
    """The forward (attn_fwd) and the backward (attn_bwd: preprocess, then
    dK/dV and dQ) of each small shape with the library's choice and with
    its split paths off (ATTN_FLAG_NO_SPLIT): microseconds per call over
    `steps` back-to-back calls between two HIP events, behind a spin kernel
    that lets the host enqueue them all first.  One JSON line per shape."""
    import torch
    from scaled_dot_product_20_amd import binding as bd
    names = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
    sid = torch.cuda.current_stream().cuda_stream

    def per_call(entry, p):
        for _ in range(5):
            bd.launch(entry, p, sid)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(spin_cycles(0.1 * steps))
        e0.record()
        for _ in range(steps):
            bd.launch(entry, p, sid)
        e1.record()
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) * 1e3 / steps, 1)

    fkw = dict(window=(WINDOW_INF, WINDOW_INF), diag="top_left", cu_seqlens_q=None, cu_seqlens_k=None,
               max_seqlen_q=None, max_seqlen_k=None)
    for dn, B, H, S, D in SPLIT_SHAPES:
        g = torch.Generator(device="cuda:0").manual_seed(S * D + H)
        q, k, v, do = (torch.randn(B, H, S, D, device="cuda:0", dtype=names[dn], generator=g) for _ in range(4))
        o, lse = bd.attn_fwd(q, k, v, scale=D ** -0.5)
        res = {}
        for split in (True, False):
            key = "split" if split else "unsplit"
            fp, fws = bd.prepare_fwd(q, k, v, torch.empty_like(o), torch.empty_like(lse), scale=D ** -0.5,
                                     split=split, **fkw)
            bp, keep = bd.prepare_bwd(do, q, k, v, o, lse, scale=D ** -0.5, split=split)
            res[key] = {"fwd_us": per_call("attn_fwd", fp), "fwd_kernels": [n for n, _, _ in bd.plan("attn_fwd", fp)],
                        "bwd_us": per_call("attn_bwd", bp), "bwd_kernels": [n for n, _, _ in bd.plan("attn_bwd", bp)]}
        print(json.dumps({"shape": f"{B}x{H}x{S}x{D}", "dtype": dn, **res}), flush=True)


_SPIN = {}


def spin_cycles(ms):
    """Cycles of torch.cuda._sleep that last about ms milliseconds on this
    device (calibrated once with HIP events)."""
    import torch
    if "per_ms" not in _SPIN:
        n = 1 << 20
        torch.cuda._sleep(n)  # first call loads the kernel
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(n)
        e1.record()
        torch.cuda.synchronize()
        _SPIN["per_ms"] = n / max(e0.elapsed_time(e1), 1e-3)
    return int(_SPIN["per_ms"] * ms) + 1


class Run:
    """One workload on the GPU: inputs in HBM, the params of each call, the
    library's launch plan, and timed steps."""

    def __init__(self, W, dtype, passes, dev):
        import torch
        from scaled_dot_product_20_amd import binding as bd

        self.W, self.dtype, self.passes, self.dev = W, dtype, passes, dev
        self.dname = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[dtype]
        q, k, v, do = (t.to(dev) for t in W.inputs(dtype))
        kw = dict(scale=W.scale, window=W.window, diag=W.diag)
        if W.layout == "thd":
            cu_q, cu_k = W.cu_seqlens()
            kw.update(cu_seqlens_q=torch.from_numpy(cu_q).to(dev), cu_seqlens_k=torch.from_numpy(cu_k).to(dev),
                      max_seqlen_q=W.seqlen_q, max_seqlen_k=W.seqlen_k)
            lens = list(zip(W.lens_q, W.lens_k))
        else:
            lens = [(W.seqlen_q, W.seqlen_k)] * W.batch
        self.pairs = W.heads * sum(visible_pairs(a, b, W.window, W.diag) for a, b in lens)
        kvis = W.heads * sum(visible_keys(a, b, W.window, W.diag) for a, b in lens)
        tq, tk = W.heads * sum(a for a, _ in lens), W.heads * sum(b for _, b in lens)
        esz, D = q.element_size(), W.head_dim
        self.fwd_bytes = esz * D * (2 * tq + 2 * kvis) + 4 * tq
        self.bwd_bytes = esz * D * (4 * tq + 4 * tk) + 4 * 3 * tq
        o, lse = bd.attn_fwd(q, k, v, **kw)
        fkw = dict(cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None)
        fkw.update(kw)
        fp, fws = bd.prepare_fwd(q, k, v, o, lse, **fkw)
        self.params = {"fwd": fp}
        self.calls = ["fwd"]
        self.keep = (q, k, v, do, o, lse, kw, fws)
        if "bwd" in passes:
            bp, self.bkeep = bd.prepare_bwd(do, q, k, v, o, lse, **kw)
            self.params["bwd_preprocess"] = self.params["bwd_dkdv_dq"] = bp
            self.calls += ["bwd_preprocess", "bwd_dkdv_dq"]
        self.stream = torch.cuda.current_stream(dev)
        self.plan = {c: bd.plan(ENTRY[c], self.params[c], self.stream.cuda_stream) for c in self.calls}

    def step(self, evs=None):
        from scaled_dot_product_20_amd import binding as bd
        sid = self.stream.cuda_stream
        for i, c in enumerate(self.calls):
            if evs is not None:
                evs[i].record(self.stream)
            bd.launch(ENTRY[c], self.params[c], sid)
        if evs is not None:
            evs[len(self.calls)].record(self.stream)

    def time(self, steps, warmup):
        """(wall ms per step, {call: average ms from HIP events on the launch stream})."""
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(self.calls) + 1)]
                  for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            self.step(events[s])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = {c: sum(ev[i].elapsed_time(ev[i + 1]) for ev in events) / steps for i, c in enumerate(self.calls)}
        return wall * 1e3 / steps, per

    def time_runs(self, steps, warmup):
        """{"fwd": ms, "bwd": ms}: each pass as a run of `steps` back-to-back
        calls (the backward: preprocess, then dK/dV + dQ) between two HIP
        events, behind a short spin kernel that lets the host enqueue the
        whole run before the device reaches it.  For calls of tens of
        microseconds an event between two launches, or a host slower than
        the device, would otherwise show up in the time."""
        import torch
        from scaled_dot_product_20_amd import binding as bd
        sid = self.stream.cuda_stream
        runs = [("fwd", ["fwd"])] + ([("bwd", ["bwd_preprocess", "bwd_dkdv_dq"])] if "bwd_dkdv_dq" in self.calls else [])
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        per = {}
        for name, calls in runs:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(spin_cycles(0.25 * steps))
            e0.record(self.stream)
            for _ in range(steps):
                for c in calls:
                    bd.launch(ENTRY[c], self.params[c], sid)
            e1.record(self.stream)
            torch.cuda.synchronize()
            per[name] = e0.elapsed_time(e1) / steps
        return per

    def kernels(self, call):
        return "+".join(name for name, _, _ in self.plan[call])

    def summary(self, per, peak):
        D = self.W.head_dim
        fwd_flop, bwd_flop = 4.0 * D * self.pairs, 10.0 * D * self.pairs
        out = {"fwd": {"ms": round(per["fwd"], 4), "tflops": round(fwd_flop / per["fwd"] / 1e9, 2),
                       "frac_of_peak": round(fwd_flop / per["fwd"] / 1e9 / peak, 4),
                       "gb_s": round(self.fwd_bytes / per["fwd"] / 1e6, 1),
                       "kernels": self.kernels("fwd")}}
        if "bwd_dkdv_dq" in per or "bwd" in per:
            ms = per["bwd"] if "bwd" in per else per["bwd_preprocess"] + per["bwd_dkdv_dq"]
            out["bwd"] = {"ms": round(ms, 4), "tflops": round(bwd_flop / ms / 1e9, 2),
                          "frac_of_peak": round(bwd_flop / ms / 1e9 / peak, 4),
                          "gb_s": round(self.bwd_bytes / ms / 1e6, 1),
                          "kernels": self.kernels("bwd_preprocess") + "," + self.kernels("bwd_dkdv_dq")}
        return out

    def release(self):
        import torch
        self.keep = self.bkeep = self.params = None
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--dtype", default=None, help="bf16 / fp16 / fp32 (default: the workload's first)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-cells", action="store_true", help="time the headline workload only")
    ap.add_argument("--cell-steps", type=int, default=10)
    ap.add_argument("--cell-warmup", type=int, default=3)
    ap.add_argument("--passes", default=None, help="fwd or fwd,bwd (default: fwd,bwd)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the attention step, run a plain device-to-device copy of MIB "
                         "MiB (the calibration kernel for HBM byte counters) and exit")
    ap.add_argument("--mfma-probe", type=int, default=0, metavar="N",
                    help="instead of the attention step, run an N x N x N bf16 GEMM (the reference for "
                         "MFMA-busy counters) and exit")
    ap.add_argument("--split-probe", action="store_true",
                    help="time the backward of small shapes with and without its split mode (JSON lines)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the attention kernels shard by head and batch with no "
              "communication, and this build runs on a single MI355X; --gpus must be 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from scaled_dot_product_20_amd import workloads as wls

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return
    if args.mfma_probe:
        mfma_probe(args.mfma_probe, args.steps)
        return
    if args.split_probe:
        split_probe(args.steps)
        return
    names = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
    wl_all = wls.workloads()
    W = wl_all[args.workload]
    dtype = names[args.dtype] if args.dtype else W.dtypes[0]
    passes = tuple(args.passes.split(",")) if args.passes else ("fwd", "bwd")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    peak_of = lambda dt: PEAK_MFMA_32 if dt == torch.float32 else PEAK_MFMA_16

    log(f"[bench] workload {W.name} dtype {dtype} passes {passes}: drawing inputs")
    run = Run(W, dtype, passes, dev)
    log(f"[bench] plan {json.dumps(run.plan)}")
    log(f"[bench] warmup {args.warmup} steps, timing {args.steps} steps")
    ms_step, per = run.time(args.steps, args.warmup)
    log("[bench] per-call ms " + json.dumps({k: round(v, 4) for k, v in per.items()}))

    peak = peak_of(dtype)
    D = W.head_dim
    fwd_flop = 4.0 * D * run.pairs
    bwd_flop = 10.0 * D * run.pairs
    total_flop = fwd_flop + (bwd_flop if "bwd" in passes else 0.0)
    value = total_flop / (ms_step * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": run.dname,
        "data": "synthetic: i.i.d. N(0,1) Q/K/V/dO from a seeded generator, cast RNE",
        "config": {"workload": W.name, "layout": W.layout, "batch": W.batch, "heads": W.heads,
                   "head_dim": D, "seqlen_q": W.seqlen_q, "seqlen_k": W.seqlen_k,
                   "window": list(W.window), "diag": W.diag, "passes": list(passes),
                   "visible_pairs": run.pairs},
        "frac_of_peak": round(value / peak, 4),
    }
    out.update(run.summary(per, peak))
    # Roofline of the call with the largest time share, priced at its
    # algorithmic work; the backward call's executed work beside it.
    dom = max(per, key=per.get)
    kname = run.kernels(dom)
    if dom == "bwd_dkdv_dq":
        ach = bwd_flop / per[dom] / 1e9
        algo = f"10*D FLOP per visible pair (S, dV, dP, dK, dQ) x {run.pairs} pairs"
        executed = round(14.0 * D * run.pairs / per[dom] / 1e9, 2)
        traffic = read_traffic(W.name, kname) if run.dname == "bf16" else None
    elif dom == "fwd":
        ach = fwd_flop / per[dom] / 1e9
        algo = f"4*D FLOP per visible pair (S, P V) x {run.pairs} pairs"
        executed, traffic = round(ach, 2), None
    else:  # the preprocess dominates only for degenerate problems
        ach, algo, executed, traffic = 0.0, "row sums only", 0.0, None
    out["roofline"] = {"kernel": kname, "call": ENTRY[dom], "bound": "mfma", "achieved": round(ach, 2),
                       "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": traffic,
                       "avg_ms": round(per[dom], 4), "algorithmic": algo, "executed_tflops": executed}
    out["kernels_ms"] = {k: round(v, 4) for k, v in per.items()}
    run.release()

    if not args.no_cells:
        cells = {}
        for name, dn in CELLS:
            if name == W.name and dn == run.dname:
                cells[f"{name}:{dn}"] = {k: out[k] for k in ("fwd", "bwd") if k in out}
                continue
            t0 = time.perf_counter()
            cw = wl_all[name]
            r = Run(cw, names[dn], ("fwd", "bwd"), dev)
            cper = r.time_runs(args.cell_steps, args.cell_warmup)
            cells[f"{name}:{dn}"] = r.summary(cper, peak_of(names[dn]))
            cells[f"{name}:{dn}"]["visible_pairs"] = r.pairs
            r.release()
            c = cells[f"{name}:{dn}"]
            log(f"[bench] cell {name}:{dn} fwd {c['fwd']['ms']} ms bwd {c['bwd']['ms']} ms "
                f"({time.perf_counter() - t0:.1f} s)")
        out["cells"] = cells
    if not args.no_cpu:
        log("[bench] timing the fp64 oracle on slices of the headline workload (CPU)")
        out["cpu_baseline"] = cpu_baseline(dataclasses.replace(W, passes=passes), dtype)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
