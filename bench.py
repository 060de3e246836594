#!/usr/bin/env python3
"""Throughput of the fused attention forward + backward on one MI355X.

One step = the whole path over one batch of synthetic input: attn_fwd (O,
LSE), then the backward's two calls (attn_bwd_preprocess for Delta, then
attn_bwd_dkdv_dq, which runs dK/dV and dQ as one fused grid or as two
kernels), all through the C ABI on torch's current stream.  Inputs are resident in HBM
before the timed region starts; K steps are timed between a synchronize on
each side, and every kernel is also bracketed by HIP events on the launch
stream so its own average duration is known.

FLOPs are counted on visible (query, key) pairs only: forward 4*D per pair
(Q K^T and P V), backward 10*D per pair (S recomputed once, dV, dP, dK, dQ).
The roofline object reports the dominant launch, attn_bwd_dkdv_dq (at
head_dim 128 one fused dK/dV + dQ kernel where the library takes that path),
against its own algorithmic work of 14*D FLOPs per visible pair (S, dV, dP,
dK for dK/dV; S, dP, dQ for dQ) and the bf16/fp16 dense MFMA peak of 2516.6
TFLOP/s (256 CUs x 2.4 GHz x 4096 FLOP/clk/CU).

The CPU baseline is the fp64 oracle timed on this host on one (sequence,
head) slice of the same workload, scaled to the same unit.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd/bwd TFLOP/s (unmasked FLOPs) + % bf16 MFMA peak, hdim 128"
PEAK_MFMA_16 = 2516.6   # TFLOP/s, bf16 and fp16 dense
PEAK_MFMA_32 = 157.3    # TFLOP/s, fp32
PEAK_HBM = 8000.0       # GB/s
DEFAULT_WORKLOAD = "long_6630"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dkdv_traffic_long_6630.txt")
KERNEL_SOURCES = ["scaled_dot_product_20_amd/csrc/attn_bwd.hip",
                  "scaled_dot_product_20_amd/csrc/attn_device.hpp",
                  "scaled_dot_product_20_amd/csrc/attn_launch.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(sq: int, sk: int, window, diag: str) -> int:
    """Visible (i, j) pairs of one sequence, by rows: key j is visible to
    query i iff i - L <= j <= i + R, (L, R) shifted by d = sk - sq under the
    bottom-right diagonal when both sides are finite."""
    import numpy as np
    inf = 2147483647
    wl, wr = window
    L, R = wl, wr
    if diag == "bottom_right" and wl != inf and wr != inf:
        L, R = wl - (sk - sq), wr + (sk - sq)
    i = np.arange(sq, dtype=np.int64)
    lo = np.zeros(sq, np.int64) if L == inf else np.maximum(0, i - L)
    hi = np.full(sq, sk - 1, np.int64) if R == inf else np.minimum(sk - 1, i + R)
    return int(np.maximum(0, hi - lo + 1).sum())


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def dkdv_kernel_name(dname: str, head_dim: int) -> str:
    """The dK/dV kernel the library launches for this dtype and head_dim."""
    if dname == "fp32":
        return "attn_bwd_dkdv_kernel"
    return "attn_bwd_dkdv16pc_kernel" if head_dim > 80 else "attn_bwd_dkdv16_kernel"


def wide_band(window) -> bool:
    """A band unbounded on one side or at least 1024 keys wide."""
    inf = 2147483647
    wl, wr = window
    return wl == inf or wr == inf or wl + wr + 1 >= 1024


def bwd_main_kernels(dname: str, head_dim: int, window, seqlen_q: int, heads: int, batch: int,
                     cus: int) -> list:
    """The kernels attn_bwd_dkdv_dq launches: the fused dK/dV + dQ grid for
    16-bit head_dim 128 when the band is wide and a separate dQ grid (two
    128-row workgroups per CU) would leave its last round at most a quarter full,
    else the dK/dV kernel then the dQ kernel."""
    slots = 2 * cus
    tail = (-(-seqlen_q // 128) * heads * batch) % slots if slots else 0
    if dname != "fp32" and head_dim > 80 and wide_band(window) and 0 < tail and 4 * tail <= slots:
        return ["attn_bwd_fused16_kernel"]
    dq = "attn_bwd_dq_kernel" if dname == "fp32" else "attn_bwd_dq16_kernel"
    return [dkdv_kernel_name(dname, head_dim), dq]


def fwd_kernel_name(dname: str, window) -> str:
    """The forward kernel the library launches: the 256-row ping-pong kernel
    for 16-bit inputs unless both window sides are finite and the band is
    under 1024 keys wide."""
    if dname == "fp32":
        return "attn_fwd_kernel"
    return "attn_fwd16pp_kernel" if wide_band(window) else "attn_fwd16_kernel"


def read_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the dK/dV (+ dQ) kernel from the committed
    counter summary, or None when there is none for this workload and kernel
    or the kernel's sources changed since."""
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
            "cores": orc.num_threads(), "kind": "oracle",
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--dtype", default=None, help="bf16 / fp16 / fp32 (default: the workload's first)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--passes", default=None, help="fwd or fwd,bwd (default: the workload's)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the attention step, run a plain device-to-device copy of MIB "
                         "MiB (the calibration kernel for HBM byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the attention kernels shard by head and batch with no "
              "communication, and this build runs on a single MI355X; --gpus must be 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from scaled_dot_product_20_amd import binding as bd
    from scaled_dot_product_20_amd import workloads as wls

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return
    W = wls.workloads()[args.workload]
    names = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
    dtype = names[args.dtype] if args.dtype else W.dtypes[0]
    dname = {v: k for k, v in names.items()}[dtype]
    passes = tuple(args.passes.split(",")) if args.passes else ("fwd", "bwd")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log(f"[bench] workload {W.name} dtype {dname} passes {passes}: drawing inputs")
    q, k, v, do = (t.to(dev) for t in W.inputs(dtype))
    cu_q, cu_k = W.cu_seqlens()
    kw = dict(scale=W.scale, window=W.window, diag=W.diag)
    if W.layout == "thd":
        kw.update(cu_seqlens_q=torch.from_numpy(cu_q).to(dev), cu_seqlens_k=torch.from_numpy(cu_k).to(dev),
                  max_seqlen_q=W.seqlen_q, max_seqlen_k=W.seqlen_k)
        lens = list(zip(W.lens_q, W.lens_k))
    else:
        lens = [(W.seqlen_q, W.seqlen_k)] * W.batch
    pairs = W.heads * sum(visible_pairs(a, b, W.window, W.diag) for a, b in lens)
    D = W.head_dim
    fwd_flop = 4.0 * D * pairs
    bwd_flop = 10.0 * D * pairs
    main_flop = 14.0 * D * pairs  # dK/dV (S, dV, dP, dK) and dQ (S, dP, dQ) as executed

    o, lse = bd.attn_fwd(q, k, v, **kw)
    fkw = dict(cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None)
    fkw.update(kw)
    fp = bd.fwd_params(q, k, v, o, lse, **fkw)
    do_bwd = "bwd" in passes
    if do_bwd:
        bp, keep = bd.prepare_bwd(do, q, k, v, o, lse, **kw)
    stream = torch.cuda.current_stream(dev)
    sid = stream.cuda_stream
    kernels = ["fwd"] + (["bwd_preprocess", "bwd_dkdv_dq"] if do_bwd else [])
    entry = {"fwd": "attn_fwd", "bwd_preprocess": "attn_bwd_preprocess", "bwd_dkdv_dq": "attn_bwd_dkdv_dq"}

    def step(evs=None):
        for i, kname in enumerate(kernels):
            if evs is not None:
                evs[i].record(stream)
            bd.launch(entry[kname], fp if kname == "fwd" else bp, sid)
        if evs is not None:
            evs[len(kernels)].record(stream)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)]
              for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_kernel = {kname: sum(ev[i].elapsed_time(ev[i + 1]) for ev in events) / args.steps
                  for i, kname in enumerate(kernels)}
    ms_step = wall * 1e3 / args.steps
    log("[bench] per-kernel ms " + json.dumps({k: round(v, 4) for k, v in per_kernel.items()}))

    peak = PEAK_MFMA_32 if dtype == torch.float32 else PEAK_MFMA_16
    total_flop = fwd_flop + (bwd_flop if do_bwd else 0.0)
    value = total_flop / (ms_step * 1e-3) / 1e12
    fwd_ms = per_kernel["fwd"]
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dname,
        "data": "synthetic: i.i.d. N(0,1) Q/K/V/dO from a seeded generator, cast RNE",
        "config": {"workload": W.name, "layout": W.layout, "batch": W.batch, "heads": W.heads,
                   "head_dim": D, "seqlen_q": W.seqlen_q, "seqlen_k": W.seqlen_k,
                   "window": list(W.window), "diag": W.diag, "passes": list(passes),
                   "visible_pairs": pairs},
        "frac_of_peak": round(value / peak, 4),
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(fwd_flop / fwd_ms / 1e9, 2),
                "frac_of_peak": round(fwd_flop / fwd_ms / 1e9 / peak, 4)},
    }
    if do_bwd:
        bwd_ms = per_kernel["bwd_preprocess"] + per_kernel["bwd_dkdv_dq"]
        out["bwd"] = {"ms": round(bwd_ms, 4), "tflops": round(bwd_flop / bwd_ms / 1e9, 2),
                      "frac_of_peak": round(bwd_flop / bwd_ms / 1e9 / peak, 4)}
        main_ms = per_kernel["bwd_dkdv_dq"]
        ach = main_flop / main_ms / 1e9
        knames = bwd_main_kernels(dname, D, W.window, W.seqlen_q, W.heads, W.batch,
                                  torch.cuda.get_device_properties(dev).multi_processor_count)
        kname = "+".join(knames)
        traffic = read_traffic(W.name, kname) if dname == "bf16" else None
        out["roofline"] = {"kernel": kname, "bound": "mfma", "achieved": round(ach, 2),
                           "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                           "traffic": traffic, "avg_ms": round(main_ms, 4),
                           "algorithmic": f"14*D FLOP per visible pair (S, dV, dP, dK; S, dP, dQ) x {pairs} pairs"}
    else:
        ach = fwd_flop / fwd_ms / 1e9
        kname = fwd_kernel_name(dname, W.window)
        out["roofline"] = {"kernel": kname, "bound": "mfma", "achieved": round(ach, 2),
                           "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                           "traffic": None, "avg_ms": round(fwd_ms, 4),
                           "algorithmic": f"4*D FLOP per visible pair x {pairs} pairs"}
    out["kernels_ms"] = {k: round(v, 4) for k, v in per_kernel.items()}
    if not args.no_cpu:
        log("[bench] timing the fp64 oracle on one slice (CPU)")
        out["cpu_baseline"] = cpu_baseline(dataclasses.replace(W, passes=passes), dtype)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
