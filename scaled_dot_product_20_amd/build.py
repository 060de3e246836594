"""Build ``libsdpa20.so`` (gfx950 code objects + the C ABI) in-tree with hipcc.

Usage: ``python -m scaled_dot_product_20_amd.build`` (or ``build()``).
Every HIP source is compiled with packed-fp32 code generation disabled (the
host compiler warns that it does not know that feature, which is harmless)
and as code object v5, which every ROCm 6/7 runtime loads, including the one
bundled with PyTorch that the library binds to when torch is imported first.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsdpa20.so")
ARCH = "gfx950"

SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "attn_bwd_f32.hip", "attn_bwd_f16.hip", "attn_bwd_bf16.hip",
           "attn_api.cpp"]
HEADERS = ["attn_device.hpp", "attn_launch.hpp", "attn_feat.hpp", "attn_bwd_kernels.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(OUT_DIR, src.replace(".", "_") + ".o")
        objs.append(obj)
        cmd = [HIPCC] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(line for line in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in line)
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        msg = "\n".join(f"--- {s}\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5",
           "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
