"""Python front of the fp64 CPU oracle (``sdpa_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module; the product path
never does.  It shares no code with the GPU library: the C file carries its
own visibility predicate, its own bf16/fp16 decoders and its own arithmetic.

Inputs are CPU torch tensors (float32, float16 or bfloat16) in one of two
contiguous layouts: dense ``[B, H, S, D]`` or packed ``[T, H, D]`` with
host ``cu_seqlens`` arrays.  Outputs are float64 numpy arrays: O and the
gradients shaped like their inputs, LSE ``[B, H, Sq]`` (dense) or ``[H, Tq]``
(packed).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sdpa_oracle.c")
LIB = os.path.join(HERE, "libsdpa_oracle.so")

WINDOW_INF = 2147483647
F32, F16, BF16 = 0, 1, 2
DENSE, PACKED = 0, 1
TOP_LEFT, BOTTOM_RIGHT = 0, 1

_DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < max(
        os.path.getmtime(SRC), os.path.getmtime(os.path.join(HERE, "sdpa_oracle.h"))
    ):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
             "-o", tmp, SRC, "-lm"]
        )
        os.replace(tmp, LIB)
    return LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("layout", ctypes.c_int),
        ("batch", ctypes.c_int),
        ("heads", ctypes.c_int),
        ("head_dim", ctypes.c_int),
        ("seqlen_q", ctypes.c_int),
        ("seqlen_k", ctypes.c_int),
        ("cu_seqlens_q", ctypes.POINTER(ctypes.c_int32)),
        ("cu_seqlens_k", ctypes.POINTER(ctypes.c_int32)),
        ("window_left", ctypes.c_int),
        ("window_right", ctypes.c_int),
        ("diag", ctypes.c_int),
        ("scale", ctypes.c_double),
        ("bias", ctypes.c_void_p),
        ("bias_stride", ctypes.c_int64 * 3),
        ("alibi_slopes", ctypes.POINTER(ctypes.c_double)),
        ("dropout_p", ctypes.c_double),
        ("philox_seed", ctypes.c_uint64),
        ("philox_offset", ctypes.c_uint64),
        ("max_seqlen_q", ctypes.c_int),
        ("max_seqlen_k", ctypes.c_int),
        ("head_dim_v", ctypes.c_int),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        vp, dp, ip = ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)
        pp = ctypes.POINTER(_Problem)
        lib.oracle_visible.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int] * 3
        lib.oracle_visible.restype = ctypes.c_int
        lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_f16.restype = ctypes.c_double
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_bf16.restype = ctypes.c_double
        lib.oracle_fwd.argtypes = [pp, vp, vp, vp, dp, dp]
        lib.oracle_bwd.argtypes = [pp, vp, vp, vp, vp, dp, dp, dp, dp, dp]
        lib.oracle_bwd_dbias.argtypes = [pp, vp, vp, vp, vp, dp, dp, dp, dp, dp, dp]
        u32p = ctypes.POINTER(ctypes.c_uint32)
        lib.oracle_philox4x32_10.argtypes = [u32p, u32p, u32p]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_dropout_keep.argtypes = [pp, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
        lib.oracle_dropout_keep.restype = ctypes.c_int
        lib.oracle_dropout_mask.argtypes = [pp, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.POINTER(ctypes.c_uint8)]
        lib.oracle_dropout_mask.restype = None
        lib.oracle_fwd_rows.argtypes = [pp, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ip, dp, dp]
        lib.oracle_bwd_dq_rows.argtypes = [pp, vp, vp, vp, vp, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ip, dp]
        lib.oracle_bwd_dkdv_cols.argtypes = [pp, vp, vp, vp, vp, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ip, dp, dp]
        for f in ("oracle_fwd", "oracle_bwd", "oracle_bwd_dbias", "oracle_fwd_rows",
                  "oracle_bwd_dq_rows", "oracle_bwd_dkdv_cols"):
            getattr(lib, f).restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _diag_code(diag) -> int:
    if diag in (TOP_LEFT, "top_left"):
        return TOP_LEFT
    if diag in (BOTTOM_RIGHT, "bottom_right"):
        return BOTTOM_RIGHT
    raise ValueError("diag must be 'top_left' or 'bottom_right'")


class _Call:
    """Keeps the marshalled inputs alive for the duration of one C call.

    Optional features (keyword arguments of every entry below): ``bias`` (a
    CPU tensor in the inputs' dtype, indexed [b, h, i, j] with local
    indices, broadcast strides allowed, unit stride on j), ``alibi_slopes``
    (one per head), ``dropout_p`` with ``philox_seed`` / ``philox_offset``,
    and ``max_seqlen_q`` / ``max_seqlen_k`` (the row length of the dropout
    counters and of dBias; default the largest lengths)."""

    def __init__(self, q, k, v, dout, window, diag, scale, cu_seqlens_q, cu_seqlens_k, bias=None,
                 alibi_slopes=None, dropout_p=0.0, philox_seed=0, philox_offset=0, max_seqlen_q=None,
                 max_seqlen_k=None):
        tensors = [q, k, v] + ([dout] if dout is not None else [])
        dt = q.dtype
        if dt not in _DTYPE_CODE or any(t.dtype != dt for t in tensors):
            raise TypeError("q, k, v (and dout) must share one of float32/float16/bfloat16")
        if any(t.device.type != "cpu" for t in tensors):
            raise TypeError("the oracle takes CPU tensors")
        self.keep = [t.contiguous() for t in tensors]
        packed = cu_seqlens_q is not None
        p = _Problem()
        p.dtype = _DTYPE_CODE[dt]
        wl, wr = window
        p.window_left, p.window_right = int(wl), int(wr)
        p.diag = _diag_code(diag)
        p.scale = float(scale)
        if packed:
            if cu_seqlens_k is None:
                raise ValueError("packed layout needs both cu_seqlens")
            self.cuq = np.ascontiguousarray(np.asarray(cu_seqlens_q, dtype=np.int32))
            self.cuk = np.ascontiguousarray(np.asarray(cu_seqlens_k, dtype=np.int32))
            if q.dim() != 3:
                raise ValueError("packed inputs are [T, H, D]")
            p.layout = PACKED
            p.batch = len(self.cuq) - 1
            p.heads, p.head_dim = q.shape[1], q.shape[2]
            p.cu_seqlens_q = self.cuq.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
            p.cu_seqlens_k = self.cuk.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
            self.lse_shape = (p.heads, int(self.cuq[-1]))
        else:
            if q.dim() != 4:
                raise ValueError("dense inputs are [B, H, S, D]")
            p.layout = DENSE
            p.batch, p.heads, p.seqlen_q, p.head_dim = q.shape
            p.seqlen_k = k.shape[2]
            self.lse_shape = (p.batch, p.heads, p.seqlen_q)
        if bias is not None:
            if bias.dtype != dt or bias.device.type != "cpu" or bias.dim() != 4:
                raise TypeError("bias is a 4-d CPU tensor in the inputs' dtype")
            if bias.stride(-1) != 1:
                bias = bias.contiguous()
            self.bias = bias
            p.bias = ctypes.c_void_p(bias.data_ptr())
            for t in range(3):
                p.bias_stride[t] = bias.stride(t) if bias.shape[t] > 1 else 0
        if alibi_slopes is not None:
            self.slopes = np.ascontiguousarray(np.asarray(alibi_slopes, dtype=np.float64))
            if self.slopes.shape != (p.heads,):
                raise ValueError("one ALiBi slope per head")
            p.alibi_slopes = self.slopes.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
        p.dropout_p = float(dropout_p)
        p.philox_seed = int(philox_seed) & (2**64 - 1)
        p.philox_offset = int(philox_offset) & (2**64 - 1)
        if packed:
            lq = np.diff(self.cuq) if len(self.cuq) > 1 else np.zeros(1, np.int32)
            lk = np.diff(self.cuk) if len(self.cuk) > 1 else np.zeros(1, np.int32)
            p.max_seqlen_q = int(lq.max()) if max_seqlen_q is None else int(max_seqlen_q)
            p.max_seqlen_k = int(lk.max()) if max_seqlen_k is None else int(max_seqlen_k)
        else:
            p.max_seqlen_q = p.seqlen_q if max_seqlen_q is None else int(max_seqlen_q)
            p.max_seqlen_k = p.seqlen_k if max_seqlen_k is None else int(max_seqlen_k)
        if v.shape[:-1] != k.shape[:-1] or (dout is not None and dout.shape[:-1] != q.shape[:-1]):
            raise ValueError("v must match k, and dout q, in every dim but the last")
        if dout is not None and dout.shape[-1] != v.shape[-1]:
            raise ValueError("dout has v's head dim")
        p.head_dim_v = v.shape[-1]
        self.p = p
        self.D, self.DV = p.head_dim, p.head_dim_v
        self.o_shape = tuple(q.shape[:-1]) + (self.DV,)

    def ptr(self, i):
        return ctypes.c_void_p(self.keep[i].data_ptr())


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def fwd(q, k, v, *, scale, window=(WINDOW_INF, WINDOW_INF), diag="top_left",
        cu_seqlens_q=None, cu_seqlens_k=None, **feat):
    """O and LSE of the whole problem (float64)."""
    c = _Call(q, k, v, None, window, diag, scale, cu_seqlens_q, cu_seqlens_k, **feat)
    o = np.zeros(c.o_shape, dtype=np.float64)
    lse = np.zeros(c.lse_shape, dtype=np.float64)
    rc = _load().oracle_fwd(ctypes.byref(c.p), c.ptr(0), c.ptr(1), c.ptr(2), _dptr(o), _dptr(lse))
    if rc:
        raise ValueError("oracle_fwd rejected the problem")
    return o, lse


def bwd(q, k, v, dout, *, scale, window=(WINDOW_INF, WINDOW_INF), diag="top_left",
        cu_seqlens_q=None, cu_seqlens_k=None, want_dbias=False, **feat):
    """(O, LSE, dQ, dK, dV) of the whole problem (float64); with
    ``want_dbias`` also dBias = d loss / d logits, [B, H, max_seqlen_q,
    max_seqlen_k] (0 where the sequence has no pair)."""
    c = _Call(q, k, v, dout, window, diag, scale, cu_seqlens_q, cu_seqlens_k, **feat)
    o = np.zeros(c.o_shape, dtype=np.float64)
    lse = np.zeros(c.lse_shape, dtype=np.float64)
    dq = np.zeros(tuple(q.shape), dtype=np.float64)
    dk = np.zeros(tuple(k.shape), dtype=np.float64)
    dv = np.zeros(tuple(v.shape), dtype=np.float64)
    db = np.zeros((c.p.batch, c.p.heads, c.p.max_seqlen_q, c.p.max_seqlen_k), dtype=np.float64) \
        if want_dbias else None
    rc = _load().oracle_bwd_dbias(ctypes.byref(c.p), c.ptr(0), c.ptr(1), c.ptr(2), c.ptr(3),
                                  _dptr(o), _dptr(lse), _dptr(dq), _dptr(dk), _dptr(dv),
                                  _dptr(db) if db is not None else None)
    if rc:
        raise ValueError("oracle_bwd rejected the problem")
    return (o, lse, dq, dk, dv, db) if want_dbias else (o, lse, dq, dk, dv)


def fwd_rows(q, k, v, b, h, rows, *, scale, window=(WINDOW_INF, WINDOW_INF),
             diag="top_left", cu_seqlens_q=None, cu_seqlens_k=None, **feat):
    """O rows [n, DV] (V's head dim) and LSE [n] for sequence-local query
    rows of (b, h)."""
    c = _Call(q, k, v, None, window, diag, scale, cu_seqlens_q, cu_seqlens_k, **feat)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    o = np.zeros((len(rows), c.DV), dtype=np.float64)
    lse = np.zeros(len(rows), dtype=np.float64)
    rc = _load().oracle_fwd_rows(ctypes.byref(c.p), c.ptr(0), c.ptr(1), c.ptr(2), int(b), int(h),
                                 len(rows), _iptr(rows), _dptr(o), _dptr(lse))
    if rc:
        raise ValueError("oracle_fwd_rows rejected the problem")
    return o, lse


def bwd_dq_rows(q, k, v, dout, b, h, rows, *, scale, window=(WINDOW_INF, WINDOW_INF),
                diag="top_left", cu_seqlens_q=None, cu_seqlens_k=None, **feat):
    """dQ rows [n, D] for sequence-local query rows of (b, h)."""
    c = _Call(q, k, v, dout, window, diag, scale, cu_seqlens_q, cu_seqlens_k, **feat)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    dq = np.zeros((len(rows), c.D), dtype=np.float64)
    rc = _load().oracle_bwd_dq_rows(ctypes.byref(c.p), c.ptr(0), c.ptr(1), c.ptr(2), c.ptr(3),
                                    int(b), int(h), len(rows), _iptr(rows), _dptr(dq))
    if rc:
        raise ValueError("oracle_bwd_dq_rows rejected the problem")
    return dq


def bwd_dkdv_cols(q, k, v, dout, b, h, cols, *, scale, window=(WINDOW_INF, WINDOW_INF),
                  diag="top_left", cu_seqlens_q=None, cu_seqlens_k=None, **feat):
    """dK rows [n, D] and dV rows [n, DV] for sequence-local key rows of
    (b, h)."""
    c = _Call(q, k, v, dout, window, diag, scale, cu_seqlens_q, cu_seqlens_k, **feat)
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int32))
    dk = np.zeros((len(cols), c.D), dtype=np.float64)
    dv = np.zeros((len(cols), c.DV), dtype=np.float64)
    rc = _load().oracle_bwd_dkdv_cols(ctypes.byref(c.p), c.ptr(0), c.ptr(1), c.ptr(2), c.ptr(3),
                                      int(b), int(h), len(cols), _iptr(cols), _dptr(dk), _dptr(dv))
    if rc:
        raise ValueError("oracle_bwd_dkdv_cols rejected the problem")
    return dk, dv


def visible(i, j, sq, sk, window_left, window_right, diag="top_left") -> bool:
    return bool(_load().oracle_visible(int(i), int(j), int(sq), int(sk), int(window_left),
                                       int(window_right), _diag_code(diag)))


def visible_matrix(sq, sk, window_left, window_right, diag="top_left") -> np.ndarray:
    """Boolean [sq, sk] visibility matrix, one C call per element."""
    f = _load().oracle_visible
    d = _diag_code(diag)
    m = np.zeros((sq, sk), dtype=bool)
    for i in range(sq):
        for j in range(sk):
            m[i, j] = bool(f(i, j, sq, sk, int(window_left), int(window_right), d))
    return m


def decode_f16(bits: int) -> float:
    return _load().oracle_decode_f16(int(bits) & 0xFFFF)


def decode_bf16(bits: int) -> float:
    return _load().oracle_decode_bf16(int(bits) & 0xFFFF)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def philox4x32_10(ctr, key):
    """The four 32-bit output words of Philox4x32-10 at counter ctr[4] under
    key key[2]."""
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    out = (ctypes.c_uint32 * 4)()
    _load().oracle_philox4x32_10(c, k, out)
    return [int(x) for x in out]


def dropout_keep(q, k, v, b, h, i, j, *, cu_seqlens_q=None, cu_seqlens_k=None, **feat):
    """1 when the dropout of the problem keeps pair (i, j) of (b, h)."""
    c = _Call(q, k, v, None, (WINDOW_INF, WINDOW_INF), "top_left", 1.0, cu_seqlens_q, cu_seqlens_k, **feat)
    return int(_load().oracle_dropout_keep(ctypes.byref(c.p), int(b), int(h), int(i), int(j)))


def dropout_mask(q, k, v, b, h, nq, nk, *, cu_seqlens_q=None, cu_seqlens_k=None, **feat):
    """bool [nq, nk]: the keep decisions of rows [0, nq) and keys [0, nk) of
    (b, h) for the problem's dropout."""
    c = _Call(q, k, v, None, (WINDOW_INF, WINDOW_INF), "top_left", 1.0, cu_seqlens_q, cu_seqlens_k, **feat)
    out = np.zeros((int(nq), int(nk)), dtype=np.uint8)
    _load().oracle_dropout_mask(ctypes.byref(c.p), int(b), int(h), int(nq), int(nk),
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    return out.astype(bool)
