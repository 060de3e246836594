"""Thin ctypes binding of ``include/attn.h``.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libsdpa20.so``.  torch supplies device memory (output and
workspace allocation) and the current stream; there is no CPU or eager
fallback, and calling into a missing library raises immediately.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (both carry the same soname), and the
streams and device pointers torch hands over belong to that runtime.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsdpa20.so")

WINDOW_INF = 2147483647
PARAMS_VERSION = 3
FLAG_LSE_TH = 1  # ATTN_FLAG_LSE_TH: packed LSE as [T, H]
FLAG_NO_SPLIT = 2  # ATTN_FLAG_NO_SPLIT: no split mode (backward), no key-split workgroups (forward)
FP32, FP16, BF16 = 0, 1, 2
BHSD, THD, VARLEN = 0, 1, 2
# Mode byte of one side under VARLEN (ATTN_SEQ_* in include/attn.h).
SEQ_STACKED = 0x01
SEQ_LEN_UNIFORM, SEQ_LEN_CUMSUM, SEQ_LEN_ARRAY = 0x00, 0x02, 0x04
SEQ_POS_UNIFORM, SEQ_POS_CUMSUM, SEQ_POS_ARRAY = 0x00, 0x08, 0x10
TOP_LEFT, BOTTOM_RIGHT = 0, 1

_DTYPE = {torch.float32: FP32, torch.float16: FP16, torch.bfloat16: BF16}
_HIP_ERRORS = {1: "hipErrorInvalidValue", 2: "hipErrorOutOfMemory", 801: "hipErrorNotSupported", 98: "hipErrorInvalidDeviceFunction",
               209: "hipErrorNoBinaryForGpu", 200: "hipErrorInvalidImage"}

_I64x3 = ctypes.c_int64 * 3


class FwdParams(ctypes.Structure):
    _fields_ = [
        ("version", ctypes.c_uint32), ("flags", ctypes.c_uint32),
        ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("seqlen_q", ctypes.c_int32), ("seqlen_k", ctypes.c_int32),
        ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
        ("diag", ctypes.c_int32), ("scale", ctypes.c_float), ("reserved0", ctypes.c_int32),
        ("total_q", ctypes.c_int64), ("total_k", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("q_stride", _I64x3), ("k_stride", _I64x3), ("v_stride", _I64x3), ("o_stride", _I64x3),
        ("seqused_q", ctypes.c_void_p), ("seqused_k", ctypes.c_void_p),
        ("varlen", ctypes.c_uint32), ("reserved1", ctypes.c_int32),
        ("seqstart_q", ctypes.c_void_p), ("seqstart_k", ctypes.c_void_p),
        ("bias", ctypes.c_void_p), ("bias_stride", _I64x3), ("alibi_slopes", ctypes.c_void_p),
        ("dropout_p", ctypes.c_float), ("head_dim_v", ctypes.c_int32),
        ("philox_seed", ctypes.c_uint64), ("philox_offset", ctypes.c_uint64),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64),
    ]


class BwdParams(ctypes.Structure):
    _fields_ = [
        ("fwd", FwdParams),
        ("dout", ctypes.c_void_p), ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p),
        ("dv", ctypes.c_void_p),
        ("do_stride", _I64x3), ("dq_stride", _I64x3), ("dk_stride", _I64x3), ("dv_stride", _I64x3),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64),
        ("dbias", ctypes.c_void_p), ("dbias_stride", _I64x3),
    ]


PLAN_MAX = 8
BWD_PREPROCESS, BWD_DKDV, BWD_DQ, BWD_ALL = 1, 2, 4, 7
# ATTN_NOALLOC_SCRATCH_BYTES: the workspace limit of attn_bwd_noalloc.
NOALLOC_SCRATCH_BYTES = 16 << 20
# Backward steps each entry point runs (attn_bwd_plan's `steps`).
ENTRY_STEPS = {"attn_bwd": BWD_ALL, "attn_bwd_noalloc": BWD_ALL, "attn_bwd_preprocess": BWD_PREPROCESS,
               "attn_bwd_dkdv": BWD_DKDV, "attn_bwd_dq": BWD_DQ, "attn_bwd_dkdv_dq": BWD_DKDV | BWD_DQ}


class Plan(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_char_p * PLAN_MAX), ("grid", ctypes.c_uint32 * PLAN_MAX),
        ("block", ctypes.c_uint32 * PLAN_MAX), ("count", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


_lib = None


def lib():
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m scaled_dot_product_20_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, ptype in (("attn_fwd", FwdParams), ("attn_bwd", BwdParams),
                            ("attn_bwd_preprocess", BwdParams), ("attn_bwd_dkdv", BwdParams),
                            ("attn_bwd_dq", BwdParams), ("attn_bwd_dkdv_dq", BwdParams),
                            ("attn_bwd_noalloc", BwdParams)):
            f = getattr(l, name)
            f.argtypes = [ctypes.POINTER(ptype), ctypes.c_void_p]
            f.restype = ctypes.c_int
        l.attn_fwd_check.argtypes = [ctypes.POINTER(FwdParams)]
        l.attn_fwd_check.restype = ctypes.c_int
        l.attn_bwd_check.argtypes = [ctypes.POINTER(BwdParams)]
        l.attn_bwd_check.restype = ctypes.c_int
        l.attn_bwd_workspace_size.argtypes = [ctypes.POINTER(BwdParams)]
        l.attn_bwd_workspace_size.restype = ctypes.c_uint64
        l.attn_fwd_workspace_size.argtypes = [ctypes.POINTER(FwdParams)]
        l.attn_fwd_workspace_size.restype = ctypes.c_uint64
        l.attn_params_version.restype = ctypes.c_uint32
        l.attn_fwd_plan.argtypes = [ctypes.POINTER(FwdParams), ctypes.c_void_p, ctypes.POINTER(Plan)]
        l.attn_fwd_plan.restype = ctypes.c_int
        l.attn_bwd_plan.argtypes = [ctypes.POINTER(BwdParams), ctypes.c_uint32, ctypes.c_void_p,
                                    ctypes.POINTER(Plan)]
        l.attn_bwd_plan.restype = ctypes.c_int
        _lib = l
    return _lib


class AttnError(RuntimeError):
    def __init__(self, call: str, code: int):
        self.code = code
        super().__init__(f"{call} failed: {_HIP_ERRORS.get(code, 'hipError')} ({code})")


def _diag(diag) -> int:
    if diag in ("top_left", TOP_LEFT):
        return TOP_LEFT
    if diag in ("bottom_right", BOTTOM_RIGHT):
        return BOTTOM_RIGHT
    raise ValueError("diag must be 'top_left' or 'bottom_right'")


def _strides(t: torch.Tensor):
    """{batch, head, row} element strides; head_dim must be contiguous."""
    if t.stride(-1) != 1:
        raise ValueError("the head_dim axis must be contiguous")
    if t.dim() == 4:  # [B, H, S, D]
        return _I64x3(t.stride(0), t.stride(1), t.stride(2))
    return _I64x3(0, t.stride(1), t.stride(0))  # [T, H, D]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _lse_flags(lse_layout: str, packed: bool) -> int:
    if lse_layout == "ht":
        return 0
    if lse_layout == "th" and packed:
        return FLAG_LSE_TH
    raise ValueError("lse_layout is 'ht', or 'th' for packed [T, H, D] inputs")


def _seqused(t: Optional[torch.Tensor], batch: int, dev):
    if t is None:
        return None
    if t.dtype != torch.int32 or t.numel() != batch or not t.is_contiguous() or t.device != dev:
        raise ValueError("seqused_q / seqused_k are contiguous int32 [batch] tensors on the inputs' device")
    return t


def _int_array(t: Optional[torch.Tensor], n: int, dev, what: str):
    if t is None:
        return None
    if t.dtype != torch.int32 or t.numel() != n or not t.is_contiguous() or t.device != dev:
        raise ValueError(f"{what} must be a contiguous int32 tensor of {n} entries on the inputs' device")
    return t


def _side(t: torch.Tensor, mode: int, cu, max_seqlen, name: str):
    """(stacked, rows or None, seqlen) of one side under an explicit mode."""
    if mode & SEQ_STACKED:
        if t.dim() != 3:
            raise ValueError(f"{name}: a stacked side is [T, H, D]")
        if max_seqlen is None:
            raise ValueError(f"{name}: a stacked side needs its max_seqlen (its uniform length for "
                             "SEQ_POS_UNIFORM)")
        return True, t.shape[0], int(max_seqlen)
    if t.dim() != 4:
        raise ValueError(f"{name}: a padded side is [B, H, S, D]")
    return False, None, t.shape[2]


def fwd_params(q, k, v, o, lse, *, scale, window, diag, cu_seqlens_q, cu_seqlens_k,
               max_seqlen_q, max_seqlen_k, lse_layout="ht", seqused_q=None, seqused_k=None,
               q_mode=None, k_mode=None, seqstart_q=None, seqstart_k=None, batch=None, bias=None,
               alibi_slopes=None, dropout_p=0.0, philox_seed=0, philox_offset=0, split=True) -> FwdParams:
    """Fill an attn_fwd_params from tensors (no device work).  ``lse_layout``
    'th' (a stacked Q side only) stores LSE as [T, H] instead of [H, T].
    ``seqused_q`` / ``seqused_k`` (int32 [batch] on the device): sequence b
    uses only its first seqused[b] rows; the rest of its room are written as
    masked.  ``q_mode`` / ``k_mode`` (SEQ_* bits) select the ATTN_VARLEN
    layout, each side addressed on its own: a stacked side is [T, H, D], a
    padded one [B, H, S, D]; ``seqstart_q`` / ``seqstart_k`` are the start
    rows of SEQ_POS_ARRAY; ``batch`` is required when no array gives it.
    Optional features: ``bias`` (inputs' dtype, indexable [B, H, seqlen_q,
    seqlen_k] with sequence-local query / key indices; size-1 axes
    broadcast; unit stride on the key axis), ``alibi_slopes`` (fp32 [H]),
    ``dropout_p`` with ``philox_seed`` / ``philox_offset``.  ``split=False``
    keeps the backward out of its split mode and the forward on its plain
    grid (ATTN_FLAG_NO_SPLIT)."""
    p = FwdParams()
    p.version = PARAMS_VERSION
    if q.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    p.dtype = _DTYPE[q.dtype]
    p.window_left, p.window_right = int(window[0]), int(window[1])
    p.diag = _diag(diag)
    p.scale = float(scale)
    p.q, p.k, p.v, p.o, p.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse)
    p.q_stride, p.k_stride, p.v_stride, p.o_stride = _strides(q), _strides(k), _strides(v), _strides(o)
    if q_mode is not None or k_mode is not None:
        if q_mode is None or k_mode is None:
            raise ValueError("q_mode and k_mode go together")
        p.layout = VARLEN
        p.varlen = (int(q_mode) & 0xFF) | ((int(k_mode) & 0xFF) << 8)
        qst, tq, p.seqlen_q = _side(q, q_mode, cu_seqlens_q, max_seqlen_q, "q")
        kst, tk, p.seqlen_k = _side(k, k_mode, cu_seqlens_k, max_seqlen_k, "k")
        p.heads, p.head_dim = q.shape[-2] if qst else q.shape[1], q.shape[-1]
        p.total_q, p.total_k = tq or 0, tk or 0
        nb = [x.numel() - 1 for x in (cu_seqlens_q, cu_seqlens_k) if x is not None]
        nb += [x.numel() for x in (seqused_q, seqused_k, seqstart_q, seqstart_k) if x is not None]
        nb += [t.shape[0] for t, st in ((q, qst), (k, kst)) if not st]
        if batch is not None:
            nb.append(int(batch))
        if not nb or any(n != nb[0] for n in nb):
            raise ValueError(f"the sides disagree on the number of sequences: {nb}")
        p.batch = nb[0]
        p.flags = FLAG_LSE_TH if lse_layout == "th" and qst else 0
        if lse_layout not in ("ht", "th") or (lse_layout == "th" and not qst):
            raise ValueError("lse_layout is 'ht', or 'th' for a stacked Q side")
        p.cu_seqlens_q, p.cu_seqlens_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k)
        p.seqstart_q = _ptr(_int_array(seqstart_q, p.batch, q.device, "seqstart_q"))
        p.seqstart_k = _ptr(_int_array(seqstart_k, p.batch, q.device, "seqstart_k"))
    elif q.dim() == 4:
        p.flags = _lse_flags(lse_layout, False)
        p.layout = BHSD
        p.batch, p.heads, p.seqlen_q, p.head_dim = q.shape
        p.seqlen_k = k.shape[2]
    elif q.dim() == 3:
        p.flags = _lse_flags(lse_layout, True)
        if cu_seqlens_q is None or cu_seqlens_k is None:
            raise ValueError("packed [T, H, D] inputs need cu_seqlens_q and cu_seqlens_k")
        p.layout = THD
        p.batch = cu_seqlens_q.numel() - 1
        p.total_q, p.heads, p.head_dim = q.shape
        p.total_k = k.shape[0]
        p.seqlen_q, p.seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
        p.cu_seqlens_q, p.cu_seqlens_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k)
    else:
        raise ValueError("inputs are [B, H, S, D] or [T, H, D]")
    p.seqused_q = _ptr(_seqused(seqused_q, p.batch, q.device))
    p.seqused_k = _ptr(_seqused(seqused_k, p.batch, q.device))
    if v.shape[-1] != q.shape[-1]:
        p.head_dim_v = v.shape[-1]
    if bias is not None:
        p.bias, p.bias_stride = _ptr(bias), _bias_strides(bias, q, "bias")
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or alibi_slopes.device != q.device or \
                alibi_slopes.shape != (p.heads,) or alibi_slopes.stride(0) != 1:
            raise ValueError("alibi_slopes: contiguous fp32 [heads] on the inputs' device")
        p.alibi_slopes = _ptr(alibi_slopes)
    if not split:
        p.flags |= FLAG_NO_SPLIT
    p.dropout_p = float(dropout_p)
    p.philox_seed = int(philox_seed) & (2**64 - 1)
    p.philox_offset = int(philox_offset) & (2**64 - 1)
    return p


def _bias_strides(t, q, name, dtype=None):
    """[b, h, i] element strides of a 4-d bias-shaped tensor (0 on size-1
    axes: broadcast)."""
    if t.dim() != 4 or t.device != q.device or t.dtype != (q.dtype if dtype is None else dtype):
        raise ValueError(f"{name}: a 4-d tensor [B, H, Sq, Sk] on the inputs' device, "
                         f"dtype {q.dtype if dtype is None else dtype}")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name}: unit stride on the key axis")
    return _I64x3(*[t.stride(i) if t.shape[i] > 1 else 0 for i in range(3)])


def _max_len(cu: torch.Tensor) -> int:
    # Reads the lengths back to the host (a sync); pass max_seqlen_* to avoid it.
    return int((cu[1:] - cu[:-1]).max().item()) if cu.numel() > 1 else 0


def _check_inputs(*ts):
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    for t in ts:
        if t.device != dev or t.dtype != ts[0].dtype:
            raise ValueError("q, k, v (o, dout) must share device and dtype")


def _cu(cu, dev):
    if cu is None:
        return None
    if cu.dtype != torch.int32 or cu.device != dev:
        raise ValueError("cu_seqlens must be int32 tensors on the inputs' device")
    return cu.contiguous()


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _problem(q, *, scale=None, window=(WINDOW_INF, WINDOW_INF), diag="top_left", cu_seqlens_q=None,
             cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, lse_layout="ht", seqused_q=None,
             seqused_k=None, q_mode=None, k_mode=None, seqstart_q=None, seqstart_k=None, batch=None,
             bias=None, alibi_slopes=None, dropout_p=0.0, philox_seed=0, philox_offset=0, split=True,
             read_back=True):
    """The keyword arguments of fwd_params for a call: default scale,
    cu_seqlens checked, and (packed [T, H, D] inputs without modes) the max
    lengths read back from cu_seqlens when not given and `read_back`."""
    dev = q.device
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    cu_q, cu_k = _cu(cu_seqlens_q, dev), _cu(cu_seqlens_k, dev)
    if q_mode is None and q.dim() == 3:
        if not read_back and (max_seqlen_q is None or max_seqlen_k is None):
            raise ValueError("packed inputs need max_seqlen_q and max_seqlen_k (no device read-back here)")
        max_seqlen_q = _max_len(cu_q) if max_seqlen_q is None else max_seqlen_q
        max_seqlen_k = _max_len(cu_k) if max_seqlen_k is None else max_seqlen_k
    return dict(scale=scale, window=window, diag=diag, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k, lse_layout=lse_layout,
                seqused_q=seqused_q, seqused_k=seqused_k, q_mode=q_mode, k_mode=k_mode,
                seqstart_q=seqstart_q, seqstart_k=seqstart_k, batch=batch, bias=bias,
                alibi_slopes=alibi_slopes, dropout_p=dropout_p, philox_seed=philox_seed,
                philox_offset=philox_offset, split=split)


def lse_shape(q: torch.Tensor, lse_layout="ht", q_mode=None):
    """Shape of the LSE a forward writes: [B, H, S] for a padded Q side,
    [H, T] or [T, H] ('th') for a stacked one."""
    stacked = q.dim() == 3 if q_mode is None else bool(q_mode & SEQ_STACKED)
    if not stacked:
        return tuple(q.shape[:3])
    return (q.shape[1], q.shape[0]) if lse_layout == "ht" else (q.shape[0], q.shape[1])


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None, **kw):
    """Forward: returns (O, LSE).  Keywords: scale (default 1/sqrt(D)),
    window, diag, cu_seqlens_q/k, max_seqlen_q/k, lse_layout, seqused_q/k,
    and for the ATTN_VARLEN layout q_mode, k_mode, seqstart_q/k, batch (see
    fwd_params).  LSE is fp32 [B, H, Sq] (padded Q), [H, T] (stacked Q) or
    [T, H] (stacked Q, ``lse_layout='th'``)."""
    _check_inputs(q, k, v)
    dev = q.device
    pk = _problem(q, **kw)
    if out is None:
        o = torch.empty(tuple(q.shape[:-1]) + (v.shape[-1],), dtype=q.dtype, device=dev)
    else:
        o = out
    if lse is None:
        lse = torch.empty(lse_shape(q, pk["lse_layout"], pk["q_mode"]), dtype=torch.float32, device=dev)
    p, _ws = prepare_fwd(q, k, v, o, lse, **pk)
    rc = lib().attn_fwd(ctypes.byref(p), ctypes.c_void_p(_stream(dev)))
    if rc:
        raise AttnError("attn_fwd", rc)
    return o, lse


def prepare_fwd(q, k, v, o, lse, *, workspace=None, **kw):
    """Params of a forward (keywords as fwd_params) with its workspace:
    attn_fwd_workspace_size bytes (the zero-padded copies of a repacked
    call, and the key-split tail's partial sums for large fp16 / bf16
    forwards), allocated when ``workspace`` is None.  Returns (params,
    workspace or None); the tensor must outlive the launches."""
    p = fwd_params(q, k, v, o, lse, **kw)
    need = int(lib().attn_fwd_workspace_size(ctypes.byref(p)))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        p.workspace = _ptr(workspace)
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    return p, workspace


def bwd_params(dout, q, k, v, o, lse, dq, dk, dv, workspace, dbias=None, **kw) -> BwdParams:
    """Fill an attn_bwd_params (keywords as for fwd_params); ``dbias``: the
    optional fp32 output d loss / d logits, [B, H, seqlen_q, seqlen_k]."""
    p = BwdParams()
    p.fwd = fwd_params(q, k, v, o, lse, **kw)
    if dbias is not None:
        p.dbias, p.dbias_stride = _ptr(dbias), _bias_strides(dbias, q, "dbias", torch.float32)
    p.dout, p.dq, p.dk, p.dv = _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv)
    p.do_stride, p.dq_stride = _strides(dout), _strides(dq)
    p.dk_stride, p.dv_stride = _strides(dk), _strides(dv)
    if workspace is not None:
        p.workspace = _ptr(workspace)
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    return p


def _bwd_outputs(q, k, v, dq, dk, dv):
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    return dq, dk, dv


def prepare_bwd(dout, q, k, v, o, lse, *, dq=None, dk=None, dv=None, workspace=None, dbias=None, **kw):
    """Allocate the outputs and workspace of a backward and fill its params
    once, for callers that launch it repeatedly or step by step (keywords as
    for attn_fwd).  Returns (params, (dq, dk, dv, workspace)); the tensors
    must outlive every launch made with the params."""
    _check_inputs(q, k, v, o, dout)
    dev = q.device
    pk = _problem(q, **kw)
    dq, dk, dv = _bwd_outputs(q, k, v, dq, dk, dv)
    p = bwd_params(dout, q, k, v, o, lse, dq, dk, dv, None, dbias=dbias, **pk)
    if workspace is None:
        need = int(lib().attn_bwd_workspace_size(ctypes.byref(p)))
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    p.workspace = _ptr(workspace)
    p.workspace_bytes = workspace.numel() * workspace.element_size()
    p._keep = (pk["cu_seqlens_q"], pk["cu_seqlens_k"])  # device cu_seqlens referenced by the params
    return p, (dq, dk, dv, workspace)


def launch(name: str, params, stream: Optional[int] = None) -> None:
    """Call one C entry point (``attn_fwd``, ``attn_bwd``,
    ``attn_bwd_preprocess``, ``attn_bwd_dkdv``, ``attn_bwd_dq`` or
    ``attn_bwd_dkdv_dq``) with filled params on ``stream`` (default: torch's
    current stream)."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    rc = getattr(lib(), name)(ctypes.byref(params), ctypes.c_void_p(stream))
    if rc:
        raise AttnError(name, rc)


def plan(name: str, params, stream: Optional[int] = None):
    """The launches entry point ``name`` would make with these params, from
    the library's own launch choice (attn_fwd_plan / attn_bwd_plan): a list
    of (kernel name, workgroups, threads per workgroup).  Host-only."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    pl = Plan()
    if name == "attn_fwd":
        rc = lib().attn_fwd_plan(ctypes.byref(params), ctypes.c_void_p(stream), ctypes.byref(pl))
    else:
        rc = lib().attn_bwd_plan(ctypes.byref(params), ENTRY_STEPS[name], ctypes.c_void_p(stream),
                                 ctypes.byref(pl))
    if rc:
        raise AttnError(name + " plan", rc)
    return [(pl.kernel[i].decode(), int(pl.grid[i]), int(pl.block[i])) for i in range(pl.count)]


def attn_bwd_noalloc(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                     lse: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor, dbias=None,
                     **kw):
    """attn_bwd_noalloc: the backward into caller-given dq, dk, dv, with its
    workspace in the library's per-device static array (nothing allocated;
    keywords as for attn_fwd, packed inputs with their max_seqlen given).
    Raises when the problem's workspace exceeds NOALLOC_SCRATCH_BYTES."""
    _check_inputs(q, k, v, o, dout)
    dev = q.device
    pk = _problem(q, read_back=False, **kw)
    p = bwd_params(dout, q, k, v, o, lse, dq, dk, dv, None, dbias=dbias, **pk)
    rc = lib().attn_bwd_noalloc(ctypes.byref(p), ctypes.c_void_p(_stream(dev)))
    if rc == 2:  # hipErrorOutOfMemory
        need = int(lib().attn_bwd_workspace_size(ctypes.byref(p)))
        raise AttnError(f"attn_bwd_noalloc (workspace {need} B > limit {NOALLOC_SCRATCH_BYTES} B)", rc)
    if rc:
        raise AttnError("attn_bwd_noalloc", rc)
    return dq, dk, dv


def attn_bwd(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
             lse: torch.Tensor, *, dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
             dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             dbias: Optional[torch.Tensor] = None, **kw):
    """Backward: returns (dQ, dK, dV) given the forward's O and LSE (in the
    layout ``lse_layout`` names; keywords as for attn_fwd, with the same
    bias / alibi / dropout arguments as the forward).  ``dbias`` (fp32,
    [B, H, seqlen_q, seqlen_k]) receives d loss / d logits for every pair of
    each sequence (0 where masked)."""
    p, (dq, dk, dv, workspace) = prepare_bwd(dout, q, k, v, o, lse, dq=dq, dk=dk, dv=dv, workspace=workspace,
                                             dbias=dbias, **kw)
    rc = lib().attn_bwd(ctypes.byref(p), ctypes.c_void_p(_stream(q.device)))
    if rc:
        raise AttnError("attn_bwd", rc)
    return dq, dk, dv


def workspace_size(dout, q, k, v, o, lse, dbias=None, **kw) -> int:
    """Bytes attn_bwd needs for its workspace (Delta and LSE, and the split
    mode's partial sums when it takes it; keywords as for attn_bwd)."""
    p = bwd_params(dout, q, k, v, o, lse, dout, dout, dout, None, dbias=dbias, **_problem(q, **kw))
    return int(lib().attn_bwd_workspace_size(ctypes.byref(p)))
