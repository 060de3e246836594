"""GPU parity of the HIP path against the fp64 oracle on small problems that
still span several tiles and ragged tails: every head dim built, windows of
every kind (none, causal sentinel, numeric top-left / bottom-right, negative,
empty, one-key), both diagonals, seqlen_q != seqlen_k both ways, packed
sequences with empty ones, strided layouts, scale 0 and negative, run-to-run
determinism, and guard memory around outputs."""
import pytest
import torch

from parity_util import INF, TOL, Case, max_err, say
from oracle import oracle as orc
from scaled_dot_product_20_amd import workloads as wl
from scaled_dot_product_20_amd import binding as bd

pytestmark = pytest.mark.gpu

WINDOWS = [
    ((INF, INF), "top_left"),
    ((INF, 0), "top_left"),        # causal sentinel
    ((INF, 0), "bottom_right"),    # sentinel: never shifted
    ((16, 0), "bottom_right"),
    ((37, 5), "top_left"),
    ((-3, 8), "top_left"),         # negative left bound
    ((5, -2), "bottom_right"),     # negative right bound
    ((-3, 1), "top_left"),         # empty window
    ((0, 0), "top_left"),          # one key
]
SHAPES = [(1, 1), (17, 17), (63, 65), (64, 64), (127, 129), (129, 127), (300, 200), (200, 300)]


# Small problems take the backward's split mode by default; each of these
# sweeps also runs with it switched off, so both paths see every window.
SPLIT = [True, False]


@pytest.mark.parametrize("split", SPLIT)
@pytest.mark.parametrize("D", [64, 80, 128])
@pytest.mark.parametrize("sq,sk", SHAPES)
def test_dense_bf16_windows(D, sq, sk, split):
    for i, (window, diag) in enumerate(WINDOWS):
        Case(B=2, H=2, Sq=sq, Sk=sk, D=D, window=window, diag=diag, seed=100 + i, split=split).check()


@pytest.mark.parametrize("split", SPLIT)
@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("D", [64, 80, 128])
def test_dense_other_dtypes(dtype, D, split):
    for i, (sq, sk) in enumerate([(65, 65), (130, 97)]):
        for j, (window, diag) in enumerate(WINDOWS[:5]):
            Case(B=1, H=3, Sq=sq, Sk=sk, D=D, dtype=dtype, window=window, diag=diag,
                 seed=200 + 10 * i + j, split=split).check()


@pytest.mark.parametrize("split", SPLIT)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("D", [32, 48, 96])
def test_more_head_dims(dtype, D, split):
    """Head dims 32, 48 and 96: dense problems spanning several tiles with
    ragged ends, under the no-mask, causal, numeric and empty windows, and a
    packed one with empty sequences."""
    for i, (sq, sk) in enumerate([(129, 127), (300, 333)]):
        for j, (window, diag) in enumerate([((INF, INF), "top_left"), ((INF, 0), "bottom_right"),
                                            ((40, 7), "bottom_right"), ((-3, 1), "top_left")]):
            Case(B=2, H=2, Sq=sq, Sk=sk, D=D, dtype=dtype, window=window, diag=diag,
                 seed=900 + 10 * i + j, split=split).check()
    Case(layout="thd", H=2, D=D, dtype=dtype, window=(64, 0), diag="bottom_right",
         lens_q=[100, 0, 37, 260], lens_k=[150, 10, 37, 300], seed=950, split=split).check()


def test_tiny_fp32_config():
    """1 x 2 heads x 128 x 64, fp32, no mask, scale 1/8 (the tiny check)."""
    Case(B=1, H=2, Sq=128, D=64, dtype=torch.float32, scale=0.125, seed=1).check()


@pytest.mark.parametrize("dtype,D,B,H,S", [(torch.float32, 64, 1, 2, 128), (torch.bfloat16, 128, 1, 2, 1000),
                                           (torch.float16, 80, 2, 3, 300),
                                           # mid-size grids over long axes: 128 dK/dV blocks at D = 64,
                                           # 64 at D = 128
                                           (torch.bfloat16, 64, 1, 8, 2048), (torch.bfloat16, 128, 1, 2, 4096)])
def test_split_mode_plan_and_bits(dtype, D, B, H, S):
    """Small problems run the backward in split mode: the plan lists the
    preprocess and one grid of split dK/dV and dQ copies (in fp32 each
    block's last copy sums the partials, in fp16 / bf16 a reduction grid
    follows), the workspace holds the partial sums and the arrival counters,
    and the results are run-to-run identical (also on a reused workspace,
    whose counters the last arrivals reset, and by stage calls) and within
    the oracle's bounds, next to the unsplit path's."""
    c = Case(B=B, H=H, Sq=S, D=D, dtype=dtype, seed=15)
    q, k, v, do = (t.cuda() for t in c.cpu)
    o, lse = bd.attn_fwd(q, k, v, scale=c.scale)
    p, ws_t = bd.prepare_bwd(do, q, k, v, o, lse, scale=c.scale)
    names = [n for n, _, _ in bd.plan("attn_bwd", p)]
    if dtype == torch.float32:
        one, want = "attn_bwd_split_kernel", ["attn_bwd_pre_kernel", "attn_bwd_split_kernel"]
    else:
        one = "attn_bwd_split16_kernel"
        want = ["attn_bwd_pre_kernel", one, "attn_bwd_reduce_kernel"]
    assert names == want, names
    p0, _ = bd.prepare_bwd(do, q, k, v, o, lse, scale=c.scale, split=False)
    assert one not in [n for n, _, _ in bd.plan("attn_bwd", p0)]
    outs = ws_t[:3]
    bd.launch("attn_bwd", p)
    first = [t.clone() for t in outs]
    # The same workspace again, by stages: separate split dK/dV and dQ
    # grids, then both in one grid.
    for t in outs:
        t.fill_(7)
    bd.launch("attn_bwd_dkdv", p)
    bd.launch("attn_bwd_dq", p)
    second = [t.clone() for t in outs]
    for t in outs:
        t.fill_(7)
    bd.launch("attn_bwd_dkdv_dq", p)
    torch.cuda.synchronize()
    for x, y, z in zip(first, second, outs):
        assert torch.equal(x, y) and torch.equal(x, z)
    ws = bd.workspace_size(do, q, k, v, o, lse, scale=c.scale)
    ws0 = bd.workspace_size(do, q, k, v, o, lse, scale=c.scale, split=False)
    assert ws > ws0
    a = bd.attn_bwd(do, q, k, v, o, lse, scale=c.scale)
    b = bd.attn_bwd(do, q, k, v, o, lse, scale=c.scale)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    c.check()
    Case(B=B, H=H, Sq=S, D=D, dtype=dtype, seed=15, split=False).check()


@pytest.mark.parametrize("dtype,D,B,H,S,window", [(torch.bfloat16, 128, 1, 2, 700, (INF, INF)),
                                                  (torch.float16, 64, 1, 3, 513, (INF, 0)),
                                                  (torch.bfloat16, 96, 2, 1, 300, (2000, 3000)),
                                                  (torch.float32, 64, 1, 2, 128, (INF, INF)),
                                                  (torch.float32, 48, 2, 1, 300, (INF, 0)),
                                                  (torch.float32, 32, 1, 2, 77, (5, 9))])
def test_small_forward_split_grid(dtype, D, B, H, S, window):
    """A small forward grid runs on key-split workgroups (fp16 / bf16: the
    whole ping-pong grid on the split kernel when it has at most a quarter
    as many 256-row blocks as CUs; fp32 at head_dim <= 64: 64-row workgroups
    over two key halves when at most half as many as CUs), and
    ATTN_FLAG_NO_SPLIT keeps the plain grid: plans, run-to-run bits, and
    both paths against the oracle."""
    c = Case(B=B, H=H, Sq=S, D=D, dtype=dtype, window=window, seed=16)
    q, k, v, _ = (t.cuda() for t in c.cpu)
    kw = dict(scale=c.scale, window=window, diag="top_left", cu_seqlens_q=None, cu_seqlens_k=None,
              max_seqlen_q=None, max_seqlen_k=None)
    o, lse = bd.attn_fwd(q, k, v, scale=c.scale, window=window)
    plans = {}
    for split in (True, False):
        p = bd.fwd_params(q, k, v, o, lse, split=split, **kw)
        plans[split] = [n for n, _, _ in bd.plan("attn_fwd", p)]
    if dtype == torch.float32:
        assert plans[True] == ["attn_fwd_ks_kernel"] and plans[False] == ["attn_fwd_kernel"], plans
    else:
        assert plans[True] == ["attn_fwd16split_kernel"] and plans[False] == ["attn_fwd16pp_kernel"], plans
    o2, lse2 = bd.attn_fwd(q, k, v, scale=c.scale, window=window)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    c.check(bwd=False)
    Case(B=B, H=H, Sq=S, D=D, dtype=dtype, window=window, seed=16, split=False).check(bwd=False)


@pytest.mark.parametrize("D", [80, 128])
@pytest.mark.parametrize("window,diag", [((5, 0), "bottom_right"), ((INF, 0), "top_left"),
                                         ((INF, INF), "top_left"), ((1 << 30, 0), "bottom_right"),
                                         ((0, 0), "top_left")])
@pytest.mark.parametrize("split", SPLIT)
def test_packed_varlen(D, window, diag, split):
    lens_q = [37, 0, 130, 1, 64, 5, 200]
    lens_k = [50, 3, 129, 0, 64, 70, 260]
    Case(layout="thd", H=3, D=D, window=window, diag=diag, lens_q=lens_q, lens_k=lens_k, seed=7,
         split=split).check()


def test_packed_varlen_fp16():
    Case(layout="thd", H=2, D=64, dtype=torch.float16, window=(9, 3), diag="bottom_right",
         lens_q=[70, 129, 0, 2], lens_k=[90, 100, 5, 40], seed=8).check()


def test_bshd_strides():
    Case(B=2, H=3, Sq=150, Sk=190, D=128, window=(INF, 0), diag="top_left", bshd=True, seed=9).check()
    Case(B=2, H=2, Sq=100, Sk=100, D=80, dtype=torch.float16, bshd=True, seed=10).check()


def test_dout_strides_differ_from_out():
    """dO addressed with its own strides (the bwd fix of the AOTriton 0.14b notes)."""
    from scaled_dot_product_20_amd import binding as bd
    c = Case(B=2, H=3, Sq=96, D=64, window=(20, 0), diag="bottom_right", seed=11)
    q, k, v, do = (t.cuda() for t in c.cpu)
    o, lse = bd.attn_fwd(q, k, v, scale=c.scale, window=c.window, diag=c.diag)
    do_bshd = do.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert do_bshd.stride() != o.stride()
    dq, dk, dv = bd.attn_bwd(do_bshd, q, k, v, o, lse, scale=c.scale, window=c.window, diag=c.diag)
    ref = c.oracle()
    tol = 2 * TOL[c.dtype]
    max_err("dq", dq, ref["dq"], tol)
    max_err("dk", dk, ref["dk"], tol)
    max_err("dv", dv, ref["dv"], tol)


@pytest.mark.parametrize("scale", [0.0, -0.3, 1.7])
def test_scale_values(scale):
    Case(B=1, H=2, Sq=100, Sk=140, D=64, window=(30, 10), diag="bottom_right", scale=scale, seed=12).check()
    Case(B=1, H=2, Sq=64, D=128, dtype=torch.float32, scale=scale, seed=13).check()


def test_deterministic_bitwise():
    for dtype in (torch.bfloat16, torch.float32):
        c = Case(B=2, H=4, Sq=257, D=64, dtype=dtype, window=(INF, 0), seed=14)
        a = c.gpu()
        b = c.gpu()
        for n in a:
            assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("kw", [
    dict(B=1, H=2, Sq=0, Sk=50), dict(B=2, H=1, Sq=33, Sk=0), dict(B=2, H=1, Sq=0, Sk=0),
    dict(B=0, H=2, Sq=10, Sk=20),
    dict(layout="thd", H=3, lens_q=[0], lens_k=[0]),
    dict(layout="thd", H=2, lens_q=[0, 0], lens_k=[5, 0]),
    dict(layout="thd", H=2, lens_q=[3, 0], lens_k=[0, 0]),
], ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_zero_size_problems(kw, dtype, D):
    """Problems with no query rows, no keys or no elements at all (the empty
    tensors' pointers are NULL): the calls succeed, and whatever has rows
    comes out as the oracle's fully masked result (O = 0, LSE = +inf,
    gradients 0)."""
    Case(D=D, dtype=dtype, seed=16, **kw).check()


def test_guard_memory_untouched():
    """Outputs written only inside their rows and head_dim columns (the early
    exit fix bounded by the head dim, AOTriton 0.15b), and no LSE write past
    the packed rows (the +inf LSE fix, AOTriton 0.14b)."""
    from scaled_dot_product_20_amd import binding as bd
    c = Case(layout="thd", H=2, D=80, window=(-3, 1), diag="top_left",  # every row empty
             lens_q=[40, 0, 33], lens_k=[10, 20, 0], seed=15)
    q, k, v, do = (t.cuda() for t in c.cpu)
    kw = c.kw_gpu("cuda")
    T, H, D = q.shape
    obuf = torch.full((T, H, 96), 7.0, dtype=q.dtype, device="cuda")
    o = obuf[..., :80]
    lbuf = torch.full((H * T + 64,), 5.0, dtype=torch.float32, device="cuda")
    lse = lbuf[: H * T].view(H, T)
    bd.attn_fwd(q, k, v, out=o, lse=lse, **kw)
    torch.cuda.synchronize()
    assert torch.all(obuf[..., 80:] == 7.0)
    assert torch.all(lbuf[H * T:] == 5.0)
    assert torch.all(o == 0) and torch.all(torch.isinf(lse)) and torch.all(lse > 0)
    gbuf = torch.full((T, H, 96), 3.0, dtype=q.dtype, device="cuda")
    dq = gbuf[..., :80]
    bd.attn_bwd(do, q, k, v, o, lse, dq=dq, **kw)
    torch.cuda.synchronize()
    assert torch.all(gbuf[..., 80:] == 3.0) and torch.all(dq == 0)


def test_multi_head_batch_mix():
    Case(B=3, H=5, Sq=190, Sk=70, D=128, window=(INF, 40), diag="top_left", seed=16).check()
    Case(B=3, H=5, Sq=70, Sk=190, D=64, window=(10, 10), diag="bottom_right", seed=17).check()


def test_zero_length_dense():
    from scaled_dot_product_20_amd import binding as bd
    q = torch.randn(1, 2, 5, 64, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = bd.attn_fwd(q, k, k)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isposinf(lse))
    say("zero-length keys ok")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("window,diag", [((1100, -40), "top_left"), ((-30, 1200), "bottom_right"),
                                         ((700, 400), "bottom_right"), ((INF, 0), "bottom_right")])
def test_wide_windows(D, window, diag):
    """Bands at least 1024 keys wide, which run on the 256-row forward kernel:
    tiles cut by the band on both sides, waves whose band misses whole tiles,
    ragged ends on both axes."""
    Case(B=1, H=2, Sq=1300, Sk=1500, D=D, window=window, diag=diag, seed=400 + D).check()
    Case(B=1, H=1, Sq=1700, Sk=1100, D=D, dtype=torch.float16, window=window, diag=diag, seed=500 + D).check()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("shape", ["dense", "dense_window", "packed", "d64"])
def test_dkdv_dq_call_equals_separate_calls(dtype, shape):
    """attn_bwd_dkdv_dq (one grid of dK/dV and dQ workgroups at head_dim 128)
    gives exactly what attn_bwd_dkdv then attn_bwd_dq give, and matches the
    oracle."""
    if shape == "dense":
        c = Case(B=2, H=3, Sq=333, Sk=290, D=128, dtype=dtype, seed=600)
    elif shape == "dense_window":
        c = Case(B=1, H=2, Sq=300, Sk=420, D=128, dtype=dtype, window=(70, -5), diag="bottom_right", seed=601)
    elif shape == "packed":
        c = Case(layout="thd", H=2, D=128, dtype=dtype, window=(INF, 0), lens_q=[37, 0, 200, 1, 65],
                 lens_k=[50, 3, 129, 0, 64], seed=602)
    else:
        c = Case(B=2, H=2, Sq=200, D=64, dtype=dtype, seed=603)
    dev = "cuda"
    q, k, v, do = (t.to(dev) for t in c.cpu)
    kw = c.kw_gpu(dev)
    o, lse = bd.attn_fwd(q, k, v, **kw)
    outs = []
    for calls in (("attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq"),
                  ("attn_bwd_preprocess", "attn_bwd_dkdv_dq")):
        bp, keep = bd.prepare_bwd(do, q, k, v, o, lse, **kw)
        for name in calls:
            bd.launch(name, bp)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in keep[:3]])
    for name, a, b in zip(("dq", "dk", "dv"), *outs):
        assert torch.equal(a, b), name
    ref = c.oracle()
    tol = TOL[dtype] * 2 * c.tol_factor()
    for name, got in zip(("dq", "dk", "dv"), outs[1]):
        max_err(name, got, ref[name], tol)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("window,diag", [((INF, INF), "top_left"), ((INF, 0), "bottom_right"), ((1200, 3), "top_left")])
def test_forward_grid_tail(D, window, diag):
    """A wide-band forward whose 256-row grid has one full round plus a few
    blocks: those rows run on the split tail kernel (64-row workgroups, key
    tiles halved and merged).  A round is one workgroup per CU, two at
    head_dim 64.  Sq = 1000 gives 4 blocks per head; heads = round / 4 + 1
    makes a round + 4 blocks, 4 of them in the tail (the last heads)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    H = cus * (2 if D <= 64 else 1) // 4 + 1
    Case(B=1, H=H, Sq=1000, Sk=1100, D=D, window=window, diag=diag, seed=700 + D).check(bwd=False)


def ks_rule(nblk, D, Sk, window):
    """The key-split tail the forward's launch takes with a workspace, from
    its documented rule: (ping-pong blocks, tail blocks r, parts np) when
    the last round (pp = 1 workgroup per CU, 2 at head_dim <= 64) of a grid
    of nblk 256-row blocks is partly filled with r blocks, np = min(8, round
    / r, band keys / F) is at least 2 (F = 512 at head_dim <= 64, else
    1024), r np fits the slots (one round of a 256-CU device), and the grid
    has more than a quarter as many blocks as CUs or r np covers the CUs;
    else None."""
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    ppc = 2 if D <= 64 else 1
    cus = cu * ppc
    kb = Sk if INF in window else min(Sk, window[0] + window[1] + 256)
    r = nblk % cus
    npart = min(8, cus // r, kb // (512 if D <= 64 else 1024)) if r else 0
    if npart >= 2 and r * npart <= 256 * ppc and (4 * nblk > cu or r * npart >= cu):
        return nblk - r, r, npart
    return None


@pytest.mark.parametrize("dtype,D,H,Sq,Sk,window,diag,tail_heads", [
    (torch.bfloat16, 128, 5, 4096, 4096, (INF, INF), "top_left", False),
    (torch.bfloat16, 128, 5, 4096, 4096, (INF, 0), "top_left", False),
    (torch.float16, 128, 5, 4096, 4096, (1500, 1500), "bottom_right", False),
    (torch.float16, 64, 560, 256, 2048, (INF, INF), "top_left", True),
    (torch.bfloat16, 128, 300, 256, 4096, (INF, INF), "top_left", True),
    (torch.bfloat16, 96, 300, 256, 4096, (INF, 0), "bottom_right", True),
    (torch.bfloat16, 128, 2, 8192, 8192, (INF, INF), "top_left", False),   # small grid, parts cover the CUs
    (torch.float16, 64, 32, 1024, 1024, (INF, 0), "top_left", False)])      # two parts of 512 keys
def test_forward_key_split_tail(dtype, D, H, Sq, Sk, window, diag, tail_heads):
    """With a workspace, the blocks of a partly filled last round of the
    ping-pong forward run as np key-split workgroups each (after the
    ping-pong grid, if any), whose partials a merge grid combines; without
    one, the earlier tail.
    Plans and grid sizes, run-to-run bits, and both paths against the
    oracle: every head, or (tail_heads, one 256-row block per head) the
    tail's heads and the ping-pong grid's first and last."""
    nq = -(-Sq // 256)
    nblk = nq * H
    rule = ks_rule(nblk, D, Sk, window)
    say(f"case key-split tail dtype={dtype} D={D} H={H} Sq={Sq} Sk={Sk} window={window} diag={diag} rule={rule}")
    if rule is None:
        pytest.skip("this device's CU count gives no key-split tail for the shape")
    nm, r, npart = rule
    q, k, v = wl.draw([(1, H, Sq, D), (1, H, Sk, D), (1, H, Sk, D)], 900 + D + H, dtype)
    gq, gk, gv = (t.cuda() for t in (q, k, v))
    kw = dict(scale=D ** -0.5, window=window, diag=diag, cu_seqlens_q=None, cu_seqlens_k=None,
              max_seqlen_q=None, max_seqlen_k=None)
    outs = {}
    for use_ws in (True, False):
        o = torch.empty_like(gq)
        lse = torch.empty(1, H, Sq, dtype=torch.float32, device="cuda")
        if use_ws:
            p, ws = bd.prepare_fwd(gq, gk, gv, o, lse, **kw)
            assert ws is not None
        else:
            p, ws = bd.fwd_params(gq, gk, gv, o, lse, **kw), None
        pl = bd.plan("attn_fwd", p)
        names = [n for n, _, _ in pl]
        say(f"  workspace={use_ws} plan {pl}")
        if use_ws:
            assert names == ["attn_fwd16pp_kernel"] * (nm > 0) + ["attn_fwd16ppks_kernel", "attn_fwd16ksmerge_kernel"]
            assert pl[-2][1] == r * npart and pl[-1][1] == 8 * -(-D // 32) * r and (nm == 0 or pl[0][1] == nm), pl
        else:
            assert "attn_fwd16ppks_kernel" not in names
        bd.launch("attn_fwd", p)
        torch.cuda.synchronize()
        o1, lse1 = o.clone(), lse.clone()
        bd.launch("attn_fwd", p)
        torch.cuda.synchronize()
        assert torch.equal(o, o1) and torch.equal(lse, lse1), "two runs differ"
        outs[use_ws] = (o1, lse1)
        del ws
    if tail_heads:
        assert nq == 1
        hs = sorted({0, nm - 1} | set(range(nm, nblk)))
    else:
        hs = list(range(H))
    ro, rl = orc.fwd(q[:, hs].contiguous(), k[:, hs].contiguous(), v[:, hs].contiguous(), scale=D ** -0.5,
                     window=window, diag=diag)
    for use_ws, (o, lse) in outs.items():
        eo = max_err("O", o[:, hs], ro, TOL[dtype])
        el = max_err("LSE", lse[:, hs], rl, TOL[dtype], inf_exact=True)
        say(f"  workspace={use_ws} heads {len(hs)}: O {eo:.2e} LSE {el:.2e}")


def test_forward_key_split_tail_varlen():
    """Packed sequences of lengths 4096, 3000, 70, 0 and 2500 (one head,
    head_dim 80): 80 ragged 256-row blocks, all in the key-split tail on a
    256-CU device; the 70-row sequence's block has two key tiles, so one of
    its three parts has none.  Plan, then both runs against the oracle."""
    lens = [4096, 3000, 70, 0, 2500]
    c = Case(layout="thd", B=len(lens), H=1, D=80, lens_q=lens, lens_k=lens, seed=910)
    rule = ks_rule(len(lens) * 16, 80, max(lens), (INF, INF))
    if rule is None:
        pytest.skip("this device's CU count gives no key-split tail for the shape")
    q, k, v, _ = (t.cuda() for t in c.cpu)
    o = torch.empty_like(q)
    lse = torch.empty(1, q.shape[0], dtype=torch.float32, device="cuda")
    p, ws = bd.prepare_fwd(q, k, v, o, lse, **{kk: vv for kk, vv in c.kw_gpu("cuda").items() if kk != "split"})
    pl = bd.plan("attn_fwd", p)
    say(f"  plan {pl}")
    assert [n for n, _, _ in pl] == ["attn_fwd16ppks_kernel", "attn_fwd16ksmerge_kernel"], pl
    assert pl[0][1] == rule[1] * rule[2] and pl[1][1] == 8 * 3 * rule[1], pl
    c.check(bwd=False)


@pytest.mark.parametrize("dtype,D,sq,sk,window,diag", [
    (torch.bfloat16, 128, 333, 333, (INF, INF), "top_left"),
    (torch.bfloat16, 64, 200, 300, (40, 7), "bottom_right"),
    (torch.float16, 80, 130, 130, (INF, 0), "top_left"),
    (torch.float32, 64, 100, 100, (INF, INF), "top_left"),
])
def test_negative_row_strides(dtype, D, sq, sk, window, diag):
    """Every operand stored with its rows last to first (row stride -D, base
    pointer at row 0, the highest address): attn_fwd, attn_bwd and
    attn_bwd_dkdv_dq give the same bits as with the rows in order, since only
    the addressing differs."""
    import ctypes
    c = Case(B=2, H=3, Sq=sq, Sk=sk, D=D, dtype=dtype, window=window, diag=diag, seed=700)
    q, k, v, do = (t.cuda() for t in c.cpu)
    kw = c.kw_gpu("cuda")
    o, lse = bd.attn_fwd(q, k, v, **kw)
    dq, dk, dv = bd.attn_bwd(do, q, k, v, o, lse, **kw)

    def rev(t):  # rows-reversed storage, base pointer of logical row 0, strides
        st = t.flip(2).contiguous()
        B, H, S, _ = t.shape
        return st, st.data_ptr() + (S - 1) * D * st.element_size(), bd._I64x3(H * S * D, S * D, -D)

    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    (qs, qb, qst), (ks, kb, kst), (vs, vb, vst) = rev(q), rev(k), rev(v)
    os_, ob, ost = rev(torch.zeros_like(o))
    lse_n = torch.empty_like(lse)
    p = bd.fwd_params(q, k, v, o, lse_n, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                      max_seqlen_k=None, **kw)
    p.q, p.k, p.v, p.o = qb, kb, vb, ob
    p.q_stride, p.k_stride, p.v_stride, p.o_stride = qst, kst, vst, ost
    assert bd.lib().attn_fwd(ctypes.byref(p), stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(os_.flip(2), o), "o"
    assert torch.equal(lse_n, lse), "lse"

    for entry in ("attn_bwd", "attn_bwd_dkdv_dq"):
        (dos, dob, dost) = rev(do)
        outs = [rev(torch.zeros_like(t)) for t in (q, k, v)]
        bp = bd.BwdParams()
        bp.fwd = p
        bp.dout, bp.do_stride = dob, dost
        (bp.dq, bp.dq_stride), (bp.dk, bp.dk_stride), (bp.dv, bp.dv_stride) = ((b, st) for _, b, st in outs)
        need = int(bd.lib().attn_bwd_workspace_size(ctypes.byref(bp)))
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        bp.workspace, bp.workspace_bytes = ws.data_ptr(), ws.numel()
        if entry == "attn_bwd":
            assert bd.lib().attn_bwd(ctypes.byref(bp), stream) == 0
        else:
            assert bd.lib().attn_bwd_preprocess(ctypes.byref(bp), stream) == 0
            assert bd.lib().attn_bwd_dkdv_dq(ctypes.byref(bp), stream) == 0
        torch.cuda.synchronize()
        for name, (st, _, _), ref in zip(("dq", "dk", "dv"), outs, (dq, dk, dv)):
            assert torch.equal(st.flip(2), ref), f"{entry} {name}"

@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float16, 80), (torch.float32, 64)])
def test_packed_lse_th_layout(dtype, D):
    """Packed LSE stored [T, H] (ATTN_FLAG_LSE_TH): the forward writes the
    transpose of its [H, T] result, the backward reads it and returns the
    same gradients, bit for bit; the [H, T] run itself matches the oracle."""
    c = Case(layout="thd", H=3, D=D, dtype=dtype, window=(64, 0), diag="bottom_right",
             lens_q=[37, 0, 130, 64, 1], lens_k=[50, 3, 129, 64, 0], seed=960)
    dev = "cuda"
    q, k, v, do = (t.to(dev) for t in c.cpu)
    kw = c.kw_gpu(dev)
    o1, l1 = bd.attn_fwd(q, k, v, **kw)
    o2, l2 = bd.attn_fwd(q, k, v, lse_layout="th", **kw)
    assert l2.shape == (q.shape[0], q.shape[1])
    assert torch.equal(o1, o2)
    assert torch.equal(l1.t(), l2)
    g1 = bd.attn_bwd(do, q, k, v, o1, l1, **kw)
    g2 = bd.attn_bwd(do, q, k, v, o2, l2, lse_layout="th", **kw)
    for name, a, b in zip(("dq", "dk", "dv"), g1, g2):
        assert torch.equal(a, b), name
    c.check(dev=dev)


def _used_rows_case(layout, dtype, D, window, diag, seed):
    """A packed problem of `used` rows per sequence (the oracle checks it),
    and the same rows spread into larger per-sequence ranges (packed) or a
    padded [B, H, S, D] tensor, with NaN in every row past the used ones."""
    used_q, used_k = [37, 0, 130, 64, 9], [50, 3, 129, 64, 0]
    alloc_q, alloc_k = [45, 7, 130, 100, 9], [60, 3, 200, 64, 12]
    c = Case(layout="thd", H=2, D=D, dtype=dtype, window=window, diag=diag, lens_q=used_q, lens_k=used_k, seed=seed)
    dev = "cuda"
    comp = [t.to(dev) for t in c.cpu]  # q, k, v, do packed over the used rows
    B, H = len(used_q), 2

    def spread(t, used, alloc):
        if layout == "thd":
            out = torch.full((sum(alloc), H, D), float("nan"), dtype=dtype, device=dev)
        else:
            out = torch.full((B, H, max(alloc), D), float("nan"), dtype=dtype, device=dev)
        src = dst = 0
        for b in range(B):
            if layout == "thd":
                out[dst:dst + used[b]] = t[src:src + used[b]]
                dst += alloc[b]
            else:
                out[b, :, :used[b]] = t[src:src + used[b]].permute(1, 0, 2)
            src += used[b]
        return out

    full = [spread(t, used_q if i in (0, 3) else used_k, alloc_q if i in (0, 3) else alloc_k)
            for i, t in enumerate(comp)]
    kw = dict(scale=c.scale, window=window, diag=diag,
              seqused_q=torch.tensor(used_q, dtype=torch.int32, device=dev),
              seqused_k=torch.tensor(used_k, dtype=torch.int32, device=dev))
    if layout == "thd":
        kw.update(cu_seqlens_q=torch.from_numpy(wl_prefix(alloc_q)).to(dev),
                  cu_seqlens_k=torch.from_numpy(wl_prefix(alloc_k)).to(dev),
                  max_seqlen_q=max(alloc_q), max_seqlen_k=max(alloc_k))
    return c, comp, full, kw, (used_q, used_k, alloc_q, alloc_k)


def wl_prefix(lengths):
    from scaled_dot_product_20_amd import workloads as wls
    return wls.prefix(lengths)


@pytest.mark.parametrize("layout", ["thd", "bhsd"])
@pytest.mark.parametrize("dtype,D,window,diag", [
    (torch.bfloat16, 128, (INF, INF), "top_left"),
    (torch.float16, 64, (40, 0), "bottom_right"),
    (torch.float32, 80, (INF, 0), "top_left"),
    (torch.bfloat16, 48, (1 << 30, 3), "bottom_right"),
])
@pytest.mark.parametrize("split", SPLIT)
def test_seqused_rows(layout, dtype, D, window, diag, split):
    """seqused_q / seqused_k: sequence b computes on its first used rows only
    (bottom-right windows shift by the used lengths), as the compact packed
    problem of those rows, which matches the oracle: bit for bit, except for
    the gradients in the backward's split mode, whose partial sums group the
    tiles by the grid (which differs between the two layouts) and so are
    held to the gradients' bound instead.  Rows past the used ones (NaN in
    the inputs) come out as fully masked rows: O = 0, LSE = +inf, dQ = dK =
    dV = 0."""
    c, comp, full, kw, (uq, uk, aq, ak) = _used_rows_case(layout, dtype, D, window, diag, seed=970)
    c.split = split
    kw["split"] = split
    dev = "cuda"
    o_c, l_c = bd.attn_fwd(*comp[:3], **c.kw_gpu(dev))
    g_c = bd.attn_bwd(comp[3], *comp[:3], o_c, l_c, **c.kw_gpu(dev))
    o_f, l_f = bd.attn_fwd(*full[:3], **kw)
    g_f = bd.attn_bwd(full[3], *full[:3], o_f, l_f, **kw)

    def same_grad(name, got, want):
        if split:
            max_err(name, got, want.double().cpu().numpy(), 2 * TOL[dtype] * c.tol_factor())
        else:
            assert torch.equal(got, want), name
    H = comp[0].shape[1]
    sq_c = sk_c = sq_f = sk_f = 0
    for b in range(len(uq)):
        def rows_f(t, start, b, n, alloc):
            return t[start:start + alloc] if layout == "thd" else t[b].permute(1, 0, 2)[:alloc]
        of = rows_f(o_f, sq_f, b, uq[b], aq[b])
        assert torch.equal(of[:uq[b]], o_c[sq_c:sq_c + uq[b]]), ("o", b)
        assert torch.count_nonzero(of[uq[b]:]) == 0, ("o pad", b)
        lf = l_f[:, sq_f:sq_f + aq[b]] if layout == "thd" else l_f[b, :, :aq[b]]
        assert torch.equal(lf[:, :uq[b]], l_c[:, sq_c:sq_c + uq[b]]), ("lse", b)
        assert bool(torch.all(lf[:, uq[b]:] == float("inf"))), ("lse pad", b)
        dqf = rows_f(g_f[0], sq_f, b, uq[b], aq[b])
        same_grad(f"dq {b}", dqf[:uq[b]], g_c[0][sq_c:sq_c + uq[b]])
        assert torch.count_nonzero(dqf[uq[b]:]) == 0, ("dq pad", b)
        for name, gf, gc in (("dk", g_f[1], g_c[1]), ("dv", g_f[2], g_c[2])):
            kf = rows_f(gf, sk_f, b, uk[b], ak[b])
            same_grad(f"{name} {b}", kf[:uk[b]], gc[sk_c:sk_c + uk[b]])
            assert torch.count_nonzero(kf[uk[b]:]) == 0, (name + " pad", b)
        sq_c += uq[b]
        sk_c += uk[b]
        sq_f += aq[b]
        sk_f += ak[b]
    c.check(dev=dev)


def test_forward_key_split_tail_repacked():
    """A repacked call (head_dim 100, run at 128 on zero-padded copies) with
    the key-split part of its workspace after the copies: the plan is the
    copy-in, the key-split grid and its merge, the copy-out; O and LSE
    against the oracle at head_dim 100."""
    H, S, D = 5, 4096, 100
    rule = ks_rule(H * S // 256, 128, S, (INF, INF))
    say(f"case key-split tail repacked H={H} S={S} D={D} rule={rule}")
    if rule is None:
        pytest.skip("this device's CU count gives no key-split tail for the shape")
    q, k, v = wl.draw([(1, H, S, D)] * 3, 920, torch.bfloat16)
    gq, gk, gv = (t.cuda() for t in (q, k, v))
    o = torch.empty_like(gq)
    lse = torch.empty(1, H, S, dtype=torch.float32, device="cuda")
    kw = dict(scale=D ** -0.5, window=(INF, INF), diag="top_left", cu_seqlens_q=None, cu_seqlens_k=None,
              max_seqlen_q=None, max_seqlen_k=None)
    p, ws = bd.prepare_fwd(gq, gk, gv, o, lse, **kw)
    pl = bd.plan("attn_fwd", p)
    say(f"  plan {pl}")
    assert [n for n, _, _ in pl] == ["attn_repack_kernel", "attn_fwd16ppks_kernel", "attn_fwd16ksmerge_kernel",
                                     "attn_repack_kernel"], pl
    bd.launch("attn_fwd", p)
    torch.cuda.synchronize()
    ro, rl = orc.fwd(q, k, v, scale=D ** -0.5)
    say(f"  O {max_err('O', o, ro, TOL[torch.bfloat16]):.2e} "
        f"LSE {max_err('LSE', lse, rl, TOL[torch.bfloat16], inf_exact=True):.2e}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("kind", ["large_logits", "growing_scores", "negative_scale"])
def test_pingpong_rescale_paths(dtype, kind):
    """The ping-pong forward computes a tile's row max only when a lane's
    sum of P against the row's current reference max passes 2^8 (or the row
    has none yet), then raises the max and recomputes P.  These inputs take
    that path: logits of tens (scale 1.7 at head_dim 128: sums overflow to
    inf before the rescale), keys whose scores grow along the sequence (the
    max rises tile after tile), and a negative scale.  O and LSE against the
    oracle in the wide band the ping-pong kernel runs, and the backward
    where the inputs stay within the tolerance model (the growing keys reach
    |K| near 1000, and dQ's error from rounding dS to 16 bits grows with
    |K|, which the N(0, 1) bounds do not cover)."""
    H, S, D = 2, 700, 128
    q, k, v, do = wl.draw([(1, H, S, D)] * 4, 930, torch.float32)
    scale = D ** -0.5
    if kind == "large_logits":
        scale = 1.7
    elif kind == "growing_scores":
        k = k * (1.0 + torch.arange(S, dtype=torch.float32).view(1, 1, S, 1) / 64.0)
        q = q.abs()  # with k's first column shifted, the scores of row i grow with j
        k[..., 0] += torch.arange(S, dtype=torch.float32).view(1, 1, S) / 8.0
    else:
        scale = -0.3
    q, k, v, do = (t.to(dtype) for t in (q, k, v, do))
    # Split paths off: the whole grid on the ping-pong kernel, whatever the
    # device's CU count.
    c = Case(B=1, H=H, Sq=S, D=D, dtype=dtype, scale=scale, seed=930, split=False)
    c.cpu = (q, k, v, do)
    pl = bd.plan("attn_fwd", bd.fwd_params(q.cuda(), k.cuda(), v.cuda(), torch.empty_like(q, device="cuda"),
                                           torch.empty(1, H, S, device="cuda"), scale=scale,
                                           window=(INF, INF), diag="top_left", cu_seqlens_q=None,
                                           cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
                                           split=False))
    assert [n for n, _, _ in pl][0] == "attn_fwd16pp_kernel", pl
    c.check(bwd=kind != "growing_scores")
