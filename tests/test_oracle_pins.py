"""Pins of the fp64 CPU oracle against facts that do not come from the oracle.

Each test ties a part of the oracle to something independent of it: the
hand-worked fixtures in ``tests/golden/``, textbook masks built with numpy's
``tril``/``triu``/``eye``, torch's own float64 SDPA and autograd on the CPU,
closed forms (scale 0, constant V, one-key windows), invariants (shifting
every key by one vector, permuting keys, row sums of gradients), finite
differences, and the reduction of the packed layout to dense runs.  A dropped
term, a wrong sign of the diagonal shift, a transposed operand or a wrong
decoder fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc

INF = orc.WINDOW_INF
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _w(x):
    return INF if x == "inf" else int(x)


def band(sq, sk, lo=None, hi=None):
    """Textbook band mask lo <= j - i <= hi via numpy (None = unbounded)."""
    m = np.ones((sq, sk), dtype=bool)
    if hi is not None:
        m &= np.tril(np.ones((sq, sk), dtype=bool), k=hi)
    if lo is not None:
        m &= np.triu(np.ones((sq, sk), dtype=bool), k=lo)
    return m


# ------------------------------------------------------------------ decoders

def test_decode_f16_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).double().numpy()
    got = np.array([orc.decode_f16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_decode_bf16_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([orc.decode_bf16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------------------------ masks

def test_golden_masks():
    for case in json.load(open(GOLDEN))["masks"]:
        got = orc.visible_matrix(case["sq"], case["sk"], _w(case["wl"]), _w(case["wr"]), case["diag"])
        assert np.array_equal(got, np.array(case["visible"], dtype=bool)), case["derivation"]


@pytest.mark.parametrize("sq,sk", [(5, 5), (3, 7), (7, 3), (1, 4), (6, 1)])
def test_mask_special_cases(sq, sk):
    d = sk - sq
    for diag in ("top_left", "bottom_right"):
        # no mask
        assert orc.visible_matrix(sq, sk, INF, INF, diag).all()
        # causal sentinel: lower triangle anchored top-left under both diagonals
        assert np.array_equal(orc.visible_matrix(sq, sk, INF, 0, diag), np.tril(np.ones((sq, sk), bool)))
        # the mirrored sentinel
        assert np.array_equal(orc.visible_matrix(sq, sk, 0, INF, diag), np.triu(np.ones((sq, sk), bool)))
    # one-key windows: (0,0) is the identity, (-t, t) the t-th superdiagonal
    for t in range(-2, 3):
        assert np.array_equal(orc.visible_matrix(sq, sk, -t, t, "top_left"), np.eye(sq, sk, k=t, dtype=bool))
    # bottom-right causal written as a huge numeric window: flash-attention's
    # bottom-right triangle, tril(k = sk - sq)
    big = 1 << 30
    assert np.array_equal(orc.visible_matrix(sq, sk, big, 0, "bottom_right"),
                          np.tril(np.ones((sq, sk), bool), k=d))
    # bottom-right sliding window (w, 0): the last w+1 keys before the shifted diagonal
    for w in (0, 1, 2):
        assert np.array_equal(orc.visible_matrix(sq, sk, w, 0, "bottom_right"), band(sq, sk, d - w, d))
    # an empty window (L + R < 0) masks everything
    assert not orc.visible_matrix(sq, sk, -3, 1, "top_left").any()


def test_bottom_right_equals_top_left_when_square():
    rng = np.random.default_rng(0)
    for _ in range(40):
        s = int(rng.integers(1, 9))
        wl, wr = (int(x) for x in rng.integers(-4, 5, size=2))
        assert np.array_equal(orc.visible_matrix(s, s, wl, wr, "bottom_right"),
                              orc.visible_matrix(s, s, wl, wr, "top_left"))


def test_mask_brute_force_against_band():
    rng = np.random.default_rng(1)
    for _ in range(200):
        sq, sk = (int(x) for x in rng.integers(0, 9, size=2))
        wl = INF if rng.random() < 0.2 else int(rng.integers(-6, 7))
        wr = INF if rng.random() < 0.2 else int(rng.integers(-6, 7))
        diag = "bottom_right" if rng.random() < 0.5 else "top_left"
        shift = (sk - sq) if (diag == "bottom_right" and wl != INF and wr != INF) else 0
        lo = None if wl == INF else -(wl - shift)
        hi = None if wr == INF else wr + shift
        assert np.array_equal(orc.visible_matrix(sq, sk, wl, wr, diag), band(sq, sk, lo, hi))


def test_mask_no_int32_overflow():
    big = INF - 1
    assert orc.visible(0, 5, 3, 1000, big, 0, "bottom_right")
    assert orc.visible(2, 999, 3, 1000, big, big, "bottom_right")
    assert not orc.visible(2, 999, 3, 1000, -big, 0, "bottom_right")


# ------------------------------------------------------------------ forward

def _dense(arr):
    return torch.tensor(arr, dtype=torch.float32)[None, None]


def test_golden_forward():
    for case in json.load(open(GOLDEN))["forward"]:
        q, k, v = _dense(case["q"]), _dense(case["k"]), _dense(case["v"])
        o, lse = orc.fwd(q, k, v, scale=case["scale"], window=(_w(case["wl"]), _w(case["wr"])),
                         diag=case["diag"])
        np.testing.assert_allclose(o[0, 0], np.array(case["o"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, 0], np.array(case["lse"]), rtol=0, atol=1e-12)


def _torch_sdpa(q, k, v, mask, scale):
    """torch float64 SDPA on the rows with at least one visible key."""
    qd, kd, vd = q.double(), k.double(), v.double()
    m = torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=m, scale=scale)
    s = torch.matmul(qd, kd.transpose(-1, -2)) * scale
    s = s.masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


CASES = [
    # sq, sk, D, window, diag
    (9, 9, 4, (INF, INF), "top_left"),
    (9, 9, 8, (INF, 0), "top_left"),
    (6, 11, 4, (2, 1), "bottom_right"),
    (11, 6, 4, (3, 0), "bottom_right"),
    (7, 7, 3, (-1, 3), "top_left"),
    (5, 8, 5, (INF, 2), "top_left"),
    (8, 5, 5, (1, 1), "top_left"),
]


@pytest.mark.parametrize("sq,sk,D,window,diag", CASES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_forward_against_torch(sq, sk, D, window, diag, dtype):
    q, k, v = (t.to(dtype) for t in (torch.randn(2, 3, sq, D), torch.randn(2, 3, sk, D), torch.randn(2, 3, sk, D)))
    scale = 0.7
    o, lse = orc.fwd(q, k, v, scale=scale, window=window, diag=diag)
    mask = orc.visible_matrix(sq, sk, window[0], window[1], diag)
    ro, rl = _torch_sdpa(q, k, v, mask, scale)
    rows = mask.any(axis=1)
    np.testing.assert_allclose(o[:, :, rows], ro[:, :, rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, rows], rl[:, :, rows], rtol=1e-12, atol=1e-12)
    assert np.all(o[:, :, ~rows] == 0.0)
    assert np.all(np.isposinf(lse[:, :, ~rows]))


@pytest.mark.parametrize("window,diag", [((INF, INF), "top_left"), ((INF, 0), "top_left"),
                                          ((2, 1), "bottom_right"), ((-2, 4), "top_left")])
def test_scale_zero_closed_form(window, diag):
    sq, sk, D = 7, 9, 3
    q, k, v = torch.randn(1, 2, sq, D), torch.randn(1, 2, sk, D), torch.randn(1, 2, sk, D)
    o, lse = orc.fwd(q, k, v, scale=0.0, window=window, diag=diag)
    mask = band(sq, sk, *_lohi(sq, sk, window, diag))
    vd = v.double().numpy()
    for i in range(sq):
        n = int(mask[i].sum())
        if n == 0:
            assert np.isposinf(lse[0, :, i]).all() and (o[0, :, i] == 0).all()
            continue
        np.testing.assert_allclose(lse[0, :, i], math.log(n), rtol=0, atol=1e-14)
        np.testing.assert_allclose(o[0, :, i], vd[0][:, mask[i]].mean(axis=1), rtol=0, atol=1e-14)


def _lohi(sq, sk, window, diag):
    wl, wr = window
    shift = (sk - sq) if (diag == "bottom_right" and wl != INF and wr != INF) else 0
    return (None if wl == INF else shift - wl), (None if wr == INF else wr + shift)


def test_constant_v_gives_constant_o():
    sq, sk, D = 6, 10, 4
    q, k = torch.randn(1, 1, sq, D), torch.randn(1, 1, sk, D)
    c = torch.tensor([0.5, -1.25, 3.0, 2.0])
    v = c.expand(1, 1, sk, D).contiguous()
    for window, diag in [((INF, INF), "top_left"), ((3, 0), "bottom_right"), ((INF, 0), "top_left")]:
        o, lse = orc.fwd(q, k, v, scale=1.3, window=window, diag=diag)
        rows = np.isfinite(lse[0, 0])
        np.testing.assert_allclose(o[0, 0, rows], np.broadcast_to(c.numpy(), (rows.sum(), D)), rtol=0, atol=1e-14)


def test_one_key_windows():
    s, D = 8, 5
    q, k, v = torch.randn(1, 1, s, D), torch.randn(1, 1, s, D), torch.randn(1, 1, s, D)
    scale = 0.3
    o, lse = orc.fwd(q, k, v, scale=scale, window=(0, 0))
    qd, kd, vd = q.double().numpy()[0, 0], k.double().numpy()[0, 0], v.double().numpy()[0, 0]
    np.testing.assert_allclose(o[0, 0], vd, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], scale * (qd * kd).sum(axis=1), rtol=1e-14, atol=1e-14)
    for t in (-2, 1, 3):
        o, lse = orc.fwd(q, k, v, scale=scale, window=(-t, t))
        for i in range(s):
            if 0 <= i + t < s:
                np.testing.assert_allclose(o[0, 0, i], vd[i + t], rtol=0, atol=1e-15)
            else:
                assert np.isposinf(lse[0, 0, i]) and (o[0, 0, i] == 0).all()


def test_key_shift_invariance():
    sq, sk, D = 5, 9, 4
    q = torch.randn(1, 2, sq, D)
    k = torch.randint(-8, 8, (1, 2, sk, D)).float() / 4
    v = torch.randn(1, 2, sk, D)
    c = torch.tensor([0.25, -0.5, 1.0, 0.75])
    scale = 0.6
    for window, diag in [((INF, INF), "top_left"), ((2, 1), "bottom_right")]:
        o1, l1 = orc.fwd(q, k, v, scale=scale, window=window, diag=diag)
        o2, l2 = orc.fwd(q, k + c, v, scale=scale, window=window, diag=diag)
        rows = np.isfinite(l1)
        np.testing.assert_allclose(o2[rows], o1[rows], rtol=0, atol=1e-12)
        shift = scale * (q.double().numpy() @ c.double().numpy())
        np.testing.assert_allclose(l2[rows], (l1 + shift)[rows], rtol=0, atol=1e-12)


def test_key_permutation_invariance():
    sq, sk, D = 6, 11, 4
    q, k, v = torch.randn(1, 2, sq, D), torch.randn(1, 2, sk, D), torch.randn(1, 2, sk, D)
    perm = torch.randperm(sk)
    o1, l1 = orc.fwd(q, k, v, scale=0.5)
    o2, l2 = orc.fwd(q, k[:, :, perm], v[:, :, perm], scale=0.5)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)


# ------------------------------------------------------------------ backward

def test_golden_backward():
    for case in json.load(open(GOLDEN))["backward"]:
        q, k, v, do = (_dense(case[n]) for n in ("q", "k", "v", "do"))
        _, _, dq, dk, dv = orc.bwd(q, k, v, do, scale=case["scale"],
                                   window=(_w(case["wl"]), _w(case["wr"])), diag=case["diag"])
        np.testing.assert_allclose(dq[0, 0], np.array(case["dq"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk[0, 0], np.array(case["dk"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv[0, 0], np.array(case["dv"]), rtol=0, atol=1e-12)


@pytest.mark.parametrize("window,diag", [((INF, INF), "top_left"), ((INF, 0), "top_left"),
                                          ((1, 1), "bottom_right"), ((-1, 2), "top_left")])
def test_backward_finite_differences(window, diag):
    """Central differences of <dO, O> in fp64, inputs on a 2^-6 grid so that
    perturbations of 2^-12 are exact in float32."""
    sq, sk, D = 4, 5, 3
    g = torch.Generator().manual_seed(7)

    def grid(*s):
        return torch.randint(-64, 64, s, generator=g).float() / 64

    q, k, v, do = grid(1, 1, sq, D), grid(1, 1, sk, D), grid(1, 1, sk, D), grid(1, 1, sq, D)
    scale, h = 0.9, 2.0 ** -12
    _, _, dq, dk, dv = orc.bwd(q, k, v, do, scale=scale, window=window, diag=diag)
    dod = do.double().numpy()

    def loss(qq, kk, vv):
        o, _ = orc.fwd(qq, kk, vv, scale=scale, window=window, diag=diag)
        return float((o * dod).sum())

    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        base = {"q": q, "k": k, "v": v}
        x = base[name]
        for idx in np.ndindex(*x.shape):
            xp, xm = x.clone(), x.clone()
            xp[idx] += h
            xm[idx] -= h
            args_p = dict(base, **{name: xp})
            args_m = dict(base, **{name: xm})
            fd = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            assert abs(fd - grad[idx]) < 2e-6, (name, idx, fd, grad[idx])


@pytest.mark.parametrize("sq,sk,D,window,diag", CASES)
def test_backward_against_torch_autograd(sq, sk, D, window, diag):
    q, k, v, do = torch.randn(1, 2, sq, D), torch.randn(1, 2, sk, D), torch.randn(1, 2, sk, D), torch.randn(1, 2, sq, D)
    scale = 0.45
    _, _, dq, dk, dv = orc.bwd(q, k, v, do, scale=scale, window=window, diag=diag)
    mask = orc.visible_matrix(sq, sk, window[0], window[1], diag)
    rows = mask.any(axis=1)
    qd, kd, vd = (t.double().requires_grad_(True) for t in (q, k, v))
    # fully masked rows are removed from the torch graph (torch would give NaN)
    o = torch.nn.functional.scaled_dot_product_attention(
        qd[:, :, rows], kd, vd, attn_mask=torch.from_numpy(mask[rows]), scale=scale)
    (o * do.double()[:, :, rows]).sum().backward()
    np.testing.assert_allclose(dq, qd.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, kd.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, vd.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_closed_forms():
    s, D = 7, 4
    q, k, v, do = (torch.randn(1, 1, s, D) for _ in range(4))
    dod = do.double().numpy()[0, 0]
    # scale 0: P uniform over J(i); dQ = dK = 0, dV_j = sum_i dO_i / |J(i)|
    _, _, dq, dk, dv = orc.bwd(q, k, v, do, scale=0.0, window=(INF, 0))
    assert np.all(dq == 0) and np.all(dk == 0)
    ref = np.zeros((s, D))
    for i in range(s):
        ref[: i + 1] += dod[i] / (i + 1)
    np.testing.assert_allclose(dv[0, 0], ref, rtol=0, atol=1e-14)
    # constant V: dS = 0 so dQ = dK = 0
    vc = torch.full((1, 1, s, D), 0.375)
    _, _, dq, dk, _ = orc.bwd(q, k, vc, do, scale=0.8, window=(2, 1), diag="bottom_right")
    np.testing.assert_allclose(dq, 0, atol=1e-14)
    np.testing.assert_allclose(dk, 0, atol=1e-14)
    # one-key window: dV_i = dO_i, dQ = dK = 0
    _, _, dq, dk, dv = orc.bwd(q, k, v, do, scale=0.8, window=(0, 0))
    np.testing.assert_allclose(dv[0, 0], dod, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dq, 0, atol=1e-14)
    np.testing.assert_allclose(dk, 0, atol=1e-14)


@pytest.mark.parametrize("window,diag", [((INF, INF), "top_left"), ((3, 0), "bottom_right"),
                                          ((-1, 1), "top_left"), ((-3, 1), "top_left")])
def test_backward_sum_invariants(window, diag):
    sq, sk, D = 9, 12, 5
    q, k, v, do = torch.randn(2, 2, sq, D), torch.randn(2, 2, sk, D), torch.randn(2, 2, sk, D), torch.randn(2, 2, sq, D)
    _, lse, dq, dk, dv = orc.bwd(q, k, v, do, scale=0.7, window=window, diag=diag)
    np.testing.assert_allclose(dk.sum(axis=2), 0, atol=1e-12)
    rows = np.isfinite(lse)[..., None]
    np.testing.assert_allclose(dv.sum(axis=2), (do.double().numpy() * rows).sum(axis=2), atol=1e-12)


# ------------------------------------------------------------------ packed

def test_packed_equals_dense_per_sequence():
    H, D = 3, 4
    lens_q = [5, 0, 9, 1, 4]
    lens_k = [7, 3, 9, 0, 2]
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    q, k, v, do = (torch.randn(int(c[-1]), H, D).to(torch.bfloat16) for c in (cq, ck, ck, cq))
    for window, diag in [((2, 0), "bottom_right"), ((INF, 0), "top_left"), ((INF, INF), "top_left")]:
        kw = dict(scale=0.5, window=window, diag=diag)
        o, lse, dq, dk, dv = orc.bwd(q, k, v, do, cu_seqlens_q=cq, cu_seqlens_k=ck, **kw)
        for b in range(len(lens_q)):
            qs, ks = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
            if lens_q[b] == 0 and lens_k[b] == 0:
                continue

            def dense(t, s):
                return t[s].permute(1, 0, 2)[None].contiguous()

            ro, rl, rdq, rdk, rdv = orc.bwd(dense(q, qs), dense(k, ks), dense(v, ks), dense(do, qs), **kw)
            np.testing.assert_array_equal(o[qs], ro[0].transpose(1, 0, 2))
            np.testing.assert_array_equal(lse[:, qs], rl[0])
            np.testing.assert_array_equal(dq[qs], rdq[0].transpose(1, 0, 2))
            np.testing.assert_array_equal(dk[ks], rdk[0].transpose(1, 0, 2))
            np.testing.assert_array_equal(dv[ks], rdv[0].transpose(1, 0, 2))


def test_row_and_column_entry_points_match_full():
    lens_q, lens_k = [6, 10], [9, 10]
    cq = np.array([0, 6, 16], np.int32)
    ck = np.array([0, 9, 19], np.int32)
    H, D = 2, 3
    q, k, v, do = (torch.randn(int(c[-1]), H, D) for c in (cq, ck, ck, cq))
    kw = dict(scale=0.8, window=(3, 1), diag="bottom_right", cu_seqlens_q=cq, cu_seqlens_k=ck)
    o, lse, dq, dk, dv = orc.bwd(q, k, v, do, **kw)
    b, h = 1, 1
    rows = [0, 4, 9]
    ro, rl = orc.fwd_rows(q, k, v, b, h, rows, **kw)
    np.testing.assert_array_equal(ro, o[cq[b] + np.array(rows), h])
    np.testing.assert_array_equal(rl, lse[h, cq[b] + np.array(rows)])
    rdq = orc.bwd_dq_rows(q, k, v, do, b, h, rows, **kw)
    np.testing.assert_allclose(rdq, dq[cq[b] + np.array(rows), h], rtol=0, atol=1e-15)
    cols = [0, 3, 8]
    rdk, rdv = orc.bwd_dkdv_cols(q, k, v, do, b, h, cols, **kw)
    np.testing.assert_array_equal(rdk, dk[ck[b] + np.array(cols), h])
    np.testing.assert_array_equal(rdv, dv[ck[b] + np.array(cols), h])


def test_rejects_malformed_problems():
    q = torch.randn(4, 1, 2)
    with pytest.raises(ValueError):
        orc.fwd(q, q, q, scale=1.0, cu_seqlens_q=np.array([0, 3, 2], np.int32),
                cu_seqlens_k=np.array([0, 2, 4], np.int32))
    with pytest.raises(ValueError):
        orc.fwd(q, q, q, scale=1.0, cu_seqlens_q=np.array([1, 4], np.int32),
                cu_seqlens_k=np.array([0, 4], np.int32))
