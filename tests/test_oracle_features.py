"""Pins of the oracle's optional features (additive bias, ALiBi, dropout)
against facts that do not come from the oracle.

- Philox4x32-10: the known-answer vectors published with the generator
  (Salmon, Moraes, Dror and Shaw, SC 2011, and its reference
  implementation), for counters and keys of all zeros, all ones, and the
  digits of pi.
- Dropout: the keep rate is 1 - p within binomial noise and differs between
  heads, seeds and offsets; p = 0 is the plain result; the forward equals the
  masked, rescaled softmax computed by torch in float64; the gradients equal
  central finite differences (the mask does not depend on the inputs); the
  packed layout of equal-length sequences equals the dense one.
- Bias: torch's float64 SDPA with the additive mask, forward and autograd
  (dQ, dK, dV and the bias gradient); a bias constant along a row leaves O
  and shifts LSE by that constant; a bias of -inf masks like the window.
- ALiBi: torch's float64 SDPA with the bias -slope_h |i + sk - sq - j|
  written out, both diagonals of a rectangular problem.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc

INF = orc.WINDOW_INF


# --------------------------------------------------------------- Philox

@pytest.mark.parametrize("ctr,key,want", [
    ([0, 0, 0, 0], [0, 0], [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]),
    ([0xffffffff] * 4, [0xffffffff] * 2, [0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]),
    ([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344], [0xa4093822, 0x299f31d0],
     [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]),
])
def test_philox_known_answers(ctr, key, want):
    assert orc.philox4x32_10(ctr, key) == want


# --------------------------------------------------------------- dropout

def _qkv(B, H, sq, sk, D, seed=0, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(B, H, s, D, generator=g).to(dtype) for s in (sq, sk, sk, sq)]


def test_dropout_keep_rate_and_streams():
    q, k, v, _ = _qkv(2, 2, 64, 250, 4)
    p = 0.3
    feat = dict(dropout_p=p, philox_seed=1234, philox_offset=77)
    masks = {(b, h): orc.dropout_mask(q, k, v, b, h, 64, 250, **feat) for b in range(2) for h in range(2)}
    n = 64 * 250
    for m in masks.values():
        kept = m.sum()
        sigma = (n * p * (1 - p)) ** 0.5
        assert abs(kept - n * (1 - p)) < 5 * sigma
    vals = list(masks.values())
    assert all(not np.array_equal(vals[0], m) for m in vals[1:])
    assert not np.array_equal(orc.dropout_mask(q, k, v, 0, 0, 64, 250, **dict(feat, philox_seed=1235)), vals[0])
    assert not np.array_equal(orc.dropout_mask(q, k, v, 0, 0, 64, 250, **dict(feat, philox_offset=78)), vals[0])
    # p = 0 keeps everything
    assert orc.dropout_mask(q, k, v, 1, 1, 64, 250, dropout_p=0.0).all()
    # the four words of one counter serve four consecutive keys: moving the
    # offset by one counter moves the mask of a row by four keys
    shifted = orc.dropout_mask(q, k, v, 0, 0, 1, 250, **dict(feat, philox_offset=78))
    assert np.array_equal(shifted[0, :-4], vals[0][0, 4:])


def test_dropout_zero_is_plain():
    q, k, v, do = _qkv(1, 2, 9, 13, 4, seed=1)
    plain = orc.bwd(q, k, v, do, scale=0.5, window=(3, 2), diag="bottom_right")
    zero = orc.bwd(q, k, v, do, scale=0.5, window=(3, 2), diag="bottom_right", dropout_p=0.0, philox_seed=9)
    for a, b in zip(plain, zero):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("window,diag", [((INF, INF), "top_left"), ((INF, 0), "top_left"), ((2, 1), "bottom_right")])
def test_dropout_forward_against_torch(window, diag):
    B, H, sq, sk, D = 2, 2, 7, 10, 5
    q, k, v, _ = _qkv(B, H, sq, sk, D, seed=2)
    p, scale = 0.25, 0.6
    feat = dict(dropout_p=p, philox_seed=99, philox_offset=5)
    o, lse = orc.fwd(q, k, v, scale=scale, window=window, diag=diag, **feat)
    vis = torch.from_numpy(orc.visible_matrix(sq, sk, window[0], window[1], diag))
    s = torch.matmul(q.double(), k.double().transpose(-1, -2)) * scale
    s = s.masked_fill(~vis, float("-inf"))
    rows = vis.any(-1)
    probs = torch.softmax(s[:, :, rows], dim=-1)
    keep = torch.stack([torch.stack([torch.from_numpy(orc.dropout_mask(q, k, v, b, h, sq, sk, **feat))
                                     for h in range(H)]) for b in range(B)])
    want = torch.matmul(probs * keep[:, :, rows].double() / (1 - p), v.double())
    np.testing.assert_allclose(o[:, :, rows.numpy()], want.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, rows.numpy()], torch.logsumexp(s[:, :, rows], -1).numpy(),
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window,diag", [((INF, INF), "top_left"), ((1, 1), "bottom_right")])
def test_dropout_backward_finite_differences(window, diag):
    """Central differences of <dO, O> with the dropout mask held fixed (it
    depends only on the seed, the offset and the position)."""
    sq, sk, D = 4, 6, 3
    g = torch.Generator().manual_seed(8)

    def grid(*s):
        return torch.randint(-64, 64, s, generator=g).float() / 64

    q, k, v, do = grid(1, 1, sq, D), grid(1, 1, sk, D), grid(1, 1, sk, D), grid(1, 1, sq, D)
    scale, h = 0.8, 2.0 ** -12
    feat = dict(dropout_p=0.4, philox_seed=31, philox_offset=2)
    assert 0 < orc.dropout_mask(q, k, v, 0, 0, sq, sk, **feat).sum() < sq * sk  # some dropped, some kept
    _, _, dq, dk, dv = orc.bwd(q, k, v, do, scale=scale, window=window, diag=diag, **feat)
    dod = do.double().numpy()

    def loss(qq, kk, vv):
        o, _ = orc.fwd(qq, kk, vv, scale=scale, window=window, diag=diag, **feat)
        return float((o * dod).sum())

    base = {"q": q, "k": k, "v": v}
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        x = base[name]
        for idx in np.ndindex(*x.shape):
            xp, xm = x.clone(), x.clone()
            xp[idx] += h
            xm[idx] -= h
            ap, am = dict(base, **{name: xp}), dict(base, **{name: xm})
            fd = (loss(ap["q"], ap["k"], ap["v"]) - loss(am["q"], am["k"], am["v"])) / (2 * h)
            assert abs(fd - grad[idx]) < 4e-6, (name, idx, fd, grad[idx])


def test_dropout_packed_equals_dense():
    """Equal-length sequences: the packed layout gives the dense counters
    (sequence b, head h, row i) and so the dense result."""
    B, H, S, D = 3, 2, 6, 4
    q, k, v, do = _qkv(B, H, S, S, D, seed=3)
    feat = dict(dropout_p=0.5, philox_seed=7, philox_offset=1000)
    dense = orc.bwd(q, k, v, do, scale=0.4, window=(2, 0), diag="top_left", **feat)
    pk = [t.permute(0, 2, 1, 3).reshape(B * S, H, D).contiguous() for t in (q, k, v, do)]
    cu = np.arange(B + 1, dtype=np.int32) * S
    packed = orc.bwd(*pk, scale=0.4, window=(2, 0), diag="top_left", cu_seqlens_q=cu, cu_seqlens_k=cu, **feat)
    for i, (a, b) in enumerate(zip(dense, packed)):
        if i == 1:  # LSE: dense [B, H, S], packed [H, T]
            b = b.reshape(H, B, S).transpose(1, 0, 2)
        else:
            b = b.reshape(B, S, H, D).transpose(0, 2, 1, 3)
        np.testing.assert_array_equal(a, b)


# ------------------------------------------------------------------ bias

def _sdpa_with_bias(q, k, v, do, bias, vis, scale):
    """torch float64 SDPA with an additive float mask (bias where visible,
    -inf elsewhere) on the rows that see a key; outputs and gradients."""
    rows = vis.any(-1)
    qd, kd, vd = (t.double().requires_grad_(True) for t in (q, k, v))
    bd = bias.double().clone().requires_grad_(True)
    m = torch.where(vis, bd, torch.tensor(float("-inf"), dtype=torch.float64))
    o = torch.nn.functional.scaled_dot_product_attention(qd[:, :, rows], kd, vd, attn_mask=m[:, :, rows],
                                                         scale=scale)
    (o * do.double()[:, :, rows]).sum().backward()
    s = torch.matmul(qd, kd.transpose(-1, -2)) * scale + m
    lse = torch.logsumexp(s[:, :, rows], -1)
    return o.detach(), lse.detach(), qd.grad, kd.grad, vd.grad, bd.grad, rows


@pytest.mark.parametrize("window,diag", [((INF, INF), "top_left"), ((INF, 0), "bottom_right"),
                                          ((2, 3), "bottom_right")])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_bias_against_torch(window, diag, dtype):
    B, H, sq, sk, D = 2, 3, 6, 9, 4
    q, k, v, do = _qkv(B, H, sq, sk, D, seed=4, dtype=dtype)
    g = torch.Generator().manual_seed(5)
    bias = (2 * torch.randn(B, H, sq, sk, generator=g)).to(dtype)
    scale = 0.55
    o, lse, dq, dk, dv, db = orc.bwd(q, k, v, do, scale=scale, window=window, diag=diag, bias=bias, want_dbias=True)
    vis = torch.from_numpy(orc.visible_matrix(sq, sk, window[0], window[1], diag))
    ro, rl, rdq, rdk, rdv, rdb, rows = _sdpa_with_bias(q, k, v, do, bias, vis, scale)
    r = rows.numpy()
    np.testing.assert_allclose(o[:, :, r], ro.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, r], rl.numpy(), rtol=1e-10, atol=1e-12)
    for got, want in ((dq, rdq), (dk, rdk), (dv, rdv), (db, rdb)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-9, atol=1e-12)


def test_bias_broadcast_strides():
    """A bias broadcast over batch and heads (stride 0) is the same as its
    expanded copy."""
    q, k, v, do = _qkv(2, 3, 5, 7, 4, seed=6)
    row = torch.randn(1, 1, 5, 7)
    a = orc.bwd(q, k, v, do, scale=0.5, bias=row.expand(2, 3, 5, 7))
    b = orc.bwd(q, k, v, do, scale=0.5, bias=row.expand(2, 3, 5, 7).contiguous())
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_bias_row_constant_shifts_lse_only():
    q, k, v, _ = _qkv(1, 2, 6, 8, 4, seed=7)
    c = torch.tensor([0.5, -1.25, 3.0, 0.0, 2.0, -0.75]).view(1, 1, 6, 1).expand(1, 2, 6, 8)
    o0, l0 = orc.fwd(q, k, v, scale=0.7, window=(INF, 1), diag="top_left")
    o1, l1 = orc.fwd(q, k, v, scale=0.7, window=(INF, 1), diag="top_left", bias=c)
    np.testing.assert_allclose(o1, o0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l0 + c[:, :, :, 0].double().numpy(), rtol=0, atol=1e-12)


def test_bias_minus_inf_masks_like_the_window():
    """A bias of -inf outside the band (1, 1) equals the window (1, 1); a row
    whose every logit is -inf is a fully masked row."""
    q, k, v, do = _qkv(1, 2, 7, 7, 4, seed=8)
    vis = torch.from_numpy(orc.visible_matrix(7, 7, 1, 1, "top_left"))
    bias = torch.where(vis, torch.tensor(0.0), torch.tensor(float("-inf"))).expand(1, 2, 7, 7).contiguous()
    bias[:, :, 3, :] = float("-inf")
    a = orc.bwd(q, k, v, do, scale=0.6, bias=bias)
    b = orc.bwd(q, k, v, do, scale=0.6, window=(1, 1))
    rows = [i for i in range(7) if i != 3]
    for i, (x, y) in enumerate(zip(a, b)):
        if i == 1:
            np.testing.assert_allclose(x[:, :, rows], y[:, :, rows], rtol=1e-12, atol=1e-13)
        elif i in (0, 2):
            np.testing.assert_allclose(x[:, :, rows], y[:, :, rows], rtol=1e-12, atol=1e-13)
    assert np.all(a[0][:, :, 3] == 0) and np.all(np.isposinf(a[1][:, :, 3])) and np.all(a[2][:, :, 3] == 0)


# ------------------------------------------------------------------ ALiBi

@pytest.mark.parametrize("sq,sk,window,diag", [(6, 9, (INF, INF), "top_left"), (9, 6, (INF, 0), "top_left"),
                                              (5, 8, (2, 0), "bottom_right")])
def test_alibi_against_torch(sq, sk, window, diag):
    B, H, D = 1, 3, 4
    q, k, v, do = _qkv(B, H, sq, sk, D, seed=9)
    slopes = [0.5, 0.125, 0.03125]
    i = torch.arange(sq).view(sq, 1).double()
    j = torch.arange(sk).view(1, sk).double()
    alibi = torch.stack([-s * (i + (sk - sq) - j).abs() for s in slopes]).unsqueeze(0)
    scale = 0.5
    o, lse, dq, dk, dv = orc.bwd(q, k, v, do, scale=scale, window=window, diag=diag, alibi_slopes=slopes)
    vis = torch.from_numpy(orc.visible_matrix(sq, sk, window[0], window[1], diag))
    ro, rl, rdq, rdk, rdv, _, rows = _sdpa_with_bias(q, k, v, do, alibi, vis, scale)
    r = rows.numpy()
    np.testing.assert_allclose(o[:, :, r], ro.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, r], rl.numpy(), rtol=1e-10, atol=1e-12)
    for got, want in ((dq, rdq), (dk, rdk), (dv, rdv)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-9, atol=1e-12)
