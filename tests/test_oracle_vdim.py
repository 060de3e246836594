"""Pins of the oracle with a value head dim different from the query/key
head dim (Hdim_vo != Hdim_qk, the AOTriton 0.15b release notes, "Kernel
Bug Fixes"), against facts that do not come from the oracle:

- torch's float64 SDPA and autograd on the CPU, which take V with its own
  last dim, forward (O, LSE) and backward (dQ, dK, dV), under textbook band
  masks from numpy;
- column split: O and dV are linear in V's columns and dQ, dK in dO's, so
  splitting V (and dO) into column blocks gives the blocks of O and dV and
  sums of dQ and dK of problems with the equal-dims path, which the other
  pins tie down;
- the packed layout of sequences reduces to dense runs, as with equal dims;
- prime head dims on either side.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc

INF = orc.WINDOW_INF


def band(sq, sk, lo=None, hi=None):
    """Textbook band mask lo <= j - i <= hi via numpy (None = unbounded)."""
    m = np.ones((sq, sk), dtype=bool)
    if hi is not None:
        m &= np.tril(np.ones((sq, sk), dtype=bool), k=hi)
    if lo is not None:
        m &= np.triu(np.ones((sq, sk), dtype=bool), k=lo)
    return m


# (sq, sk, D, DV, window, band bounds lo, hi for top-left)
CASES = [
    (9, 11, 8, 5, (INF, INF), None, None),
    (10, 10, 3, 16, (INF, 0), None, 0),
    (7, 12, 13, 7, (2, 3), -2, 3),
    (12, 6, 4, 11, (INF, 1), None, 1),
]


@pytest.mark.parametrize("sq,sk,D,DV,window,lo,hi", CASES)
def test_forward_and_backward_against_torch(sq, sk, D, DV, window, lo, hi):
    g = torch.Generator().manual_seed(sq * 100 + DV)
    q, k = torch.randn(2, 3, sq, D, generator=g), torch.randn(2, 3, sk, D, generator=g)
    v, do = torch.randn(2, 3, sk, DV, generator=g), torch.randn(2, 3, sq, DV, generator=g)
    scale = 0.6
    o, lse, dq, dk, dv = orc.bwd(q, k, v, do, scale=scale, window=window, diag="top_left")
    assert o.shape == (2, 3, sq, DV) and dv.shape == (2, 3, sk, DV) and dq.shape == (2, 3, sq, D)
    mask = band(sq, sk, lo, hi)
    rows = mask.any(axis=1)
    qd, kd, vd = (t.double().requires_grad_(True) for t in (q, k, v))
    m = torch.from_numpy(mask[rows])
    ro = torch.nn.functional.scaled_dot_product_attention(qd[:, :, rows], kd, vd, attn_mask=m, scale=scale)
    s = (torch.matmul(qd[:, :, rows], kd.transpose(-1, -2)) * scale).masked_fill(~m, float("-inf"))
    rl = torch.logsumexp(s, dim=-1)
    np.testing.assert_allclose(o[:, :, rows], ro.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, rows], rl.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.all(o[:, :, ~rows] == 0.0) and np.all(np.isposinf(lse[:, :, ~rows]))
    (ro * do.double()[:, :, rows]).sum().backward()
    np.testing.assert_allclose(dq, qd.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, kd.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, vd.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("D,DV", [(6, 12), (6, 18), (5, 10)])
def test_column_split_reduces_to_equal_dims(D, DV):
    """V = [V_1 | ... | V_n] with D columns each (dO likewise): O = [O_1 |
    ... | O_n], dV = [dV_1 | ...], dQ = sum of dQ_t and dK = sum of dK_t
    over the equal-dims problems (Q, K, V_t, dO_t), LSE of any of them."""
    g = torch.Generator().manual_seed(D * DV)
    sq, sk, n = 9, 13, DV // D
    q, k = torch.randn(1, 2, sq, D, generator=g), torch.randn(1, 2, sk, D, generator=g)
    v, do = torch.randn(1, 2, sk, DV, generator=g), torch.randn(1, 2, sq, DV, generator=g)
    kw = dict(scale=0.5, window=(4, 1), diag="bottom_right")
    o, lse, dq, dk, dv = orc.bwd(q, k, v, do, **kw)
    dq_sum, dk_sum = np.zeros_like(dq), np.zeros_like(dk)
    for t in range(n):
        cols = slice(t * D, (t + 1) * D)
        ot, lt, dqt, dkt, dvt = orc.bwd(q, k, v[..., cols].contiguous(), do[..., cols].contiguous(), **kw)
        np.testing.assert_allclose(o[..., cols], ot, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(dv[..., cols], dvt, rtol=1e-13, atol=1e-13)
        np.testing.assert_array_equal(lse, lt)
        dq_sum += dqt
        dk_sum += dkt
    np.testing.assert_allclose(dq, dq_sum, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, dk_sum, rtol=1e-11, atol=1e-12)


def test_packed_equals_dense_per_sequence():
    g = torch.Generator().manual_seed(7)
    lq, lk, H, D, DV = [5, 0, 9], [7, 3, 4], 2, 7, 3
    cuq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cuk = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q, k = torch.randn(cuq[-1], H, D, generator=g), torch.randn(cuk[-1], H, D, generator=g)
    v, do = torch.randn(cuk[-1], H, DV, generator=g), torch.randn(cuq[-1], H, DV, generator=g)
    kw = dict(scale=0.4, window=(3, 0), diag="bottom_right")
    o, lse, dq, dk, dv = orc.bwd(q, k, v, do, cu_seqlens_q=cuq, cu_seqlens_k=cuk, **kw)
    for b in range(3):
        rq, rk = slice(cuq[b], cuq[b + 1]), slice(cuk[b], cuk[b + 1])
        dense = [t[r].permute(1, 0, 2).unsqueeze(0).contiguous() for t, r in ((q, rq), (k, rk), (v, rk), (do, rq))]
        od, ld, dqd, dkd, dvd = orc.bwd(*dense, **kw)
        np.testing.assert_array_equal(o[rq], od[0].transpose(1, 0, 2))
        np.testing.assert_array_equal(lse[:, rq], ld[0])
        np.testing.assert_array_equal(dq[rq], dqd[0].transpose(1, 0, 2))
        np.testing.assert_array_equal(dk[rk], dkd[0].transpose(1, 0, 2))
        np.testing.assert_array_equal(dv[rk], dvd[0].transpose(1, 0, 2))


def test_row_and_column_entry_points_take_value_dim():
    g = torch.Generator().manual_seed(3)
    q, k = torch.randn(1, 1, 6, 5, generator=g), torch.randn(1, 1, 8, 5, generator=g)
    v, do = torch.randn(1, 1, 8, 11, generator=g), torch.randn(1, 1, 6, 11, generator=g)
    kw = dict(scale=0.3, window=(INF, 1), diag="top_left")
    o, lse, dq, dk, dv = orc.bwd(q, k, v, do, **kw)
    ro, rl = orc.fwd_rows(q, k, v, 0, 0, [0, 3, 5], **kw)
    np.testing.assert_array_equal(ro, o[0, 0, [0, 3, 5]])
    np.testing.assert_array_equal(rl, lse[0, 0, [0, 3, 5]])
    np.testing.assert_array_equal(orc.bwd_dq_rows(q, k, v, do, 0, 0, [1, 4], **kw), dq[0, 0, [1, 4]])
    ck, cv = orc.bwd_dkdv_cols(q, k, v, do, 0, 0, [0, 7], **kw)
    np.testing.assert_array_equal(ck, dk[0, 0, [0, 7]])
    np.testing.assert_array_equal(cv, dv[0, 0, [0, 7]])


def test_mismatched_value_shapes_rejected():
    q, k = torch.randn(1, 1, 4, 3), torch.randn(1, 1, 5, 3)
    with pytest.raises(ValueError):
        orc.fwd(q, k, torch.randn(1, 1, 4, 3), scale=1.0)          # V rows != K rows
    with pytest.raises(ValueError):
        orc.bwd(q, k, torch.randn(1, 1, 5, 6), torch.randn(1, 1, 4, 3), scale=1.0)  # dO dim != V dim
