"""The GPU tests' comparison (tests/parity_util.py) on the CPU: the spacing
it allows per element is the output type's own, each element is held to the
absolute bound plus half that spacing only where the spacing exceeds the
bound, and the elements admitted that way are counted."""
import numpy as np
import pytest
import torch

import parity_util
from parity_util import half_ulp_bound, max_err, ulp


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_ulp_is_the_type_spacing(dtype):
    v = torch.tensor([1e-3, 0.3, 1.0, 1.5, 7.9, 8.0, 23.28, -23.28, 1000.0], dtype=dtype)
    up = torch.nextafter(v.abs(), torch.tensor(float("inf"), dtype=dtype)) - v.abs()
    assert np.array_equal(ulp(v.double().numpy(), dtype), up.double().numpy())


def test_bound_per_element():
    ref = np.array([23.2791748046875, 0.5])
    # correctly rounded to bf16: 0.029 off at 23.28 (spacing 0.125 > 0.04) passes
    max_err("dv", torch.tensor(ref).to(torch.bfloat16), ref, 0.04)
    # one bf16 step further: 0.096 <= 0.04 + 0.0625
    max_err("dv", torch.tensor([23.375, 0.5], dtype=torch.bfloat16), ref, 0.04)
    # two steps off fails
    with pytest.raises(AssertionError):
        max_err("dv", torch.tensor([23.5, 0.5], dtype=torch.bfloat16), ref, 0.04)
    # at 0.5 the spacing (2^-8) is below the bound: the bound decides
    with pytest.raises(AssertionError):
        max_err("dv", torch.tensor([23.25, 0.5469], dtype=torch.bfloat16), ref, 0.04)
    # a float64 result (no output type) is held to the plain bound
    with pytest.raises(AssertionError):
        max_err("x", np.array([23.33, 0.5]), ref, 0.04)
    # NaN always fails
    with pytest.raises(AssertionError):
        max_err("o", torch.tensor([float("nan"), 0.5]), ref, 1.0)


def test_half_ulp_not_a_full_ulp():
    """The bound is tol + 1/2 ulp, not one ulp: at |x| in [16, 32) bf16's
    spacing is 0.125, so with tol 0.01 the bound is 0.0725 there."""
    ref = np.array([20.0])
    b = half_ulp_bound(np.array([20.0625]), ref, 0.01, torch.bfloat16)
    assert b[0] == pytest.approx(0.0725)
    # 20.0625 is not a bf16 value; 20.125 (one ulp, 0.125 off) must fail
    with pytest.raises(AssertionError):
        max_err("dk", torch.tensor([20.125], dtype=torch.bfloat16), ref, 0.01)
    # a reference at the midpoint rounded either way passes (0.0625 <= 0.0725)
    mid = np.array([20.0625])
    max_err("dk", torch.tensor([20.0], dtype=torch.bfloat16), mid, 0.01)
    max_err("dk", torch.tensor([20.125], dtype=torch.bfloat16), mid, 0.01)


def test_spacing_taken_on_the_coarser_side():
    """A value rounded up across a power of two is held to the spacing above
    it: ref just below 8 (bf16 spacing 2^-5 below, 2^-4 above)."""
    ref = np.array([7.99])
    b = half_ulp_bound(np.array([8.0625]), ref, 0.02, torch.bfloat16)
    assert b[0] == pytest.approx(0.02 + 0.03125)
    max_err("dv", torch.tensor([8.0], dtype=torch.bfloat16), ref, 0.02)


def test_admitted_elements_are_counted():
    parity_util.HALF_ULP_ADMITTED.clear()
    ref = np.array([23.2791748046875, 23.30, 0.5])
    got = torch.tensor([23.25, 23.375, 0.5], dtype=torch.bfloat16)
    max_err("cnt", got, ref, 0.04)
    # 23.25 is 0.029 off (within tol); 23.375 is 0.075 off (admitted by the half ulp)
    assert parity_util.HALF_ULP_ADMITTED == {"cnt": 1}
