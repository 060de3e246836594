"""The GPU tests' comparison (tests/parity_util.py) on the CPU: the spacing
it allows per element is the output type's own, and the absolute bound still
decides wherever that spacing is below it."""
import numpy as np
import pytest
import torch

from parity_util import max_err, ulp


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_ulp_is_the_type_spacing(dtype):
    v = torch.tensor([1e-3, 0.3, 1.0, 1.5, 7.9, 8.0, 23.28, -23.28, 1000.0], dtype=dtype)
    up = torch.nextafter(v.abs(), torch.tensor(float("inf"), dtype=dtype)) - v.abs()
    assert np.array_equal(ulp(v.double().numpy(), dtype), up.double().numpy())


def test_bound_per_element():
    ref = np.array([23.2791748046875, 0.5])
    # correctly rounded to bf16: 0.029 off at 23.28 (spacing 0.125 > 0.04) passes
    max_err("dv", torch.tensor(ref).to(torch.bfloat16), ref, 0.04)
    # one bf16 step further is still within one ulp there
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
