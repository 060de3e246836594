"""Seeded random parity sweep against the fp64 oracle: each case draws its
dtype, head dim, layout (dense, dense viewed from [B, S, H, D], packed),
window bounds (sentinels, zero, positive, negative), diagonal, scale and
ragged lengths (packed sequences of 0, 1 or up to 300 rows; dense lengths up
to 700) from its own seed, so a failure names one reproducible problem.  The
fixed-shape tests pick the corners; this sweep covers their combinations."""
import random

import pytest
import torch

from parity_util import INF, Case

pytestmark = pytest.mark.gpu

N_CASES = 48


def draw_case(n: int) -> Case:
    rng = random.Random(7000 + n)
    dtype = rng.choice([torch.bfloat16, torch.float16, torch.float32])
    D = rng.choice([32, 48, 64, 80, 96, 128])
    wl = rng.choice([INF, 0, 3, 17, 64, 200, -5])
    wr = rng.choice([INF, 0, 2, 33, -4, 100])
    diag = rng.choice(["top_left", "bottom_right"])
    scale = rng.choice([None, None, None, 0.3, -0.1])
    common = dict(D=D, dtype=dtype, window=(wl, wr), diag=diag, scale=scale, seed=7000 + n)
    if rng.random() < 0.4:
        nb = rng.randint(1, 5)
        lq = [rng.choice([0, 1, rng.randint(1, 300)]) for _ in range(nb)]
        lk = [rng.choice([0, 1, rng.randint(1, 300)]) for _ in range(nb)]
        return Case(layout="thd", H=rng.randint(1, 3), lens_q=lq, lens_k=lk, **common)
    return Case(B=rng.randint(1, 3), H=rng.randint(1, 3), Sq=rng.randint(1, 700), Sk=rng.randint(1, 700),
                bshd=rng.random() < 0.3, **common)


@pytest.mark.parametrize("n", range(N_CASES))
def test_random_case(n):
    draw_case(n).check()
