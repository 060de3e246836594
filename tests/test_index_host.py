"""Host checks of the kernels' index helpers, compiled from the same header
the kernels include: the XCD block remap is a bijection, the operand
permutation matches the accumulator layout, and tile classification is sound
against the oracle's visibility predicate (an EMPTY tile has no visible
pair, a FULL tile has only visible pairs)."""
import os
import subprocess

import numpy as np
import pytest

from oracle import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "scaled_dot_product_20_amd", "csrc")
INF = orc.WINDOW_INF
EMPTY, PARTIAL, FULL = 0, 1, 2


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("idx") / "index_harness")
    subprocess.check_call(["/opt/rocm/bin/hipcc", "-O1", "-std=c++17", "-x", "hip",
                           "--offload-arch=gfx950", "-I" + CSRC,
                           os.path.join(ROOT, "tests", "index_harness.cpp"), "-o", exe],
                          stderr=subprocess.DEVNULL)
    return exe


def test_remap_grid_permutation_and_full_range(harness):
    out = subprocess.run([harness], input=b"", capture_output=True, check=True).stdout.decode()
    assert "remap_ok" in out and "grid_ok" in out and "perm_ok" in out and "full_ok" in out


def test_visibility_bits_against_oracle(harness):
    """Bit r of the kernels' mask for (query qi, key block jb) is set iff key
    jb + r is visible to qi under the oracle's predicate."""
    rng = np.random.default_rng(5)
    cases = []
    for _ in range(2000):
        sq, sk = (int(x) for x in rng.integers(1, 80, size=2))
        wl = INF if rng.random() < 0.25 else int(rng.integers(-20, 21))
        wr = INF if rng.random() < 0.25 else int(rng.integers(-20, 21))
        diag = int(rng.integers(0, 2))
        qi = int(rng.integers(0, sq))
        jb = int(rng.integers(0, sk))
        cases.append((sq, sk, wl, wr, diag, qi, jb))
    text = "\n".join(" ".join(str(x) for x in c) for c in cases) + "\n"
    out = subprocess.run([harness, "vis"], input=text.encode(), capture_output=True, check=True).stdout.decode()
    masks = [int(x) for x in out.split()]
    assert len(masks) == len(cases)
    for c, mask in zip(cases, masks):
        sq, sk, wl, wr, diag, qi, jb = c
        d = "bottom_right" if diag else "top_left"
        for r in range(32):
            want = jb + r < sk and orc.visible(qi, jb + r, sq, sk, wl, wr, d)
            assert bool(mask >> r & 1) == want, (c, r)


def test_classify_sound_against_oracle(harness):
    rng = np.random.default_rng(3)
    cases = []
    for _ in range(3000):
        sq, sk = (int(x) for x in rng.integers(1, 40, size=2))
        wl = INF if rng.random() < 0.25 else int(rng.integers(-12, 13))
        wr = INF if rng.random() < 0.25 else int(rng.integers(-12, 13))
        diag = int(rng.integers(0, 2))
        nr, nc = int(rng.choice([1, 4, 8, 16])), int(rng.choice([1, 4, 8, 16]))
        i0 = int(rng.integers(0, sq))
        j0 = int(rng.integers(0, sk + 4))
        cases.append((sq, sk, wl, wr, diag, i0, nr, j0, nc))
    text = "\n".join(" ".join(str(x) for x in c) for c in cases) + "\n"
    out = subprocess.run([harness], input=text.encode(), capture_output=True, check=True).stdout.decode()
    classes = [int(x) for x in out.split() if not x.endswith("_ok")]
    assert len(classes) == len(cases)
    mats = {}
    for c, cls in zip(cases, classes):
        sq, sk, wl, wr, diag, i0, nr, j0, nc = c
        key = (sq, sk, wl, wr, diag)
        if key not in mats:
            mats[key] = orc.visible_matrix(sq, sk, wl, wr, "bottom_right" if diag else "top_left")
        m = mats[key]
        rows = range(i0, min(i0 + nr, sq))
        cols = range(j0, j0 + nc)
        vis = [m[i, j] if j < sk else False for i in rows for j in cols]
        if cls == EMPTY:
            assert not any(vis), c
        elif cls == FULL:
            assert all(vis) and j0 + nc <= sk, c
        if nr == 1 and nc == 1 and i0 < sq and j0 < sk:
            assert cls == (FULL if m[i0, j0] else EMPTY), c  # exact on single pairs
