"""Seeded random shapes through the blocked path (odd and ragged m, n and a forced N_B), every
product form included: the eight-wave tiles, split products, complex products in real form and
on-load. Each case is checked against the CPU oracle on sampled right-hand-side columns."""
import numpy as np
import pytest

import oracle
from _gpu_util import TOL_LARGE, colmajor_inputs, rel_err, say, to_dev, views

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f64", "c64", "c128"]


def cases(count=32, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(count):
        dt = DTYPES[c % 4]
        m = int(rng.integers(65, 2600))
        n = int(rng.integers(1, 700))
        nb = int(rng.choice([64, 128, 256, 512, 1024]))
        if dt == "c128" and nb > 512:
            nb = 512
        if nb > m:
            nb = 64
        out.append((c, dt, m, n, nb))
    return out


@pytest.fixture(scope="module")
def hs():
    import torch  # noqa: F401
    import triangular_solve_amd as hs
    return hs


@pytest.mark.parametrize("c,dt,m,n,nb", cases())
def test_random_blocked_shape(hs, c, dt, m, n, nb):
    import torch
    say("random blocked", c, dt, m, n, nb)
    A, B = colmajor_inputs(dt, m, n, 1, seed=1000 + c)
    dA, dB = to_dev(A), to_dev(B)
    alpha = 1.0 if c % 3 else (0.5 - 0.25j if dt.startswith("c") else -0.75)
    st = hs.entry("ex", dt)(m, n, alpha, dA, m, dB, m, {"nb": nb, "path": hs.PATH_BLOCKED})
    torch.cuda.synchronize()
    assert st == hs.SUCCESS, hs.status_string(st)
    cols = np.sort(np.random.default_rng(c).choice(n, size=min(n, 8), replace=False))
    Av, Bv = views(A, B, m)
    Xo = oracle.trsm(np.ascontiguousarray(Av), np.ascontiguousarray(Bv[:, :, cols]), alpha)
    Xg = dB.cpu().numpy()[:, :, :m].transpose(0, 2, 1)[:, :, cols]
    assert rel_err(Xg, Xo) <= TOL_LARGE[dt]
