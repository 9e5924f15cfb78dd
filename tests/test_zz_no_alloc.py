"""hsma_trsm_noalloc (the solve without device allocation, workspace from the
library's fixed per-GPU scratch) against hsma_trsm_{s,d,c,z}, through the C
ABI: two calls in a row, the second smaller, per dtype; column chunks under
a lowered scratch limit; and the oracle on sampled columns."""
import numpy as np
import pytest

import oracle
from _gpu_util import TOL_LARGE, TOL_SMALL, colmajor_inputs, rel_err, say, to_dev, views

pytestmark = pytest.mark.gpu

CODE = {"f32": 0, "f64": 1, "c64": 2, "c128": 3}


@pytest.fixture(scope="module")
def hs():
    import torch  # noqa: F401
    import triangular_solve_amd as hs
    return hs


def both(hs, dt, m, n, alpha, seed):
    """X from hsma_trsm_* and from hsma_trsm_noalloc on the same inputs."""
    import torch
    A, B = colmajor_inputs(dt, m, n, 1, seed=seed)
    dA, dB1, dB2 = to_dev(A), to_dev(B), to_dev(B)
    hs.check(hs.entry("trsm", dt)(m, n, alpha, dA, m, dB1, m), "trsm_" + dt)
    hs.check(hs.hsma_trsm_noalloc(CODE[dt], m, n, alpha, dA, m, dB2, m), "noalloc " + dt)
    torch.cuda.synchronize()
    X1 = dB1.cpu().numpy()[:, :, :m].transpose(0, 2, 1)
    X2 = dB2.cpu().numpy()[:, :, :m].transpose(0, 2, 1)
    return A, B, X1, X2


@pytest.mark.parametrize("dt,first,second,alpha", [
    ("f32", (2048, 2048), (300, 100), 1.0),
    ("f64", (1500, 700), (64, 64), -0.5),
    ("c64", (1024, 512), (200, 30), 1.0),
    ("c128", (1024, 1024), (130, 70), 0.5 - 2j),
])
def test_noalloc_matches_trsm_twice(hs, dt, first, second, alpha):
    for (m, n) in (first, second):
        say("noalloc", dt, m, n, alpha)
        A, B, X1, X2 = both(hs, dt, m, n, alpha, seed=m + n)
        tol = (TOL_SMALL if m <= 64 else TOL_LARGE)[dt]
        assert np.isfinite(X2).all()
        assert rel_err(X2, X1) <= tol, (dt, m, n)
        cols = np.arange(0, n, max(1, n // 16))
        Av, Bv = views(A, B, m)
        assert rel_err(X2[:, :, cols], oracle.trsm(Av, Bv[:, :, cols], alpha=alpha)) <= tol


def test_noalloc_column_chunks(hs, monkeypatch):
    """A 1 MiB scratch limit forces N_B = 256 and eight column chunks for
    m = 512, n = 4000 (f32); then a 600 kB limit with m = 1000 (f64) forces
    N_B = 32 on the column-substitution inversion."""
    monkeypatch.setenv("HSMA_NOALLOC_LIMIT", str(1 << 20))
    A, B, X1, X2 = both(hs, "f32", 512, 4000, 1.0, seed=5)
    assert rel_err(X2, X1) <= TOL_LARGE["f32"]
    monkeypatch.setenv("HSMA_NOALLOC_LIMIT", "600000")
    A, B, X1, X2 = both(hs, "f64", 1000, 500, 2.0, seed=6)
    assert rel_err(X2, X1) <= TOL_LARGE["f64"]
