"""GPU parity of the blocked solve with few right-hand sides, where the
products run split along K (partial products summed in a fixed order):
against the oracle, bitwise repeatable, and exact on an integer system."""
import numpy as np
import pytest

import oracle
from _gpu_util import TOL_LARGE, colmajor_inputs, rel_err, say, to_dev, views

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f64", "c64", "c128"]


@pytest.fixture(scope="module")
def hs():
    import torch  # noqa: F401
    import triangular_solve_amd as hs
    return hs


def solve(hs, dt, A, B, m, n, nb):
    import torch
    dA, dB = to_dev(A), to_dev(B)
    st = hs.entry("ex", dt)(m, n, 1.0, dA, m, dB, m, {"nb": nb, "path": hs.PATH_BLOCKED})
    torch.cuda.synchronize()
    assert st == hs.SUCCESS
    return dB.cpu().numpy()


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("m,n,nb", [(2048, 64, 1024), (2048, 8, 512), (4096, 1, 2048), (3000, 100, 512),
                                    (1024, 256, 256), (2560, 33, 512)])
def test_few_rhs_parity_and_repeat(hs, dt, m, n, nb):
    if dt == "c128" and nb > 512 and m % nb:
        pytest.skip("not offered")
    say("few rhs", dt, m, n, nb)
    A, B = colmajor_inputs(dt, m, n, 1, seed=m + n)
    X1 = solve(hs, dt, A, B, m, n, nb)
    X2 = solve(hs, dt, A, B, m, n, nb)
    assert np.array_equal(X1, X2)                     # fixed summation order
    Av, Bv = views(A, B, m)
    assert rel_err(X1[:, :, :m].transpose(0, 2, 1), oracle.trsm(Av, Bv)) <= TOL_LARGE[dt]


def test_few_rhs_largest(hs):
    m, n = 8192, 64
    for dt in ("f32", "c128"):
        A, B = colmajor_inputs(dt, m, n, 1, seed=3)
        nb = hs.hsma_trsm_block_size(hs.DTYPE_CODE[dt], m, n)
        X = solve(hs, dt, A, B, m, n, nb)
        cols = np.arange(0, n, 8)
        Av, Bv = views(A, B, m)
        Xo = oracle.trsm(Av, np.ascontiguousarray(Bv[:, :, cols]))
        assert rel_err(X[:, cols, :m].transpose(0, 2, 1), Xo) <= TOL_LARGE[dt]


def test_few_rhs_exact_integer(hs):
    """Bidiagonal (1, -1) A and small-integer B: X is the running sum of B's
    rows, every partial product and sum an exact small integer."""
    m, n, nb = 4096, 16, 1024
    L = np.zeros((m, m))
    L[np.diag_indices(m)] = 1
    L[np.arange(1, m), np.arange(m - 1)] = -1
    L[np.triu_indices(m, 1)] = np.nan
    A = np.ascontiguousarray(L.T)[None]
    rng = np.random.default_rng(0)
    B = rng.integers(-4, 5, (1, n, m)).astype(np.float64)
    X = solve(hs, "f64", A, B, m, n, nb)
    assert np.array_equal(X[0], np.cumsum(B[0], axis=1))


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("m,n,nb", [(1024, 1024, 256), (1500, 700, 512), (2048, 513, 512),
                                    (1000, 300, 256), (2048, 2048, 256)])
def test_split_products_many_rhs(hs, dt, m, n, nb):
    """Products with few output tiles split along K at any n (ragged last
    block rows and chunk counts that must divide K): parity with the oracle
    and the same bits on a repeat."""
    say("split products", dt, m, n, nb)
    A, B = colmajor_inputs(dt, m, n, 1, seed=m + 3 * n)
    X1 = solve(hs, dt, A, B, m, n, nb)
    X2 = solve(hs, dt, A, B, m, n, nb)
    assert np.array_equal(X1, X2)
    cols = np.unique(np.linspace(0, n - 1, 40).astype(np.int64))
    Av, Bv = views(A, B, m)
    Xo = oracle.trsm(Av, np.ascontiguousarray(Bv[:, :, cols]))
    assert rel_err(X1[:, cols, :m].transpose(0, 2, 1), Xo) <= TOL_LARGE[dt]
