"""Batched solves with 64 < m <= 256 (block rows of 64 over the whole batch)
against the CPU oracle."""
import numpy as np
import pytest

import oracle
from _gpu_util import (EPS, TOL_LARGE, colmajor_inputs, rel_err, say, scaled_residual, to_dev,
                       views)

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f64", "c64", "c128"]


@pytest.fixture(scope="module")
def hs():
    import torch  # noqa: F401
    import triangular_solve_amd as hs
    return hs


def batched(hs, dtype, m, n, batch, alpha=1.0, lda=None, ldb=None, shared_a=False, seed=0):
    import torch
    lda, ldb = lda or m, ldb or m
    A, B = colmajor_inputs(dtype, m, n, batch, lda=lda, ldb=ldb, seed=seed, shared_a=shared_a)
    dA, dB = to_dev(A), to_dev(B)
    strideA = 0 if shared_a else lda * m
    st = hs.entry("strided_batched", dtype)(m, n, alpha, dA, lda, strideA, dB, ldb, ldb * n, batch)
    torch.cuda.synchronize()
    assert st == hs.SUCCESS, hs.status_string(st)
    return A, B, dB.cpu().numpy()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("m,n,batch", [(65, 1, 3), (100, 7, 5), (128, 64, 6), (200, 100, 2),
                                       (256, 33, 4), (192, 64, 50)])
def test_medium_batched(hs, dtype, m, n, batch):
    say("medium batched", dtype, m, n, batch)
    A, B, X = batched(hs, dtype, m, n, batch, seed=m + n + batch)
    Av, Bv = views(A, B, m)
    Xo = oracle.trsm(Av, Bv)
    Xg = X[:, :, :m].transpose(0, 2, 1)
    assert rel_err(Xg, Xo) <= TOL_LARGE[dtype]
    assert scaled_residual(np.ascontiguousarray(Av), Xg, Bv, 1.0) <= 10 * m * EPS[dtype]


@pytest.mark.parametrize("dtype", DTYPES)
def test_medium_batched_alpha_padding_shared_a(hs, dtype):
    cplx = dtype.startswith("c")
    alpha = 0.3 - 0.8j if cplx else -2.5
    say("medium alpha/padding", dtype)
    A, B, X = batched(hs, dtype, 150, 40, 3, alpha=alpha, lda=157, ldb=152, seed=11)
    Av, Bv = views(A, B, 150)
    assert rel_err(X[:, :, :150].transpose(0, 2, 1), oracle.trsm(Av, Bv, alpha)) <= TOL_LARGE[dtype]
    assert np.array_equal(X[:, :, 150:], B[:, :, 150:])   # rows below m untouched
    say("medium shared A", dtype)
    A, B, X = batched(hs, dtype, 130, 20, 4, shared_a=True, seed=12)
    Av, Bv = views(A, B, 130)
    Av = np.broadcast_to(Av, (B.shape[0],) + Av.shape[1:])
    assert rel_err(X[:, :, :130].transpose(0, 2, 1), oracle.trsm(Av, Bv)) <= TOL_LARGE[dtype]


def test_medium_batched_exact_integer(hs):
    """Bidiagonal (1, -1) systems with integer B: running sums exactly, across block rows."""
    import torch
    m, n, batch = 200, 12, 3
    L = np.full((m, m), np.nan)
    L[np.tril_indices(m, -1)] = 0
    L[np.diag_indices(m)] = 1
    L[np.arange(1, m), np.arange(m - 1)] = -1
    rng = np.random.default_rng(5)
    Bm = rng.integers(-30, 30, (batch, m, n)).astype(np.float64)
    dA = to_dev(np.ascontiguousarray(L.T))
    dB = to_dev(np.ascontiguousarray(Bm.transpose(0, 2, 1)))
    assert hs.hsma_trsm_strided_batched_d(m, n, 1.0, dA, m, 0, dB, m, m * n, batch) == hs.SUCCESS
    torch.cuda.synchronize()
    assert np.array_equal(dB.cpu().numpy().transpose(0, 2, 1), np.cumsum(Bm, axis=1))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("m,n", [(64, 64), (40, 9), (128, 64), (200, 33)])
def test_batch_member_equals_solo_solve(hs, dtype, m, n):
    """A problem's result inside a strided batch is bitwise the one it gets when
    solved as a batch of one: nothing in a problem's arithmetic depends on its
    neighbours (small regime and block rows alike)."""
    import torch
    batch = 6
    A, B = colmajor_inputs(dtype, m, n, batch, seed=21 + m + n)
    dA, dB = to_dev(A), to_dev(B)
    f = hs.entry("strided_batched", dtype)
    assert f(m, n, 1.0, dA, m, m * m, dB, m, m * n, batch) == hs.SUCCESS
    for p in (0, 3, 5):
        dA1, dB1 = to_dev(A[p:p + 1]), to_dev(B[p:p + 1])
        assert f(m, n, 1.0, dA1, m, m * m, dB1, m, m * n, 1) == hs.SUCCESS
        torch.cuda.synchronize()
        solo = dB1.cpu().numpy()[0]
        if m > 64:
            # a batch of one takes the blocked path, whose rounding differs: compare
            # against a batch of two holding the same problem twice instead
            dA2, dB2 = to_dev(np.concatenate([A[p:p + 1]] * 2)), to_dev(np.concatenate([B[p:p + 1]] * 2))
            assert f(m, n, 1.0, dA2, m, m * m, dB2, m, m * n, 2) == hs.SUCCESS
            torch.cuda.synchronize()
            solo = dB2.cpu().numpy()[1]
        assert np.array_equal(dB.cpu().numpy()[p], solo)
