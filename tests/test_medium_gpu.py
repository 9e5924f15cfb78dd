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
                                       (256, 33, 4), (192, 64, 50), (300, 20, 3), (512, 64, 4),
                                       (457, 129, 2)])
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


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("m,n", [(30, 5), (65, 1), (128, 64), (200, 300), (256, 17)])
def test_rows64_route_single_problem(hs, dtype, m, n):
    """The block-rows-of-64 route asked for by name on one problem (and on
    m <= 64, where it is one block row), with alpha and padded leading
    dimensions, against the oracle; rows below m stay untouched."""
    import torch
    cplx = dtype.startswith("c")
    alpha = 1.5 - 0.25j if cplx else 0.75
    lda, ldb = m + 3, m + 5
    say("rows64 single", dtype, m, n)
    A, B = colmajor_inputs(dtype, m, n, 1, lda=lda, ldb=ldb, seed=31 + m + n)
    dA, dB = to_dev(A), to_dev(B)
    st = hs.entry("ex", dtype)(m, n, alpha, dA, lda, dB, ldb, {"path": hs.PATH_ROWS64})
    torch.cuda.synchronize()
    assert st == hs.SUCCESS, hs.status_string(st)
    X = dB.cpu().numpy()
    Av, Bv = views(A, B, m)
    assert rel_err(X[:, :, :m].transpose(0, 2, 1), oracle.trsm(Av, Bv, alpha)) <= TOL_LARGE[dtype]
    assert np.array_equal(X[:, :, m:], B[:, :, m:])


@pytest.mark.parametrize("dtype", DTYPES)
def test_rows64_single_equals_batch_member(hs, dtype):
    """One problem through the block-rows route gives bitwise the result it
    gets as a member of a strided batch (which always takes that route)."""
    import torch
    m, n, batch = 177, 40, 4
    A, B = colmajor_inputs(dtype, m, n, batch, seed=77)
    dA, dB = to_dev(A), to_dev(B)
    assert hs.entry("strided_batched", dtype)(m, n, 1.0, dA, m, m * m, dB, m, m * n, batch) == hs.SUCCESS
    dA1, dB1 = to_dev(A[2:3]), to_dev(B[2:3])
    assert hs.entry("ex", dtype)(m, n, 1.0, dA1, m, dB1, m, {"path": hs.PATH_ROWS64}) == hs.SUCCESS
    torch.cuda.synchronize()
    assert np.array_equal(dB.cpu().numpy()[2], dB1.cpu().numpy()[0])


@pytest.mark.parametrize("dtype", DTYPES)
def test_single_problem_auto_route(hs, dtype):
    """AUTO on one problem takes the block-rows route for 64 < m <= 192 with
    n <= 16 and the blocked path otherwise (bitwise the explicit routes)."""
    import torch
    f = hs.entry("ex", dtype)
    for m, n, want in ((177, 1, hs.PATH_ROWS64), (177, 16, hs.PATH_ROWS64), (192, 9, hs.PATH_ROWS64),
                       (177, 17, hs.PATH_BLOCKED), (193, 4, hs.PATH_BLOCKED), (256, 1, hs.PATH_BLOCKED)):
        say("single auto route", dtype, m, n)
        A, B = colmajor_inputs(dtype, m, n, 1, seed=n)
        dA, dB1, dB2 = to_dev(A), to_dev(B), to_dev(B)
        assert f(m, n, 1.0, dA, m, dB1, m, {"path": hs.PATH_AUTO}) == hs.SUCCESS
        assert f(m, n, 1.0, dA, m, dB2, m, {"path": want}) == hs.SUCCESS
        torch.cuda.synchronize()
        assert np.array_equal(dB1.cpu().numpy(), dB2.cpu().numpy()), (m, n)
