"""GPU parity of the other TRSM variants (side, triangle, op N/T/C, unit
diagonal) against the oracle's variant solve, through the C ABI: the small
regime (order <= 64, strided views), batches of order 64 < k <= 256 (gathered
block rows) and the blocked regime (gathered copies), with padded leading
dimensions and non-square B."""
import itertools

import numpy as np
import pytest

import oracle
import synth
from _gpu_util import TOL_LARGE, TOL_SMALL, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f64", "c64", "c128"]
VARIANTS = list(itertools.product("LR", "LU", "NTC", "NU"))


@pytest.fixture(scope="module")
def hs():
    import torch  # noqa: F401
    import triangular_solve_amd as hs
    return hs


def stored_a(dt, k, lda, uplo, diag, batch, seed):
    """Column-major storage (batch, k, lda) of a k x k triangular A: lower from
    synth, upper = its transpose (synth's row-major layout read column-major);
    NaN in the unused triangle and, for a unit diagonal, on the diagonal."""
    A = synth.tri(dt, k, batch, seed=seed, ld=lda, layout="col" if uplo == "L" else "row")
    if diag == "U":
        idx = np.arange(k)
        A[:, idx, idx] = np.nan
    return A


def run_variant(hs, dt, side, uplo, trans, diag, m, n, batch, alpha, seed, pad=(0, 0)):
    import torch
    k = m if side == "L" else n
    lda, ldb = k + pad[0], m + pad[1]
    A = stored_a(dt, k, lda, uplo, diag, batch, seed)
    B = synth.rhs(dt, m, n, batch, seed=seed + 1, ld=ldb)
    dA, dB = to_dev(A), to_dev(B)
    codes = (hs.SIDE[side], hs.UPLO[uplo], hs.OP[trans], hs.DIAG[diag])
    if batch == 1:
        st = hs.entry("general", dt)(*codes, m, n, alpha, dA, lda, dB, ldb)
    else:
        st = hs.entry("strided_batched_general", dt)(*codes, m, n, alpha, dA, lda, k * lda, dB, ldb,
                                                     n * ldb, batch)
    torch.cuda.synchronize()
    assert st == hs.SUCCESS, st
    Bg = dB.cpu().numpy()
    assert np.array_equal(Bg[:, :, m:], B[:, :, m:])   # ldb padding untouched
    Xg = Bg[:, :, :m].transpose(0, 2, 1)
    Av = A[:, :, :k].transpose(0, 2, 1)
    Bv = B[:, :, :m].transpose(0, 2, 1)
    Xo = oracle.trsm_general(Av, Bv, side, uplo, trans, diag, alpha)
    return Xg, Xo


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("side,uplo,trans,diag", VARIANTS)
def test_variants_small(hs, dt, side, uplo, trans, diag):
    say("variant small", dt, side, uplo, trans, diag)
    alpha = 1.5 - (0.25j if dt.startswith("c") else 0)
    for (m, n, batch, pad) in [(64, 64, 3, (0, 0)), (37, 50, 2, (3, 5)), (64, 6, 4, (0, 0)),
                               (5, 64, 1, (1, 0))]:
        Xg, Xo = run_variant(hs, dt, side, uplo, trans, diag, m, n, batch, alpha, seed=m + n, pad=pad)
        assert rel_err(Xg, Xo) <= TOL_SMALL[dt], (m, n, batch)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("side,uplo,trans,diag", VARIANTS)
def test_variants_medium_batched(hs, dt, side, uplo, trans, diag):
    say("variant medium batched", dt, side, uplo, trans, diag)
    for m, n, batch in ((130, 70, 5), (390, 40, 3)):
        if side != "L":
            m, n = n, m
        Xg, Xo = run_variant(hs, dt, side, uplo, trans, diag, m, n, batch, 1.0, seed=7, pad=(2, 3))
        assert rel_err(Xg, Xo) <= TOL_LARGE[dt], (m, n, batch)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("side,uplo,trans,diag", VARIANTS)
def test_variants_blocked(hs, dt, side, uplo, trans, diag):
    """Orders 700 (several diagonal blocks, a short last one: column
    substitution) and 1024 (blocked-inverse formula), m != n."""
    say("variant blocked", dt, side, uplo, trans, diag)
    alpha = -0.5 + (1j if dt.startswith("c") else 0)
    for k, other in ((700, 90), (1024, 64)):
        m, n = (k, other) if side == "L" else (other, k)
        Xg, Xo = run_variant(hs, dt, side, uplo, trans, diag, m, n, 1, alpha, seed=k, pad=(4, 1))
        assert np.isfinite(Xg).all()
        assert rel_err(Xg, Xo) <= TOL_LARGE[dt], (m, n)


def test_variant_argument_checks(hs):
    f = hs.entry("general", "f64")
    BAD = 0xDEAD000
    assert f(2, 0, 0, 0, 4, 4, 1, BAD, 4, BAD, 4) == hs.INVALID_VALUE
    assert f(0, 0, 3, 0, 4, 4, 1, BAD, 4, BAD, 4) == hs.INVALID_VALUE
    assert f(0, 0, 0, 2, 4, 4, 1, BAD, 4, BAD, 4) == hs.INVALID_VALUE
    assert f(1, 0, 0, 0, 4, 9, 1, BAD, 8, BAD, 4) == hs.INVALID_SIZE   # right: lda >= n
    assert f(1, 0, 0, 0, 4, 9, 1, BAD, 9, BAD, 3) == hs.INVALID_SIZE   # ldb >= m
    assert f(1, 1, 1, 1, 0, 9, 1, None, 9, None, 1) == hs.SUCCESS
