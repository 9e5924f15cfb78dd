"""Pins for the CPU oracle (oracle/), all on the CPU.

The oracle is checked against things other than itself: exact rational
arithmetic (with a multiply-back check of the exact solution), LAPACK's
triangular solver (scipy.linalg.solve_triangular), closed forms, and
invariants of the definition X = tril(A)^{-1} (alpha B). A planted-mistake test
compiles mutated copies of oracle.c and requires these pins to reject each.
"""
import ctypes
import os
import random
import re
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth

EPS64 = np.finfo(np.float64).eps


def colview(Acol):
    """(batch, m, ld) column-major storage -> (batch, m, m) view with [b, i, j]."""
    m = Acol.shape[1]
    return Acol[:, :, :m].transpose(0, 2, 1)


def rowview(Arow, n=None):
    """(batch, m, ld) row-major storage -> (batch, m, n) view with [b, i, j]."""
    n = Arow.shape[1] if n is None else n
    return Arow[:, :, :n]


def exact_solve(A, b, alpha=1):
    """Forward substitution in exact rationals; A, b given as exact values."""
    m = len(b)
    x = [None] * m
    for i in range(m):
        s = Fraction(alpha) * Fraction(b[i])
        for j in range(i):
            s -= Fraction(A[i][j]) * x[j]
        x[i] = s / Fraction(A[i][i])
    # multiply back: tril(A) x must reproduce alpha*b exactly
    for i in range(m):
        assert sum(Fraction(A[i][j]) * x[j] for j in range(i + 1)) == Fraction(alpha) * Fraction(b[i])
    return x


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6])
def test_exact_rational_real(m):
    A = colview(synth.tri("f64", m, seed=100 + m))[0]
    B = synth.rhs("f64", m, 3, seed=200 + m).transpose(0, 2, 1)[0]
    X = oracle.trsm(A, B, alpha=1.0)
    for c in range(3):
        xe = exact_solve([[float(A[i, j]) for j in range(m)] for i in range(m)],
                         [float(v) for v in B[:, c]])
        xe = np.array([float(v) for v in xe])
        err = np.linalg.norm(X[:, c] - xe) / np.linalg.norm(xe)
        assert err <= 8 * m * EPS64, err


def test_exact_dyadic_bitwise():
    """Integer off-diagonals, power-of-two diagonals, integer B: the exact
    solution is a short dyadic rational, so double arithmetic is exact."""
    rng = random.Random(7)
    checked = 0
    for trial in range(200):
        m = rng.randint(1, 8)
        A = np.full((m, m), np.nan)
        for i in range(m):
            A[i, i] = rng.choice([1.0, 2.0, 4.0, 0.5, -1.0, -2.0])
            for j in range(i):
                A[i, j] = float(rng.randint(-3, 3))
        B = np.array([[float(rng.randint(-9, 9)) for _ in range(2)] for _ in range(m)])
        xe = [exact_solve(A.tolist(), B[:, c].tolist()) for c in range(2)]
        if any(abs(v.numerator) >= 2 ** 50 or (v.denominator & (v.denominator - 1)) or v.denominator > 2 ** 20
               for col in xe for v in col):
            continue
        X = oracle.trsm(A, B)
        for c in range(2):
            assert [float(v) for v in xe[c]] == X[:, c].tolist()
        checked += 1
    assert checked > 150


def test_exact_gaussian_integer_complex():
    """Complex with Gaussian-integer entries and unit-modulus diagonals (1, -1, i, -i):
    exact solution is Gaussian-integer, double arithmetic exact."""
    rng = random.Random(11)
    for trial in range(60):
        m = rng.randint(1, 6)
        A = np.full((m, m), np.nan + 1j * np.nan)
        for i in range(m):
            A[i, i] = rng.choice([1, -1, 1j, -1j])
            for j in range(i):
                A[i, j] = complex(rng.randint(-2, 2), rng.randint(-2, 2))
        B = np.array([[complex(rng.randint(-5, 5), rng.randint(-5, 5))] for _ in range(m)])
        # exact solve over Gaussian rationals: represent as (re, im) Fractions
        x = []
        for i in range(m):
            sr, si = Fraction(B[i, 0].real), Fraction(B[i, 0].imag)
            for j in range(i):
                ar, ai = Fraction(A[i, j].real), Fraction(A[i, j].imag)
                xr, xi = x[j]
                sr -= ar * xr - ai * xi
                si -= ar * xi + ai * xr
            dr, di = Fraction(A[i, i].real), Fraction(A[i, i].imag)
            den = dr * dr + di * di
            x.append(((sr * dr + si * di) / den, (si * dr - sr * di) / den))
        X = oracle.trsm(A.astype(np.complex128), B.astype(np.complex128))
        for i in range(m):
            assert X[i, 0] == complex(float(x[i][0]), float(x[i][1]))


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c128"])
def test_lapack_trtrs(dtype):
    """Against LAPACK's triangular solve on the upcast lower triangle."""
    m, n = 100, 7
    A = colview(synth.tri(dtype, m, seed=5))[0]
    B = synth.rhs(dtype, m, n, seed=6).transpose(0, 2, 1)[0]
    X = oracle.trsm(A, B, alpha=0.75 + (0.5j if dtype.startswith("c") else 0))
    big = np.complex128 if dtype.startswith("c") else np.float64
    alpha = 0.75 + (0.5j if dtype.startswith("c") else 0)
    ref = scipy.linalg.solve_triangular(np.tril(np.nan_to_num(A.astype(big))), alpha * B.astype(big),
                                        lower=True)
    err = np.linalg.norm(X - ref) / np.linalg.norm(ref)
    assert err < 1e-13, err
    # scaled residual in double
    AL = np.tril(np.nan_to_num(A.astype(big)))
    res = np.linalg.norm(AL @ X - alpha * B.astype(big)) / (np.linalg.norm(AL) * np.linalg.norm(X))
    assert res <= 10 * m * EPS64


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c128"])
def test_identity(dtype):
    m, n = 17, 5
    A = np.full((m, m), np.nan, dtype=synth.NP_DTYPE[dtype])
    A[np.tril_indices(m, -1)] = 0
    A[np.diag_indices(m)] = 1
    B = synth.rhs(dtype, m, n, seed=1).transpose(0, 2, 1)[0]
    for alpha in (1.0, 2.0, -0.5):
        X = oracle.trsm(A, B, alpha)
        assert np.array_equal(X, alpha * B.astype(X.dtype))


def test_diagonal_correctly_rounded():
    m, n = 33, 4
    A = colview(synth.tri("f64", m, seed=3))[0].copy()
    A[np.tril_indices(m, -1)] = 0.0
    B = synth.rhs("f64", m, n, seed=4).transpose(0, 2, 1)[0]
    X = oracle.trsm(A, B, alpha=3.0)
    assert np.array_equal(X, (3.0 * B) / np.diag(A)[:, None])


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c128"])
def test_bidiagonal_prefix_sums(dtype):
    """1 on the diagonal, -1 below it: X is the running sum of B down each column."""
    m, n = 40, 6
    A = np.full((m, m), np.nan, dtype=synth.NP_DTYPE[dtype])
    A[np.tril_indices(m, -1)] = 0
    A[np.diag_indices(m)] = 1
    A[np.arange(1, m), np.arange(m - 1)] = -1
    rng = np.random.default_rng(0)
    B = rng.integers(-50, 50, size=(m, n)).astype(synth.NP_DTYPE[dtype])
    if dtype.startswith("c"):
        B = B + 1j * rng.integers(-50, 50, size=(m, n)).astype(synth.NP_DTYPE[dtype])
    X = oracle.trsm(A, B)
    assert np.array_equal(X, np.cumsum(B.astype(X.dtype), axis=0))


def test_all_ones_lower_differences():
    """All ones on and below the diagonal: x_0 = b_0, x_i = b_i - b_{i-1}."""
    m, n = 31, 3
    A = np.full((m, m), np.nan)
    A[np.tril_indices(m)] = 1.0
    rng = np.random.default_rng(1)
    B = rng.integers(-1000, 1000, size=(m, n)).astype(np.float64)
    X = oracle.trsm(A, B)
    expect = B.copy()
    expect[1:] -= B[:-1]
    assert np.array_equal(X, expect)


@pytest.mark.parametrize("dtype", ["f32", "c128"])
def test_column_independence_and_threads(dtype):
    m, n = 64, 20
    A = colview(synth.tri(dtype, m, seed=9))[0]
    B = synth.rhs(dtype, m, n, seed=10).transpose(0, 2, 1)[0]
    X1 = oracle.trsm(A, B, threads=1)
    X7 = oracle.trsm(A, B, threads=7)
    assert np.array_equal(X1, X7)
    S = [3, 4, 17, 19]
    XS = oracle.trsm(A, np.ascontiguousarray(B[:, S]))
    assert np.array_equal(XS, X1[:, S])


@pytest.mark.parametrize("dtype", ["f64", "c64"])
def test_upper_triangle_never_read(dtype):
    m, n = 25, 4
    Anan = colview(synth.tri(dtype, m, seed=12, upper="nan"))[0]
    Azero = colview(synth.tri(dtype, m, seed=12, upper="zero"))[0]
    B = synth.rhs(dtype, m, n, seed=13).transpose(0, 2, 1)[0]
    Xn = oracle.trsm(Anan, B)
    assert np.isfinite(Xn).all()
    assert np.array_equal(Xn, oracle.trsm(Azero, B))


def test_alpha_scaling_exact():
    m, n = 50, 3
    A = colview(synth.tri("f64", m, seed=14))[0]
    B = synth.rhs("f64", m, n, seed=15).transpose(0, 2, 1)[0]
    assert np.array_equal(oracle.trsm(A, B, 2.0), 2.0 * oracle.trsm(A, B, 1.0))
    assert np.array_equal(oracle.trsm(A, B, 0.0), np.zeros((m, n)))


def test_complex_with_zero_imaginary_matches_real():
    m, n = 30, 2
    A = colview(synth.tri("f64", m, seed=16))[0]
    B = synth.rhs("f64", m, n, seed=17).transpose(0, 2, 1)[0]
    Xr = oracle.trsm(A, B)
    Xc = oracle.trsm(A.astype(np.complex128), B.astype(np.complex128))
    assert np.all(Xc.imag == 0)
    assert np.allclose(Xc.real, Xr, rtol=8 * EPS64, atol=0)


def test_layouts_and_batches_agree():
    """Row-major (ggml) and column-major storage of the same logical problems give
    the same bits; batched calls equal per-problem calls."""
    m, n, batch = 64, 6, 8
    Acol = colview(synth.tri("f32", m, batch, seed=18, offdiag_div=64))
    Arow = rowview(synth.tri("f32", m, batch, seed=18, offdiag_div=64, layout="row"))
    assert np.array_equal(np.nan_to_num(Acol), np.nan_to_num(Arow))
    Bcol = synth.rhs("f32", m, n, batch, seed=19).transpose(0, 2, 1)
    Brow = synth.rhs("f32", m, n, batch, seed=19, layout="row")
    X1 = oracle.trsm(Acol, Bcol)
    X2 = oracle.trsm(Arow, Brow)
    assert np.array_equal(X1, X2)
    for b in range(batch):
        assert np.array_equal(X1[b], oracle.trsm(Acol[b], Bcol[b]))


def test_gemm_against_numpy():
    rng = np.random.default_rng(2)
    for dt, tol in (("f32", 1e-12), ("f64", 1e-13), ("c64", 1e-12), ("c128", 1e-13)):
        A = rng.standard_normal((13, 29))
        B = rng.standard_normal((29, 11))
        if dt.startswith("c"):
            A = A + 1j * rng.standard_normal(A.shape)
            B = B + 1j * rng.standard_normal(B.shape)
        A = A.astype(synth.NP_DTYPE[dt])
        B = B.astype(synth.NP_DTYPE[dt])
        big = np.complex128 if dt.startswith("c") else np.float64
        C = oracle.gemm(A, B)
        ref = A.astype(big) @ B.astype(big)
        assert np.linalg.norm(C - ref) <= tol * np.linalg.norm(ref)
    Ai = rng.integers(-8, 8, (16, 16)).astype(np.float64)
    Bi = rng.integers(-8, 8, (16, 5)).astype(np.float64)
    assert np.array_equal(oracle.gemm(Ai, Bi), Ai @ Bi)


def test_empty_problems():
    A = np.zeros((0, 0))
    B = np.zeros((0, 3))
    assert oracle.trsm(A, B).shape == (0, 3)
    A = colview(synth.tri("f64", 4, seed=1))[0]
    assert oracle.trsm(A, np.zeros((4, 0))).shape == (4, 0)


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant of oracle.c must fail at least one pin.

MUTANTS = {
    "sign": ("w[2 * i] -= ar * xr - ai * xi;", "w[2 * i] += ar * xr - ai * xi;"),
    "real_sign": ("w[2 * i] -= ar * xr;\n", "w[2 * i] += ar * xr;\n"),
    "dropped_term": ("for (int64_t i = j + 1; i < m; ++i) {", "for (int64_t i = j + 2; i < m; ++i) {"),
    "transposed": ("get(J->dtype, J->A, b * J->sab + i * J->sai + j * J->saj, &ar, &ai);",
                   "get(J->dtype, J->A, b * J->sab + j * J->sai + i * J->saj, &ar, &ai);"),
    "conj_div": ("xi = (w[2 * j + 1] * dr - w[2 * j] * di) / den;",
                 "xi = (w[2 * j + 1] * dr + w[2 * j] * di) / den;"),
    "alpha_im": ("w[2 * i + 1] = J->ar * bi + J->ai * br;", "w[2 * i + 1] = J->ar * bi - J->ai * br;"),
}


def _pins_pass(lib):
    """A compact run of the pins above against a library handle; True if all pass."""
    i64, p, i = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.oracle_trsm.argtypes = [i, i64, i64, i64, p, p, i64, i64, i64, p, i64, i64, i64, p, i]

    def solve(A, B, alpha=1.0):
        dt = {np.float64: "f64", np.complex128: "c128"}[A.dtype.type]
        m, n = B.shape
        X = np.empty((n, m), dtype=np.complex128 if dt == "c128" else np.float64)
        al = np.array([complex(alpha).real, complex(alpha).imag])
        sai, saj = (s // A.itemsize for s in A.strides)
        sbi, sbj = (s // B.itemsize for s in B.strides)
        lib.oracle_trsm(oracle.CODE[dt], m, n, 1, al.ctypes.data, A.ctypes.data, sai, saj, 0,
                        B.ctypes.data, sbi, sbj, 0, X.ctypes.data, 1)
        return X.T

    ok = True
    for dt in ("f64", "c128"):
        m = 60
        A = colview(synth.tri(dt, m, seed=5))[0]
        B = synth.rhs(dt, m, 4, seed=6).transpose(0, 2, 1)[0]
        alpha = 0.75 + (0.5j if dt == "c128" else 0)
        X = solve(A, B, alpha)
        big = np.complex128 if dt == "c128" else np.float64
        ref = scipy.linalg.solve_triangular(np.tril(np.nan_to_num(A)).astype(big), alpha * B.astype(big),
                                            lower=True)
        ok &= bool(np.all(np.isfinite(X))) and np.linalg.norm(X - ref) <= 1e-13 * np.linalg.norm(ref)
    return ok


def test_planted_mistakes_are_caught():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    with tempfile.TemporaryDirectory() as td:
        # the unmutated source passes the compact pins
        path = os.path.join(td, "o.c")
        so = os.path.join(td, "o.so")
        open(path, "w").write(src)
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-o", so, path,
                               "-lpthread"])
        assert _pins_pass(ctypes.CDLL(so))
        for name, (old, new) in MUTANTS.items():
            assert src.count(old) == 1, name
            path = os.path.join(td, name + ".c")
            so = os.path.join(td, name + ".so")
            open(path, "w").write(src.replace(old, new))
            subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-o", so, path,
                                   "-lpthread"])
            assert not _pins_pass(ctypes.CDLL(so)), "mutant %s not caught" % name
