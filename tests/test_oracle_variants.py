"""Pins for the oracle's TRSM variants (oracle.trsm_general), all on the CPU.

Each variant (side, triangle, op = N/T/C, unit diagonal) is checked against
things other than the oracle itself: LAPACK's triangular solver
(scipy.linalg.solve_triangular; right-side systems through the transposed
problem), and exact dyadic / Gaussian-integer systems solved by Gauss-Jordan
elimination on the explicitly formed op(A) in rational arithmetic (a
different method from substitution), bitwise. The triangle not used, and the
diagonal of a unit-diagonal system, hold NaN, so a read of them shows.
Planted mistakes in the variant code must fail these pins.
"""
import ctypes
import itertools
import os
import random
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth

VARIANTS = list(itertools.product("LR", "LU", "NTC", "NU"))
EPS64 = np.finfo(np.float64).eps


def stored_matrix(dt, k, uplo, diag, seed):
    """k x k column-major A holding a triangle of the synthetic distribution
    (lower from synth; upper = its transpose), NaN in the other triangle and,
    for a unit diagonal, on the diagonal. Returned as the [i, j] view."""
    L = synth.tri(dt, k, seed=seed)[0].T.copy()          # [i, j], NaN above the diagonal
    A = L if uplo == "L" else L.T.copy()
    if diag == "U":
        A[np.diag_indices(k)] = np.nan
    return A


def op_dense(A, uplo, trans, diag):
    """op(A) as a dense complex128/float64 matrix with the unused triangle zero."""
    big = np.complex128 if np.iscomplexobj(A) else np.float64
    T = np.nan_to_num(A.astype(big), nan=0.0)
    T = np.tril(T) if uplo == "L" else np.triu(T)
    if diag == "U":
        T[np.diag_indices(len(T))] = 1
    if trans == "T":
        T = T.T
    elif trans == "C":
        T = T.conj().T
    return T


def lapack_ref(A, B, side, uplo, trans, diag, alpha):
    big = np.complex128 if np.iscomplexobj(A) else np.float64
    Ad = np.nan_to_num(A.astype(big), nan=0.0)
    Ad = np.tril(Ad) if uplo == "L" else np.triu(Ad)
    Bd = alpha * B.astype(big)
    unit = diag == "U"
    if side == "L":
        return scipy.linalg.solve_triangular(Ad, Bd, trans={"N": 0, "T": 1, "C": 2}[trans],
                                             lower=uplo == "L", unit_diagonal=unit, check_finite=False)
    # X op(A) = alpha B  <=>  op(A)^T X^T = alpha B^T
    if trans == "N":
        Xt = scipy.linalg.solve_triangular(Ad, Bd.T, trans=1, lower=uplo == "L", unit_diagonal=unit,
                                           check_finite=False)
    elif trans == "T":
        Xt = scipy.linalg.solve_triangular(Ad, Bd.T, trans=0, lower=uplo == "L", unit_diagonal=unit,
                                           check_finite=False)
    else:   # op(A)^T = conj(A)
        Xt = scipy.linalg.solve_triangular(Ad.conj(), Bd.T, trans=0, lower=uplo == "L",
                                           unit_diagonal=unit, check_finite=False)
    return Xt.T


@pytest.mark.parametrize("dt", ["f32", "f64", "c64", "c128"])
@pytest.mark.parametrize("side,uplo,trans,diag", VARIANTS)
def test_lapack_variants(dt, side, uplo, trans, diag):
    m, n = 37, 23
    k = m if side == "L" else n
    A = stored_matrix(dt, k, uplo, diag, seed=11)
    B = synth.rhs(dt, m, n, seed=12)[0].T
    alpha = 0.75 - (0.5j if dt.startswith("c") else 0)
    X = oracle.trsm_general(A, B, side, uplo, trans, diag, alpha)
    ref = lapack_ref(A, B, side, uplo, trans, diag, alpha)
    assert np.isfinite(X).all()
    assert np.linalg.norm(X - ref) <= 1e-13 * np.linalg.norm(ref)
    # scaled residual of the defining equation in double
    T = op_dense(A, uplo, trans, diag)
    R = (T @ X if side == "L" else X @ T) - alpha * B.astype(T.dtype)
    assert np.linalg.norm(R) <= 10 * k * EPS64 * np.linalg.norm(T) * np.linalg.norm(X)


def gauss_jordan(T, rhs):
    """Exact solution of T y = rhs (T square, entries (re, im) Fractions) by
    Gauss-Jordan elimination with row pivoting."""
    k = len(T)
    M = [[T[i][j] for j in range(k)] + [rhs[i]] for i in range(k)]
    mul = lambda a, b: (a[0] * b[0] - a[1] * b[1], a[0] * b[1] + a[1] * b[0])
    sub = lambda a, b: (a[0] - b[0], a[1] - b[1])

    def div(a, b):
        d = b[0] * b[0] + b[1] * b[1]
        return ((a[0] * b[0] + a[1] * b[1]) / d, (a[1] * b[0] - a[0] * b[1]) / d)
    zero = (Fraction(0), Fraction(0))
    for c in range(k):
        p = next(r for r in range(c, k) if M[r][c] != zero)
        M[c], M[p] = M[p], M[c]
        piv = M[c][c]
        M[c] = [div(v, piv) for v in M[c]]
        for r in range(k):
            if r != c and M[r][c] != zero:
                f = M[r][c]
                M[r] = [sub(M[r][j], mul(f, M[c][j])) for j in range(k + 1)]
    return [M[i][k] for i in range(k)]


def frac(z):
    z = complex(z)
    return (Fraction(z.real), Fraction(z.imag))


def exact_variant(A, B, side, uplo, trans, diag):
    """Exact X of the variant: the dense op(A) formed exactly, each vector by Gauss-Jordan."""
    T = op_dense(A, uplo, trans, diag)
    Tf = [[frac(v) for v in row] for row in T]
    m, n = B.shape
    X = [[None] * n for _ in range(m)]
    if side == "L":
        for c in range(n):
            y = gauss_jordan(Tf, [frac(B[i, c]) for i in range(m)])
            for i in range(m):
                X[i][c] = y[i]
    else:   # x T = b  <=>  T^T x^T = b^T
        TT = [[Tf[j][i] for j in range(n)] for i in range(n)]
        for r in range(m):
            y = gauss_jordan(TT, [frac(B[r, j]) for j in range(n)])
            for j in range(n):
                X[r][j] = y[j]
    return X


def representable(X):
    return all(abs(v.numerator) < 2 ** 50 and v.denominator <= 2 ** 20 and
               not (v.denominator & (v.denominator - 1)) for row in X for e in row for v in e)


@pytest.mark.parametrize("side,uplo,trans,diag", VARIANTS)
def test_exact_dyadic_variants_bitwise(side, uplo, trans, diag):
    """Integer off-diagonals, power-of-two (or unit) diagonals, integer B:
    a dyadic exact solution, which double arithmetic reaches exactly."""
    rng = random.Random(hash((side, uplo, trans, diag)) & 0xffff)
    checked = 0
    for trial in range(60):
        m, n = rng.randint(1, 6), rng.randint(1, 5)
        k = m if side == "L" else n
        A = np.full((k, k), np.nan)
        for i in range(k):
            A[i, i] = np.nan if diag == "U" else rng.choice([1.0, 2.0, 4.0, 0.5, -1.0, -2.0])
            for j in range(k):
                if (j < i) == (uplo == "L") and i != j:
                    A[i, j] = float(rng.randint(-3, 3))
        B = np.array([[float(rng.randint(-9, 9)) for _ in range(n)] for _ in range(m)])
        Xe = exact_variant(A, B, side, uplo, trans, diag)
        if not representable(Xe):
            continue
        X = oracle.trsm_general(A, B, side, uplo, trans, diag)
        assert [[float(e[0]) for e in row] for row in Xe] == X.tolist()
        checked += 1
    assert checked >= 40


@pytest.mark.parametrize("side,uplo,trans,diag", VARIANTS)
def test_exact_gaussian_integer_variants_bitwise(side, uplo, trans, diag):
    """Gaussian-integer entries, diagonals in {1, -1, i, -i} (or unit): the
    exact solution is Gaussian-integer and double arithmetic reaches it; the
    conjugate transpose differs from the transpose here."""
    rng = random.Random(hash((side, uplo, trans, diag, "c")) & 0xffff)
    for trial in range(25):
        m, n = rng.randint(1, 5), rng.randint(1, 4)
        k = m if side == "L" else n
        A = np.full((k, k), np.nan + 1j * np.nan)
        for i in range(k):
            if diag == "N":
                A[i, i] = rng.choice([1, -1, 1j, -1j])
            for j in range(k):
                if (j < i) == (uplo == "L") and i != j:
                    A[i, j] = complex(rng.randint(-2, 2), rng.randint(-2, 2))
        B = np.array([[complex(rng.randint(-5, 5), rng.randint(-5, 5)) for _ in range(n)]
                      for _ in range(m)])
        Xe = exact_variant(A, B, side, uplo, trans, diag)
        X = oracle.trsm_general(A, B, side, uplo, trans, diag)
        for i in range(m):
            for c in range(n):
                assert X[i, c] == complex(float(Xe[i][c][0]), float(Xe[i][c][1]))


@pytest.mark.parametrize("dt", ["f32", "c128"])
def test_variants_threads_and_base_case(dt):
    """Bitwise independent of the thread count; the base variant gives the
    bits of oracle.trsm (same operation order)."""
    m, n = 50, 33
    for side, uplo, trans, diag in [("L", "U", "C", "N"), ("R", "L", "T", "U")]:
        k = m if side == "L" else n
        A = stored_matrix(dt, k, uplo, diag, seed=3)
        B = synth.rhs(dt, m, n, seed=4)[0].T
        X1 = oracle.trsm_general(A, B, side, uplo, trans, diag, 0.5, threads=1)
        X7 = oracle.trsm_general(A, B, side, uplo, trans, diag, 0.5, threads=7)
        assert np.array_equal(X1, X7)
    A = stored_matrix(dt, m, "L", "N", seed=3)
    B = synth.rhs(dt, m, n, seed=4)[0].T
    assert np.array_equal(oracle.trsm_general(A, B, alpha=2.0), oracle.trsm(A, B, alpha=2.0))


# Planted mistakes in the variant code: each must fail the compact pins below.
GENERAL_MUTANTS = {
    "no_conj": ("if (J->trans == 2) *im = -*im;", "if (J->trans == 3) *im = -*im;"),
    "unit_ignored": ("if (J->diag == 1 && i == j) { *re = 1.0; *im = 0.0; return; }",
                     "if (J->diag == 7 && i == j) { *re = 1.0; *im = 0.0; return; }"),
    "wrong_direction": ("const int forward = left ? op_lower : !op_lower;",
                        "const int forward = left ? op_lower : op_lower;"),
    "right_not_transposed": ("else op_a(J, b, j, i, &opr, &opi);           /* x_j op(A)(j, i) */",
                             "else op_a(J, b, i, j, &opr, &opi);           /* x_j op(A)(j, i) */"),
    "no_transpose": ("const int64_t r = J->trans ? j : i;", "const int64_t r = i;"),
    "rhs_index": ("const int64_t row = left ? i : c, col = left ? c : i;\n        get(",
                  "const int64_t row = left ? i : c, col = left ? c : c;\n        get("),
}


def _general_pins_pass(lib):
    i64, p, i = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.oracle_trsm_general.argtypes = [i, i, i, i, i, i64, i64, i64, p, p, i64, i64, i64,
                                        p, i64, i64, i64, p, i]
    ok = True
    for dt in ("f64", "c128"):
        for side, uplo, trans, diag in VARIANTS:
            if dt == "f64" and trans == "C":
                continue
            m, n = 9, 7
            k = m if side == "L" else n
            A = stored_matrix(dt, k, uplo, diag, seed=21)
            B = synth.rhs(dt, m, n, seed=22)[0].T
            alpha = 0.75 - (0.5j if dt == "c128" else 0)
            X = np.empty((n, m), dtype=np.complex128 if dt == "c128" else np.float64)
            al = np.array([complex(alpha).real, complex(alpha).imag])
            sai, saj = (s // A.itemsize for s in A.strides)
            sbi, sbj = (s // B.itemsize for s in B.strides)
            rc = lib.oracle_trsm_general(oracle.CODE[dt], oracle.SIDE[side], oracle.UPLO[uplo],
                                         oracle.TRANS[trans], oracle.DIAG[diag], m, n, 1,
                                         al.ctypes.data, A.ctypes.data, sai, saj, 0,
                                         B.ctypes.data, sbi, sbj, 0, X.ctypes.data, 1)
            ref = lapack_ref(A, B, side, uplo, trans, diag, alpha)
            ok &= rc == 0 and bool(np.all(np.isfinite(X))) and \
                np.linalg.norm(X.T - ref) <= 1e-13 * np.linalg.norm(ref)
    return ok


def test_planted_mistakes_in_variants_are_caught():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    with tempfile.TemporaryDirectory() as td:
        def compiled(text, name):
            path, so = os.path.join(td, name + ".c"), os.path.join(td, name + ".so")
            open(path, "w").write(text)
            subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-o", so,
                                   path, "-lpthread"])
            return ctypes.CDLL(so)
        assert _general_pins_pass(compiled(src, "o"))
        for name, (old, new) in GENERAL_MUTANTS.items():
            assert src.count(old) == 1, name
            assert not _general_pins_pass(compiled(src.replace(old, new), name)), \
                "mutant %s not caught" % name
