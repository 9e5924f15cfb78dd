"""CPU oracle for the lower-triangular solve A*X = alpha*B (see oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
bench.py's CPU-baseline leg, never by the library. It shares no code with the
HIP path. Every function computes in double precision and returns float64 or
complex128 numpy arrays.

Pinned by tests/test_oracle.py against exact rational arithmetic, LAPACK's
triangular solver, closed forms and invariants; no function here is "parity
unpinned".
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CODE = {"f32": 0, "f64": 1, "c64": 2, "c128": 3}
NP_DTYPE = {"f32": np.float32, "f64": np.float64, "c64": np.complex64, "c128": np.complex128}
COMPLEX = {"c64", "c128"}


def build(force=False):
    """Compile oracle.c (gcc -O2 -ffp-contract=off, plain C, pthreads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                               "-o", tmp, _SRC, "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _get():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, p, i = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.oracle_trsm.argtypes = [i, i64, i64, i64, p, p, i64, i64, i64, p, i64, i64, i64, p, i]
        lib.oracle_trsm.restype = i
        lib.oracle_gemm.argtypes = [i, i64, i64, i64, p, i64, i64, p, i64, i64, p]
        lib.oracle_gemm.restype = i
        lib.oracle_trsm_general.argtypes = [i, i, i, i, i, i64, i64, i64, p, p, i64, i64, i64,
                                            p, i64, i64, i64, p, i]
        lib.oracle_trsm_general.restype = i
        _lib = lib
    return _lib


def default_threads():
    return max(1, min(16, os.cpu_count() or 1))


def _dtype_of(arr):
    for k, v in NP_DTYPE.items():
        if arr.dtype == v:
            return k
    raise TypeError("unsupported dtype %s" % arr.dtype)


def _strides(arr):
    return tuple(s // arr.itemsize for s in arr.strides)


def trsm(A, B, alpha=1.0, threads=None):
    """X = tril(A)^{-1} (alpha B) per problem, in double precision.

    A: (batch, m, m) array view whose [b, i, j] is element (i, j) of problem b
       (any strides; the upper triangle is never read).
    B: (batch, m, n) array view, [b, i, c] = element (i, c).
    Returns X as (batch, m, n) float64 / complex128.
    """
    A = np.asarray(A)
    B = np.asarray(B)
    if A.ndim == 2:
        return trsm(A[None], B[None], alpha, threads)[0]
    dt = _dtype_of(A)
    if _dtype_of(B) != dt:
        raise TypeError("A and B dtypes differ")
    batch, m, m2 = A.shape
    b2, mb, n = B.shape
    if m != m2 or mb != m or b2 != batch:
        raise ValueError("shape mismatch")
    sab, sai, saj = _strides(A)
    sbb, sbi, sbj = _strides(B)
    if batch == 1:
        sab = sbb = 0
    cp = dt in COMPLEX
    X = np.empty((batch, n, m), dtype=np.complex128 if cp else np.float64)  # column-major per problem
    al = np.array([complex(alpha).real, complex(alpha).imag], dtype=np.float64)
    rc = _get().oracle_trsm(CODE[dt], m, n, batch, al.ctypes.data,
                            A.ctypes.data, sai, saj, sab, B.ctypes.data, sbi, sbj, sbb,
                            X.ctypes.data, threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_trsm failed")
    return X.transpose(0, 2, 1)


SIDE = {"L": 0, "R": 1}
UPLO = {"L": 0, "U": 1}
TRANS = {"N": 0, "T": 1, "C": 2}
DIAG = {"N": 0, "U": 1}


def trsm_general(A, B, side="L", uplo="L", trans="N", diag="N", alpha=1.0, threads=None):
    """One TRSM variant per problem, in double precision (see oracle.c):
    side "L": op(A) X = alpha B; side "R": X op(A) = alpha B; op = "N", "T" or
    "C" (conjugate transpose); uplo "L"/"U" says which triangle of A is used
    (the other is never read); diag "U": unit diagonal (never read).

    A: (batch, k, k) array view, [b, i, j] = element (i, j), k = m for the left
       side and n for the right side (any strides).
    B: (batch, m, n) array view, [b, i, c] = element (i, c).
    Returns X as (batch, m, n) float64 / complex128.
    """
    A = np.asarray(A)
    B = np.asarray(B)
    if A.ndim == 2:
        return trsm_general(A[None], B[None], side, uplo, trans, diag, alpha, threads)[0]
    dt = _dtype_of(A)
    if _dtype_of(B) != dt:
        raise TypeError("A and B dtypes differ")
    batch, k, k2 = A.shape
    b2, m, n = B.shape
    if k != k2 or b2 != batch or k != (m if side == "L" else n):
        raise ValueError("shape mismatch")
    sab, sai, saj = _strides(A)
    sbb, sbi, sbj = _strides(B)
    if batch == 1:
        sab = sbb = 0
    cp = dt in COMPLEX
    X = np.empty((batch, n, m), dtype=np.complex128 if cp else np.float64)
    al = np.array([complex(alpha).real, complex(alpha).imag], dtype=np.float64)
    rc = _get().oracle_trsm_general(CODE[dt], SIDE[side], UPLO[uplo], TRANS[trans], DIAG[diag],
                                    m, n, batch, al.ctypes.data, A.ctypes.data, sai, saj, sab,
                                    B.ctypes.data, sbi, sbj, sbb, X.ctypes.data,
                                    threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_trsm_general failed")
    return X.transpose(0, 2, 1)


def gemm(A, B):
    """C = A @ B in double precision with plain triple loops (A: M x K, B: K x N)."""
    A = np.asarray(A)
    B = np.asarray(B)
    dt = _dtype_of(A)
    if _dtype_of(B) != dt:
        raise TypeError("A and B dtypes differ")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("shape mismatch")
    sai, saj = _strides(A)
    sbi, sbj = _strides(B)
    cp = dt in COMPLEX
    C = np.empty((N, M), dtype=np.complex128 if cp else np.float64)
    rc = _get().oracle_gemm(CODE[dt], M, N, K, A.ctypes.data, sai, saj, B.ctypes.data, sbi, sbj,
                            C.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_gemm failed")
    return C.T
