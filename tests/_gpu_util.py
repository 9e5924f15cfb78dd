"""Helpers for the GPU parity tests: seeded inputs from synth, the solve through
the C ABI binding, the reference from the CPU oracle, and the error measures."""
import sys

import numpy as np

import oracle
import synth

# Parity bars (relative Frobenius error of X against the oracle, per problem).
TOL_SMALL = {"f32": 1e-5, "c64": 1e-5, "f64": 1e-12, "c128": 1e-12}
TOL_LARGE = {"f32": 1e-4, "c64": 1e-4, "f64": 1e-12, "c128": 1e-12}
EPS = {"f32": 2.0 ** -23, "c64": 2.0 ** -23, "f64": 2.0 ** -52, "c128": 2.0 ** -52}
TORCH_DTYPE_NAME = {"f32": "float32", "f64": "float64", "c64": "complex64", "c128": "complex128"}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(arr):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def rel_err(Xg, Xo):
    """Max over problems of ||Xg - Xo||_F / ||Xo||_F (arrays [batch, m, n]),
    both scaled by the problem's largest |Xo| first so that the squares
    cannot overflow."""
    Xg = Xg.astype(Xo.dtype)
    sc = np.max(np.abs(Xo), axis=(-2, -1), keepdims=True)
    sc = np.where(sc == 0, 1.0, sc)
    num = np.sqrt(np.sum(np.abs((Xg - Xo) / sc) ** 2, axis=(-2, -1)))
    den = np.sqrt(np.sum(np.abs(Xo / sc) ** 2, axis=(-2, -1)))
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))


def scaled_residual(A, X, B, alpha):
    """Max over problems of ||tril(A) X - alpha B||_F / (||tril(A)||_F ||X||_F), in double."""
    big = np.complex128 if np.iscomplexobj(A) else np.float64
    AL = np.tril(np.nan_to_num(A.astype(big), nan=0.0))
    Xd = X.astype(big)
    R = AL @ Xd - alpha * B.astype(big)
    num = np.sqrt(np.sum(np.abs(R) ** 2, axis=(-2, -1)))
    den = np.sqrt(np.sum(np.abs(AL) ** 2, axis=(-2, -1))) * np.sqrt(np.sum(np.abs(Xd) ** 2, axis=(-2, -1)))
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))


def colmajor_inputs(dtype, m, n, batch, lda=None, ldb=None, seed=0, shared_a=False, offdiag_div=None):
    """Column-major storage: A (batchA, m, lda) with [b, j, :m] = column j; B (batch, n, ldb)."""
    lda = lda or max(1, m)
    ldb = ldb or max(1, m)
    A = synth.tri(dtype, m, 1 if shared_a else batch, seed=seed, ld=lda, offdiag_div=offdiag_div)
    B = synth.rhs(dtype, m, n, batch, seed=seed + 1, ld=ldb)
    return A, B


def views(A, B, m):
    """[b, i, j] views of column-major storage."""
    return A[:, :, :m].transpose(0, 2, 1), B[:, :, :m].transpose(0, 2, 1)
