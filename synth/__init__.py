"""Seeded synthetic inputs for the triangular solve (see synth.c for the recipe).

Shared by the CPU oracle's tests and by the HIP library's tests and benchmark:
both sides get the same arrays from here. Nothing in this module performs any
step of the solve.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

DTYPES = ("f32", "f64", "c64", "c128")
NP_DTYPE = {"f32": np.float32, "f64": np.float64, "c64": np.complex64, "c128": np.complex128}
CODE = {"f32": 0, "f64": 1, "c64": 2, "c128": 3}

# Tags keep A and B streams apart for the same seed.
TAG_A = 0x41
TAG_B = 0x42


def build(force=False):
    """Compile synth.c into libsynth.so (gcc, plain C)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                               "-o", tmp, _SRC, "-lpthread", "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _get():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, u64, p, d, i = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p,
                             ctypes.c_double, ctypes.c_int)
        lib.synth_fill_tri.argtypes = [i, i64, i64, d, u64, u64, p, i64, i64, i64, i, i]
        lib.synth_fill_rhs.argtypes = [i, i64, i64, i64, u64, u64, p, i64, i64, i64, p, i]
        lib.synth_pick.argtypes = [i64, i64, u64, p, p]
        lib.synth_mix64.argtypes = [u64]
        lib.synth_mix64.restype = u64
        _lib = lib
    return _lib


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def mix64(z):
    return int(_get().synth_mix64(ctypes.c_uint64(z)))


def tri(dtype, m, batch=1, seed=0, offdiag_div=None, upper="nan", layout="col", ld=None):
    """Batch of lower-triangular m x m matrices as a numpy array.

    layout "col": shape (batch, m, ld) where [b, j, :m] is column j (column-major,
    leading dimension ld >= m); layout "row": shape (batch, m, ld) where [b, i, :m]
    is row i (row-major, ggml style). Padding elements are zero.
    upper: "nan" (garbage above the diagonal), "zero".
    """
    ld = m if ld is None else ld
    div = float(m) if offdiag_div is None else float(offdiag_div)
    out = np.zeros((batch, m, ld), dtype=NP_DTYPE[dtype])
    if out.size == 0:
        return out
    rs, cs = (1, ld) if layout == "col" else (ld, 1)
    _get().synth_fill_tri(CODE[dtype], m, batch, div, seed, TAG_A, out.ctypes.data,
                          rs, cs, m * ld, {"nan": 0, "zero": 1}[upper], _threads())
    return out


def rhs(dtype, m, n, batch=1, seed=0, layout="col", ld=None, cols=None):
    """Batch of m x n right-hand sides as a numpy array.

    layout "col": shape (batch, n, ld), [b, c, :m] is column c; layout "row":
    shape (batch, m, ld) with ld >= n, [b, i, :n] is row i. With cols given, output
    column c holds logical column cols[c] of the full right-hand side.
    """
    if cols is not None:
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        n = len(cols)
    if layout == "col":
        ld = m if ld is None else ld
        out = np.zeros((batch, n, ld), dtype=NP_DTYPE[dtype])
        rs, cs, bs = 1, ld, n * ld
    else:
        ld = n if ld is None else ld
        out = np.zeros((batch, m, ld), dtype=NP_DTYPE[dtype])
        rs, cs, bs = ld, 1, m * ld
    if out.size == 0:
        return out
    _get().synth_fill_rhs(CODE[dtype], m, n, batch, seed, TAG_B, out.ctypes.data, rs, cs, bs,
                          None if cols is None else cols.ctypes.data, _threads())
    return out


def pick_columns(n, k, seed):
    """k distinct sorted column indices out of n, drawn from the seed."""
    work = np.empty(n, dtype=np.int64)
    out = np.empty(k, dtype=np.int64)
    _get().synth_pick(n, k, seed, work.ctypes.data, out.ctypes.data)
    return out
