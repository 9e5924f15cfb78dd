"""Python binding of libhsma_trsm.so (include/hsma_trsm.h), argument marshalling only.

Every function has the name and argument order of its C entry point and
returns the C status code (0 = success). Array arguments are device pointers:
pass torch CUDA tensors (their data_ptr() is used) or plain integers.
`stream` is a torch.cuda.Stream, a raw hipStream_t integer, or None for
torch's current stream. All compute happens in the HIP library; there is no
fallback: the first call raises if the library has not been built.

The library is loaded on first use, not at import, so that the build module
(triangular_solve_amd.build) can be imported and run from a checkout that has
no built library yet. A process that has loaded the library keeps that
mapping: rebuild before the first call, not after it.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhsma_trsm.so")

SUCCESS = 0
INVALID_SIZE = 1
INVALID_POINTER = 2
NOT_SUPPORTED = 3
ALLOC_FAILED = 4
HIP_ERROR = 5
INVALID_VALUE = 6
SCRATCH_TOO_SMALL = 7

DTYPE_F32, DTYPE_F64, DTYPE_C64, DTYPE_C128 = 0, 1, 2, 3
SIDE = {"L": 0, "R": 1}
UPLO = {"L": 0, "U": 1}
OP = {"N": 0, "T": 1, "C": 2}
DIAG = {"N": 0, "U": 1}
PATH_AUTO, PATH_SMALL, PATH_BLOCKED, PATH_ROWS64 = 0, 1, 2, 3
INV_AUTO, INV_BLOCKED, INV_FUSED, INV_COLUMN = 0, 1, 2, 3

# Phase codes of the blocked path's timing events (hsma_trsm_opts.events).
PHASE_END, PHASE_SCALE, PHASE_DIAG_INV, PHASE_INV_GEMM, PHASE_COPY, PHASE_TRAILING = -1, 0, 1, 2, 3, 4
PHASE_NAMES = {PHASE_SCALE: "scale", PHASE_DIAG_INV: "diag_inv", PHASE_INV_GEMM: "inv_gemm",
               PHASE_COPY: "copy", PHASE_TRAILING: "trailing_gemm"}


class FloatComplex(ctypes.Structure):
    _fields_ = [("re", ctypes.c_float), ("im", ctypes.c_float)]


class DoubleComplex(ctypes.Structure):
    _fields_ = [("re", ctypes.c_double), ("im", ctypes.c_double)]


class TrsmOpts(ctypes.Structure):
    _fields_ = [("nb", ctypes.c_int32), ("ib", ctypes.c_int32), ("path", ctypes.c_int32),
                ("inv", ctypes.c_int32), ("n_events", ctypes.c_int32), ("events", ctypes.POINTER(ctypes.c_void_p)),
                ("event_phase", ctypes.POINTER(ctypes.c_int32)),
                ("events_used", ctypes.POINTER(ctypes.c_int32))]


class HsmaError(RuntimeError):
    def __init__(self, status, name=""):
        self.status = status
        super().__init__("%s: %s (%d)" % (name, status_string(status), status))


_i64, _i32, _p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
_SCAL = {"s": ctypes.c_float, "d": ctypes.c_double, "c": FloatComplex, "z": DoubleComplex}
_REAL = {"s": ctypes.c_float, "d": ctypes.c_double, "c": ctypes.c_float, "z": ctypes.c_double}

# Prototype of every entry point: name -> (argument types, result type).
_PROTO = {}
for _t in "sdcz":
    S, Rl = _SCAL[_t], _REAL[_t]
    _PROTO["hsma_trsm_" + _t] = ([_i64, _i64, S, _p, _i64, _p, _i64, _p], ctypes.c_int)
    _PROTO["hsma_trsm_strided_batched_" + _t] = (
        [_i64, _i64, S, _p, _i64, _i64, _p, _i64, _i64, _i64, _p], ctypes.c_int)
    _PROTO["hsma_trsm_ex_" + _t] = (
        [_i64, _i64, S, _p, _i64, _p, _i64, ctypes.POINTER(TrsmOpts), _p], ctypes.c_int)
    _PROTO["hsma_diag_inv_" + _t] = ([_i64, _i32, _i32, _p, _i64, _p, _p], ctypes.c_int)
    _PROTO["hsma_diag_inv_ex_" + _t] = ([_i64, ctypes.POINTER(TrsmOpts), _p, _i64, _p, _p], ctypes.c_int)
    _PROTO["hsma_gemm_" + _t] = (
        [_i64, _i64, _i64, Rl, _p, _i64, _p, _i64, Rl, _p, _i64, _i32, _p], ctypes.c_int)
for _t in "sdcz":
    S = _SCAL[_t]
    _PROTO["hsma_trsm_general_" + _t] = (
        [_i32, _i32, _i32, _i32, _i64, _i64, S, _p, _i64, _p, _i64, _p], ctypes.c_int)
    _PROTO["hsma_trsm_strided_batched_general_" + _t] = (
        [_i32, _i32, _i32, _i32, _i64, _i64, S, _p, _i64, _i64, _p, _i64, _i64, _i64, _p], ctypes.c_int)
_PROTO["hsma_solve_tri_f32"] = ([_i64, _i64, _p, _p, _p] + [_i64] * 11 + [_p], ctypes.c_int)
_PROTO["hsma_trsm_block_size"] = ([_i32, _i64, _i64], ctypes.c_int32)
_PROTO["hsma_status_string"] = ([ctypes.c_int], ctypes.c_char_p)
_PROTO["hsma_trsm_noalloc"] = ([_i32, _i64, _i64, _p, _p, _i64, _p, _i64, _p], ctypes.c_int)

EXPORTS = sorted(_PROTO)

_lib = None
_F = {}


def load():
    """The loaded library (loaded on the first call). Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libhsma_trsm.so is not built; run `python -m triangular_solve_amd.build` "
                               "(or __graft_entry__.build()) first")
        # Load torch first when it is installed: its bundled HIP runtime then
        # serves this library too (same soname), so torch's streams and
        # allocations are valid here.
        try:
            import torch  # noqa: F401
        except ImportError:  # pragma: no cover
            pass
        _lib = ctypes.CDLL(LIB_PATH)
    return _lib


def loaded():
    """Whether this process has loaded the library."""
    return _lib is not None


def _fn(name):
    f = _F.get(name)
    if f is None:
        args, res = _PROTO[name]
        f = getattr(load(), name)
        f.argtypes = args
        f.restype = res
        _F[name] = f
    return f


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _scalar(t, v):
    if t in "cz":
        v = complex(v)
        return _SCAL[t](v.real, v.imag)
    return float(v)


def _opts(o):
    if o is None:
        return None
    if isinstance(o, TrsmOpts):
        return ctypes.byref(o)
    return ctypes.byref(TrsmOpts(int(o.get("nb", 0)), int(o.get("ib", 0)), int(o.get("path", 0)),
                                 int(o.get("inv", 0))))


def _mk(t):
    def trsm(m, n, alpha, A, lda, B, ldb, stream=None):
        return _fn("hsma_trsm_" + t)(m, n, _scalar(t, alpha), _ptr(A), lda, _ptr(B), ldb, _stream(stream))

    def strided_batched(m, n, alpha, A, lda, strideA, B, ldb, strideB, batch_count, stream=None):
        return _fn("hsma_trsm_strided_batched_" + t)(m, n, _scalar(t, alpha), _ptr(A), lda, strideA,
                                                     _ptr(B), ldb, strideB, batch_count, _stream(stream))

    def ex(m, n, alpha, A, lda, B, ldb, opts=None, stream=None):
        return _fn("hsma_trsm_ex_" + t)(m, n, _scalar(t, alpha), _ptr(A), lda, _ptr(B), ldb,
                                        _opts(opts), _stream(stream))

    def diag_inv(m, nb, ib, A, lda, invA, stream=None):
        return _fn("hsma_diag_inv_" + t)(m, nb, ib, _ptr(A), lda, _ptr(invA), _stream(stream))

    def gemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, a_lower=0, stream=None):
        return _fn("hsma_gemm_" + t)(M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb, float(beta),
                                     _ptr(C), ldc, int(a_lower), _stream(stream))

    def general(side, uplo, trans, diag, m, n, alpha, A, lda, B, ldb, stream=None):
        return _fn("hsma_trsm_general_" + t)(side, uplo, trans, diag, m, n, _scalar(t, alpha), _ptr(A),
                                             lda, _ptr(B), ldb, _stream(stream))

    def strided_batched_general(side, uplo, trans, diag, m, n, alpha, A, lda, strideA, B, ldb,
                                strideB, batch_count, stream=None):
        return _fn("hsma_trsm_strided_batched_general_" + t)(
            side, uplo, trans, diag, m, n, _scalar(t, alpha), _ptr(A), lda, strideA, _ptr(B), ldb,
            strideB, batch_count, _stream(stream))

    def diag_inv_ex(m, opts, A, lda, invA, stream=None):
        return _fn("hsma_diag_inv_ex_" + t)(m, _opts(opts), _ptr(A), lda, _ptr(invA), _stream(stream))

    globals()["hsma_diag_inv_ex_" + t] = diag_inv_ex
    globals()["hsma_trsm_general_" + t] = general
    globals()["hsma_trsm_strided_batched_general_" + t] = strided_batched_general
    return trsm, strided_batched, ex, diag_inv, gemm


(hsma_trsm_s, hsma_trsm_strided_batched_s, hsma_trsm_ex_s, hsma_diag_inv_s, hsma_gemm_s) = _mk("s")
(hsma_trsm_d, hsma_trsm_strided_batched_d, hsma_trsm_ex_d, hsma_diag_inv_d, hsma_gemm_d) = _mk("d")
(hsma_trsm_c, hsma_trsm_strided_batched_c, hsma_trsm_ex_c, hsma_diag_inv_c, hsma_gemm_c) = _mk("c")
(hsma_trsm_z, hsma_trsm_strided_batched_z, hsma_trsm_ex_z, hsma_diag_inv_z, hsma_gemm_z) = _mk("z")


def hsma_solve_tri_f32(n, k, A, B, X, ne02, ne03, sA1, sA2, sA3, sB1, sB2, sB3, sX1, sX2, sX3,
                       stream=None):
    return _fn("hsma_solve_tri_f32")(n, k, _ptr(A), _ptr(B), _ptr(X), ne02, ne03, sA1, sA2, sA3,
                                     sB1, sB2, sB3, sX1, sX2, sX3, _stream(stream))


_CTYPE_OF_CODE = {DTYPE_F32: ctypes.c_float, DTYPE_F64: ctypes.c_double, DTYPE_C64: FloatComplex,
                  DTYPE_C128: DoubleComplex}


def hsma_trsm_noalloc(dtype, m, n, alpha, A, lda, B, ldb, stream=None):
    """dtype is a DTYPE_* code; alpha a Python number (passed by address)."""
    ct = _CTYPE_OF_CODE.get(dtype)
    if ct is None:
        a = ctypes.c_double(0.0)
    elif dtype in (DTYPE_C64, DTYPE_C128):
        v = complex(alpha)
        a = ct(v.real, v.imag)
    else:
        a = ct(float(alpha))
    return _fn("hsma_trsm_noalloc")(dtype, m, n, ctypes.byref(a), _ptr(A), lda, _ptr(B), ldb,
                                    _stream(stream))


def hsma_trsm_block_size(dtype, m, n=None):
    return _fn("hsma_trsm_block_size")(dtype, m, m if n is None else n)


def hsma_status_string(status):
    return _fn("hsma_status_string")(status).decode()


status_string = hsma_status_string

# letter of the BLAS-style entry points per element type name
LETTER = {"f32": "s", "f64": "d", "c64": "c", "c128": "z"}
DTYPE_CODE = {"f32": DTYPE_F32, "f64": DTYPE_F64, "c64": DTYPE_C64, "c128": DTYPE_C128}


def entry(kind, dtype):
    """The binding function of one entry point, e.g. entry("trsm", "c64") -> hsma_trsm_c."""
    names = {"trsm": "hsma_trsm_%s", "strided_batched": "hsma_trsm_strided_batched_%s",
             "ex": "hsma_trsm_ex_%s", "diag_inv": "hsma_diag_inv_%s", "gemm": "hsma_gemm_%s",
             "general": "hsma_trsm_general_%s", "diag_inv_ex": "hsma_diag_inv_ex_%s",
             "strided_batched_general": "hsma_trsm_strided_batched_general_%s"}
    return globals()[names[kind] % LETTER[dtype]]


def check(status, name="hsma"):
    if status != SUCCESS:
        raise HsmaError(status, name)
