"""GPU edge cases through the C ABI: zero pivots (no singularity check, IEEE
non-finite values in the same places as the oracle on every path), alpha and
pivots at the ends of the exponent range, and the blocked path's phase events."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from _gpu_util import TOL_LARGE, TOL_SMALL, colmajor_inputs, rel_err, say, to_dev, views

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f64", "c64", "c128"]


@pytest.fixture(scope="module")
def hs():
    import torch  # noqa: F401
    import triangular_solve_amd as hs
    return hs


def solve_colmajor(hs, dt, A, B, m, n, batch, route, alpha=1.0):
    """Column-major solve through one route; returns X as [batch, m, n]."""
    import torch
    dA, dB = to_dev(A), to_dev(B)
    lda, ldb = A.shape[2], B.shape[2]
    if route == "batched":
        st = hs.entry("strided_batched", dt)(m, n, alpha, dA, lda, A.shape[1] * lda if A.shape[0] > 1 else 0,
                                             dB, ldb, n * ldb, batch)
    elif route.startswith("blocked"):
        nb = int(route.split(":")[1])
        assert batch == 1
        st = hs.entry("ex", dt)(m, n, alpha, dA, lda, dB, ldb, {"nb": nb, "path": hs.PATH_BLOCKED})
    else:
        raise ValueError(route)
    torch.cuda.synchronize()
    assert st == hs.SUCCESS, (route, st)
    return dB.cpu().numpy()[:, :, :m].transpose(0, 2, 1)


def check_pattern(Xg, Xo, tol, what):
    fin_g, fin_o = np.isfinite(Xg), np.isfinite(Xo)
    assert np.array_equal(fin_g, fin_o), "%s: non-finite pattern differs (%d vs %d)" % (
        what, (~fin_g).sum(), (~fin_o).sum())
    assert (~fin_o).any(), what
    if fin_o.any():
        d = np.abs(np.where(fin_o, Xg.astype(Xo.dtype) - Xo, 0))
        ref = np.sqrt(np.sum(np.abs(np.where(fin_o, Xo, 0)) ** 2))
        assert np.sqrt(np.sum(d ** 2)) <= tol * max(ref, 1e-300), what


ZERO_CASES = [  # (m, n, batch, route, zero pivot row)
    (64, 64, 4, "batched", 0), (64, 64, 4, "batched", 37), (64, 64, 4, "batched", 63),
    (64, 6, 4, "batched", 20), (37, 64, 2, "batched", 30),
    (150, 64, 3, "batched", 100),                 # block rows of 64 over the batch
    (400, 30, 2, "batched", 350),                 # the same up to m = 512
    (150, 8, 1, "batched", 120),                  # one problem with few columns: block rows
    (300, 40, 1, "blocked:128", 5), (300, 40, 1, "blocked:128", 200),   # column route
    (512, 40, 1, "blocked:256", 70), (512, 40, 1, "blocked:256", 300),  # blocked-inverse route
]


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("m,n,batch,route,k", ZERO_CASES)
def test_zero_pivot_matches_oracle(hs, dt, m, n, batch, route, k):
    say("zero pivot", dt, m, n, batch, route, k)
    A, B = colmajor_inputs(dt, m, n, batch, seed=900 + k)
    A[:, k, k] = 0   # column k, row k
    Xg = solve_colmajor(hs, dt, A, B, m, n, batch, route)
    Av, Bv = views(A, B, m)
    Xo = oracle.trsm(Av, Bv)
    tol = (TOL_SMALL if m <= 64 else TOL_LARGE)[dt]
    check_pattern(Xg, Xo, tol, "%s %s k=%d" % (dt, route, k))
    # rows above the pivot are finite and rows from it on are not, as the
    # definition says
    assert np.isfinite(Xo[:, :k, :]).all() and not np.isfinite(Xo[:, k:, :]).any()


@pytest.mark.parametrize("n,k", [(64, 10), (16, 10), (200, 100), (128, 127), (100, 3), (256, 230),
                                 (150, 140), (193, 64)])
def test_zero_pivot_solve_tri(hs, n, k):
    import torch
    say("zero pivot solve_tri", n, k)
    kk, e2, e3 = 6, 2, 2
    A = synth.tri("f32", n, e2 * e3, seed=77, offdiag_div=n, layout="row")
    B = synth.rhs("f32", n, kk, e2 * e3, seed=78, layout="row")
    A[:, k, k] = 0
    dA, dB = to_dev(A), to_dev(B)
    dX = torch.empty_like(dB)
    st = hs.hsma_solve_tri_f32(n, kk, dA, dB, dX, e2, e3, n, n * n, e2 * n * n, kk, n * kk,
                               e2 * n * kk, kk, n * kk, e2 * n * kk)
    torch.cuda.synchronize()
    assert st == hs.SUCCESS
    check_pattern(dX.cpu().numpy(), oracle.trsm(A, B), 1e-5, "solve_tri n=%d" % n)


def test_f64_zero_and_subnormal_pivots_agree_across_kernels(hs):
    """Lane-per-column (n = 64) and lane-per-row (n = 6) kernels give the same
    non-finite pattern for a zero pivot, and accurate results for a subnormal
    pivot whose reciprocal is finite."""
    m = 64
    for piv, k in [(0.0, 12), (-0.0, 40), (1e-308, 25), (-3e-309, 50)]:
        A, B = colmajor_inputs("f64", m, 64, 2, seed=31)
        A[:, k, k] = piv
        Xw = solve_colmajor(hs, "f64", A, B, m, 64, 2, "batched")
        Xn = solve_colmajor(hs, "f64", A, B[:, :6].copy(), m, 6, 2, "batched")
        assert np.array_equal(np.isfinite(Xw[:, :, :6]), np.isfinite(Xn)), piv
        Av, Bv = views(A, B, m)
        Xo = oracle.trsm(Av, Bv)
        if piv == 0:
            check_pattern(Xw, Xo, 1e-12, "f64 zero pivot n=64")
            check_pattern(Xn, Xo[:, :, :6], 1e-12, "f64 zero pivot n=6")
        else:
            fin = np.isfinite(Xo)
            assert fin.all() == np.isfinite(Xw).all()
            if fin.all():
                assert rel_err(Xw, Xo) <= 1e-12 and rel_err(Xn, Xo[:, :, :6]) <= 1e-12, piv


@pytest.mark.parametrize("alpha", [1e-200, 1e200 * (0.6 + 0.8j), -3.5 + 2j])
def test_c128_alpha_extremes(hs, alpha):
    """alpha at the ends of the double range through the two-panel c128
    kernel (m = n = 64) and the lane-per-row kernel (n = 6)."""
    for n in (64, 6):
        A, B = colmajor_inputs("c128", 64, n, 3, seed=44)
        Xg = solve_colmajor(hs, "c128", A, B, 64, n, 3, "batched", alpha=alpha)
        Av, Bv = views(A, B, 64)
        Xo = oracle.trsm(Av, Bv, alpha=alpha)
        assert np.isfinite(Xg).all()
        # compared in units of alpha (the squares in the norms would overflow)
        sc = 1.0 / abs(alpha)
        assert rel_err(Xg * sc, Xo * sc) <= 1e-12, (alpha, n)


@pytest.mark.parametrize("dt,e", [("c64", 83), ("c64", -83), ("c128", 530), ("c128", -530)])
@pytest.mark.parametrize("m,n,route", [(64, 64, "batched"), (64, 6, "batched"), (40, 64, "batched"),
                                       (300, 40, "blocked:128"), (512, 40, "blocked:256")])
def test_complex_pivots_over_the_exponent_range(hs, dt, e, m, n, route):
    """A scaled by 2^e, beyond where |a_jj|^2 is representable: the solution
    scales by exactly 2^-e (power-of-two scaling changes no rounding), and the
    unscaled solve matches the oracle."""
    say("complex range", dt, e, m, n, route)
    A, B = colmajor_inputs(dt, m, n, 1, seed=55)
    X1 = solve_colmajor(hs, dt, A, B, m, n, 1, route)
    As = (A * np.float64(2.0) ** e).astype(A.dtype)
    Xs = solve_colmajor(hs, dt, As, B, m, n, 1, route)
    assert np.isfinite(Xs).all()
    assert np.array_equal(Xs, (X1 * np.float64(2.0) ** -e).astype(X1.dtype)), (dt, e, route)
    Av, Bv = views(A, B, m)
    assert rel_err(X1, oracle.trsm(Av, Bv)) <= (TOL_SMALL if m <= 64 else TOL_LARGE)[dt]


@pytest.mark.parametrize("dt", ["f32", "c128"])
@pytest.mark.parametrize("m,nb,alpha", [(1000, 128, 1.0), (1024, 256, 2.0), (512, 512, 1.0)])
def test_phase_events(hs, dt, m, nb, alpha):
    """The blocked path records one event per phase in launch order, and a
    timed solve gives the same bits as an untimed one."""
    import torch
    say("phase events", dt, m, nb, alpha)
    n = 96
    A, B = colmajor_inputs(dt, m, n, 1, seed=66)
    dA, dB1, dB2 = to_dev(A), to_dev(B), to_dev(B)
    f = hs.entry("ex", dt)
    hs.check(f(m, n, alpha, dA, m, dB1, m, {"nb": nb, "path": hs.PATH_BLOCKED}), "untimed")
    nt = (m + nb - 1) // nb
    need = 3 * nt + 1 + (0 if alpha == 1.0 else 1)
    cap = need + 3
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(cap)]
    for ev in evs:
        ev.record(stream)
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * cap)(*[ev.cuda_event for ev in evs])
    phases = (ctypes.c_int32 * cap)()
    used = ctypes.c_int32(0)
    o = hs.TrsmOpts(nb, 0, hs.PATH_BLOCKED, 0, cap, handles, phases, ctypes.pointer(used))
    hs.check(f(m, n, alpha, dA, m, dB2, m, o, stream), "timed")
    torch.cuda.synchronize()
    assert used.value == need
    seq = list(phases[:used.value])
    want = ([hs.PHASE_SCALE] if alpha != 1.0 else []) + [hs.PHASE_DIAG_INV]
    for t in range(nt):
        want += [hs.PHASE_INV_GEMM, hs.PHASE_COPY] + ([hs.PHASE_TRAILING] if t + 1 < nt else [])
    want += [hs.PHASE_END]
    assert seq == want
    ms = [evs[k].elapsed_time(evs[k + 1]) for k in range(used.value - 1)]
    assert all(x >= 0 for x in ms)
    assert torch.equal(dB1, dB2)


@pytest.mark.parametrize("dt", ["f32", "c64"])
def test_copy_on_second_stream_same_bits(hs, dt):
    """Block rows of N_B x n >= 2^22 elements copy W into B on a second
    stream beside the trailing product; a phase-timed solve keeps every copy
    on the caller's stream. Both give the same bits, on every repeat, and
    match the oracle on sampled columns."""
    import torch
    m, n, nb = 4096, 2048, 2048          # two block rows of 2048 x 2048 = 2^22
    say("copy overlap", dt, m, n, nb)
    A, B = colmajor_inputs(dt, m, n, 1, seed=71)
    dA = to_dev(A)
    f = hs.entry("ex", dt)
    outs = []
    for _ in range(3):
        dB = to_dev(B)
        hs.check(f(m, n, 1.0, dA, m, dB, m, {"nb": nb, "path": hs.PATH_BLOCKED}), "overlapped")
        outs.append(dB)
    cap = 3 * 2 + 1
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(cap)]
    for ev in evs:
        ev.record(stream)
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * cap)(*[ev.cuda_event for ev in evs])
    phases = (ctypes.c_int32 * cap)()
    used = ctypes.c_int32(0)
    o = hs.TrsmOpts(nb, 0, hs.PATH_BLOCKED, 0, cap, handles, phases, ctypes.pointer(used))
    dBt = to_dev(B)
    hs.check(f(m, n, 1.0, dA, m, dBt, m, o, stream), "timed")
    torch.cuda.synchronize()
    assert used.value == cap
    for dB in outs:
        assert torch.equal(dB, dBt)
    cols = np.array([0, 1, 777, 2047])
    X = dBt.cpu().numpy()[0][cols, :m].T
    Av, Bv = views(A, B, m)
    Xo = oracle.trsm(np.ascontiguousarray(Av), np.ascontiguousarray(Bv[:, :, cols]))
    assert rel_err(X[None], Xo) <= TOL_LARGE[dt]
