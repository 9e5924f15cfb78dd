"""GPU parity of the small regime (m <= 64) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
import synth
from _gpu_util import (EPS, TOL_SMALL, colmajor_inputs, rel_err, say, scaled_residual, to_dev,
                       views)

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f64", "c64", "c128"]


@pytest.fixture(scope="module")
def hs():
    import torch  # noqa: F401
    import triangular_solve_amd as hs
    return hs


def solve_batched(hs, dtype, A, B, m, n, lda, ldb, alpha=1.0, shared_a=False):
    import torch
    dA, dB = to_dev(A), to_dev(B)
    batch = B.shape[0]
    strideA = 0 if shared_a else A.shape[1] * A.shape[2]
    st = hs.entry("strided_batched", dtype)(m, n, alpha, dA, lda, strideA, dB, ldb,
                                            B.shape[1] * B.shape[2], batch)
    torch.cuda.synchronize()
    assert st == hs.SUCCESS, hs.status_string(st)
    return dB.cpu().numpy()


def check(dtype, A, B, X, m, alpha, shared_a=False, tol=None):
    Av, Bv = views(A, B, m)
    if shared_a:
        Av = np.broadcast_to(Av, (B.shape[0],) + Av.shape[1:])
    Xo = oracle.trsm(Av, Bv, alpha)
    Xg = X[:, :, :m].transpose(0, 2, 1)
    err = rel_err(Xg, Xo)
    res = scaled_residual(np.ascontiguousarray(Av), Xg, Bv, alpha)
    assert err <= (tol or TOL_SMALL[dtype]), err
    assert res <= 10 * m * EPS[dtype], res
    # rows of B below m (the leading-dimension padding) are never written
    assert np.array_equal(X[:, :, m:], B[:, :, m:])
    return err


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("m", [1, 2, 3, 7, 31, 32, 33, 63, 64])
@pytest.mark.parametrize("n", [1, 6, 33, 64, 200])
def test_shapes(hs, dtype, m, n):
    say("small", dtype, m, n)
    A, B = colmajor_inputs(dtype, m, n, 3, seed=m * 1000 + n)
    X = solve_batched(hs, dtype, A, B, m, n, m, m)
    check(dtype, A, B, X, m, 1.0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_padded_leading_dims_alpha_and_shared_a(hs, dtype):
    cplx = dtype.startswith("c")
    # odd ldb: B's columns are not 16-byte aligned (lane-per-row kernel for
    # the real and c64 types); ldb 68 / 72: aligned padding, lane-per-column
    # kernel with its LDS tile (n = 100: a partial second group of columns)
    for (m, n, lda, ldb) in [(64, 64, 70, 67), (64, 40, 64, 65), (20, 9, 33, 21),
                             (64, 64, 70, 68), (64, 100, 66, 72)]:
        for alpha in [2.0, -0.5] + ([0.3 + 0.7j] if cplx else []):
            say("padded", dtype, m, n, lda, ldb, alpha)
            A, B = colmajor_inputs(dtype, m, n, 4, lda=lda, ldb=ldb, seed=7)
            X = solve_batched(hs, dtype, A, B, m, n, lda, ldb, alpha)
            check(dtype, A, B, X, m, alpha)
    say("shared A", dtype)
    A, B = colmajor_inputs(dtype, 64, 64, 5, seed=8, shared_a=True)
    X = solve_batched(hs, dtype, A, B, 64, 64, 64, 64, 1.0, shared_a=True)
    check(dtype, A, B, X, 64, 1.0, shared_a=True)


@pytest.mark.parametrize("dtype", DTYPES)
def test_alpha_zero_sets_zero_without_reading_a(hs, dtype):
    import torch
    say("alpha0", dtype)
    A, B = colmajor_inputs(dtype, 64, 64, 2, seed=9)
    dB = to_dev(B)
    # A is NULL: with alpha == 0 it must not be read
    st = hs.entry("strided_batched", dtype)(64, 64, 0.0, None, 64, 4096, dB, 64, 4096, 2)
    torch.cuda.synchronize()
    assert st == hs.SUCCESS
    assert not dB.cpu().numpy().any()


@pytest.mark.parametrize("dtype", DTYPES)
def test_single_problem_entry(hs, dtype):
    import torch
    for (m, n) in [(64, 64), (64, 6), (50, 64)]:
        say("single", dtype, m, n)
        A, B = colmajor_inputs(dtype, m, n, 1, seed=11)
        dA, dB = to_dev(A), to_dev(B)
        st = hs.entry("trsm", dtype)(m, n, 1.0, dA, m, dB, m)
        torch.cuda.synchronize()
        assert st == hs.SUCCESS
        check(dtype, A, B, dB.cpu().numpy(), m, 1.0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_throughput_batch_4096(hs, dtype):
    """The batched workload: 4096 problems of 64 x 64 with 64 right-hand sides."""
    say("batch4096", dtype)
    A, B = colmajor_inputs(dtype, 64, 64, 4096, seed=0x5EED0001, offdiag_div=64)
    X = solve_batched(hs, dtype, A, B, 64, 64, 64, 64)
    err = check(dtype, A, B, X, 64, 1.0)
    say("  rel err", err)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", [64, 96])
def test_launch_size_forms_bitwise_equal(hs, dtype, n):
    """f64 and c64 solve the problems of a launch with many problems per CU in four row panels
    and those of a smaller launch in one pass; every element takes its updates in the same
    order either way, so the same problems must give the same bits in both (the other dtypes
    have one form and must agree as well). n = 96: a second, ragged group of columns."""
    say("launch forms", dtype, n)
    A, B = colmajor_inputs(dtype, 64, n, 4096, seed=0x5EED0007, offdiag_div=64)
    Xbig = solve_batched(hs, dtype, A, B, 64, n, 64, 64)
    Xsmall = solve_batched(hs, dtype, np.ascontiguousarray(A[:256]), np.ascontiguousarray(B[:256]),
                           64, n, 64, 64)
    assert np.array_equal(Xbig[:256].view(np.uint8), Xsmall.view(np.uint8))
    sel = np.arange(0, 4096, 16)
    err = check(dtype, np.ascontiguousarray(A[sel]), np.ascontiguousarray(B[sel]),
                np.ascontiguousarray(Xbig[sel]), 64, 1.0)
    say("  rel err", err)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("m,n", [(64, 64), (40, 5)])
def test_exact_integer_cases_bitwise(hs, dtype, m, n):
    """Bidiagonal (1, -1) gives running sums, all-ones lower gives differences:
    every intermediate is a small integer, so the result must be exact."""
    import torch
    npdt = synth.NP_DTYPE[dtype]
    rng = np.random.default_rng(m + n)
    for kind in ("bidiag", "ones"):
        say("exact", dtype, m, n, kind)
        L = np.full((m, m), np.nan, dtype=npdt)
        L[np.tril_indices(m, -1)] = 0
        L[np.diag_indices(m)] = 1
        if kind == "bidiag":
            L[np.arange(1, m), np.arange(m - 1)] = -1
        else:
            L[np.tril_indices(m, -1)] = 1
        Bm = rng.integers(-20, 20, size=(m, n)).astype(npdt)
        if dtype.startswith("c"):
            Bm = Bm + 1j * rng.integers(-20, 20, size=(m, n)).astype(npdt)
        A = np.ascontiguousarray(L.T)[None]           # column-major storage
        B = np.ascontiguousarray(Bm.T)[None]
        dA, dB = to_dev(A), to_dev(B)
        st = hs.entry("trsm", dtype)(m, n, 1.0, dA, m, dB, m)
        torch.cuda.synchronize()
        assert st == hs.SUCCESS
        Xg = dB.cpu().numpy()[0].T
        expect = np.cumsum(Bm, axis=0) if kind == "bidiag" else np.concatenate([Bm[:1], np.diff(Bm, axis=0)])
        assert np.array_equal(Xg, expect.astype(npdt))


def ggml_case(hs, n, k, ne02, ne03, seed):
    import torch
    nb = ne02 * ne03
    A = synth.tri("f32", n, nb, seed=seed, offdiag_div=64, layout="row")    # (nb, n, n) row-major
    B = synth.rhs("f32", n, k, nb, seed=seed + 1, layout="row")              # (nb, n, k) row-major
    dA, dB = to_dev(A), to_dev(B)
    dX = torch.full((nb, n, k), float("nan"), dtype=torch.float32, device="cuda")
    st = hs.hsma_solve_tri_f32(n, k, dA, dB, dX, ne02, ne03, n, n * n, ne02 * n * n,
                               k, n * k, ne02 * n * k, k, n * k, ne02 * n * k)
    torch.cuda.synchronize()
    assert st == hs.SUCCESS
    X = dX.cpu().numpy()
    Xo = oracle.trsm(A, B)
    assert np.array_equal(dB.cpu().numpy(), B)   # B is read-only
    return X, Xo, A, B


def test_solve_tri_ggml_shapes(hs):
    # [64,64,4,2]/[6,64,4,2]: the PR's perf shape; [64,64,2,2]/[10,64,2,2]: its race case
    for (n, k, e2, e3) in [(64, 6, 4, 2), (64, 10, 2, 2), (17, 3, 3, 1), (64, 64, 2, 1), (5, 130, 1, 2)]:
        say("solve_tri", n, k, e2, e3)
        X, Xo, A, B = ggml_case(hs, n, k, e2, e3, seed=n + k)
        assert rel_err(X, Xo) <= TOL_SMALL["f32"]
        nmse = float(np.sum((X - Xo) ** 2) / np.sum(Xo ** 2))
        assert nmse <= 1e-7    # the test-backend-ops gate on the SOLVE_TRI page


def test_solve_tri_medium_sizes(hs):
    """64 < n <= 256: block rows of 64 (the PR's [128,128,4,1] / [8,128,4,1]
    case included), ragged last blocks, k above and below the 8-column
    update groups."""
    # n <= 128: one launch, 2 / 4 / 8 columns per workgroup for k <= 8 / <= 32 / more;
    # n > 128: block rows of 64
    for (n, k, e2, e3) in [(128, 8, 4, 1), (100, 5, 2, 3), (65, 1, 1, 1), (96, 20, 2, 1),
                           (128, 70, 1, 2), (256, 6, 1, 2), (200, 130, 1, 1), (192, 64, 2, 1)]:
        say("solve_tri medium", n, k, e2, e3)
        X, Xo, A, B = ggml_case(hs, n, k, e2, e3, seed=n + 3 * k)
        assert rel_err(X, Xo) <= TOL_SMALL["f32"]
        nmse = float(np.sum((X - Xo) ** 2) / np.sum(Xo ** 2))
        assert nmse <= 1e-7


# n = 48: rows staged through LDS; n = 64 with 16-byte aligned row strides:
# rows of A kept in registers; n = 64 with odd strides: back to LDS staging
@pytest.mark.parametrize("n,sA1,pa2,pa3", [(48, 50, 5, 7), (64, 68, 4, 8), (64, 65, 5, 7),
                                           (150, 152, 4, 8), (130, 131, 5, 7), (100, 103, 5, 7)])
def test_solve_tri_strided_views(hs, n, sA1, pa2, pa3):
    """Non-contiguous batches: A, B, X inside larger buffers with padded strides."""
    import torch
    k, e2, e3 = 7, 3, 2
    sB1, sX1 = 9, 11
    sA2, sB2, sX2 = n * sA1 + pa2, n * sB1 + 3, n * sX1 + 2
    sA3, sB3, sX3 = e2 * sA2 + pa3, e2 * sB2 + 1, e2 * sX2 + 4
    rng = np.random.default_rng(3)
    Abuf = rng.standard_normal(e3 * sA3).astype(np.float32)
    Bbuf = rng.standard_normal(e3 * sB3).astype(np.float32)
    L = synth.tri("f32", n, e2 * e3, seed=5, layout="row")
    Bl = synth.rhs("f32", n, k, e2 * e3, seed=6, layout="row")
    for i3 in range(e3):
        for i2 in range(e2):
            b = i3 * e2 + i2
            for i in range(n):
                Abuf[i2 * sA2 + i3 * sA3 + i * sA1: i2 * sA2 + i3 * sA3 + i * sA1 + n] = L[b, i]
                Bbuf[i2 * sB2 + i3 * sB3 + i * sB1: i2 * sB2 + i3 * sB3 + i * sB1 + k] = Bl[b, i]
    dA, dB = to_dev(Abuf), to_dev(Bbuf)
    dX = torch.full((e3 * sX3,), 7.0, dtype=torch.float32, device="cuda")
    st = hs.hsma_solve_tri_f32(n, k, dA, dB, dX, e2, e3, sA1, sA2, sA3, sB1, sB2, sB3, sX1, sX2, sX3)
    torch.cuda.synchronize()
    assert st == hs.SUCCESS
    Xbuf = dX.cpu().numpy()
    Xo = oracle.trsm(L, Bl)
    written = np.zeros(e3 * sX3, dtype=bool)
    for i3 in range(e3):
        for i2 in range(e2):
            b = i3 * e2 + i2
            for i in range(n):
                o = i2 * sX2 + i3 * sX3 + i * sX1
                np.testing.assert_allclose(Xbuf[o:o + k], Xo[b, i], rtol=1e-5, atol=1e-6)
                written[o:o + k] = True
    assert np.all(Xbuf[~written] == 7.0)   # nothing outside X's elements is touched


@pytest.mark.parametrize("dtype", DTYPES)
def test_repeat_runs_bitwise_identical(hs, dtype):
    """Race detector: the kernels are deterministic, so any run-to-run
    difference is a race. 1000 runs of each path (small regime in both
    kernels, the 64 < m <= 256 band, the blocked path with split products),
    each compared with the first bit for bit on the device. The batch of 4096 runs the row-panel
    form of f64 and c64."""
    import torch
    cases = [(64, 64, 16, None), (64, 64, 4096, None), (64, 10, 16, None), (37, 6, 16, None),
             (150, 64, 8, None), (300, 40, 1, 128), (1024, 16, 1, 256)]
    for (m, n, batch, nb) in cases:
        say("repeat x1000", dtype, m, n, batch, nb)
        A, B = colmajor_inputs(dtype, m, n, batch, seed=21)
        dA, dB0 = to_dev(A), to_dev(B)
        dB = torch.empty_like(dB0)
        ref = None
        for it in range(1000):
            dB.copy_(dB0)
            if nb is None:
                st = hs.entry("strided_batched", dtype)(m, n, 1.0, dA, m, m * m, dB, m, m * n, batch)
            else:
                st = hs.entry("ex", dtype)(m, n, 1.0, dA, m, dB, m, {"nb": nb, "path": hs.PATH_BLOCKED})
            assert st == hs.SUCCESS
            if ref is None:
                ref = dB.clone()
            else:   # raw bits, so NaN compares too
                assert torch.equal(dB.view(torch.uint8), ref.view(torch.uint8)), (m, n, it)
        torch.cuda.synchronize()


def test_repeat_solve_tri_bitwise_identical(hs):
    """The SOLVE_TRI kernels (one wave per group of right-hand sides, the
    two-wave 128-row kernel and the four-wave 256-row kernel), 1000 runs
    each, bit for bit."""
    import torch
    for n, k, e2, e3 in [(64, 6, 4, 2), (64, 10, 2, 2), (128, 8, 4, 1), (256, 8, 4, 1), (200, 40, 2, 1)]:
        A = synth.tri("f32", n, e2 * e3, seed=5, offdiag_div=n, layout="row")
        B = synth.rhs("f32", n, k, e2 * e3, seed=6, layout="row")
        dA, dB = to_dev(A), to_dev(B)
        dX = torch.empty_like(dB)
        args = (n, k, dA, dB, dX, e2, e3, n, n * n, e2 * n * n, k, n * k, e2 * n * k, k, n * k, e2 * n * k)
        assert hs.hsma_solve_tri_f32(*args) == hs.SUCCESS
        ref = dX.clone()
        for it in range(1000):
            dX.fill_(7.0)
            assert hs.hsma_solve_tri_f32(*args) == hs.SUCCESS
            assert torch.equal(dX.view(torch.uint8), ref.view(torch.uint8)), (n, k, it)
        torch.cuda.synchronize()
