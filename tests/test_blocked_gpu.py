"""GPU parity of the blocked regime against the CPU oracle, through the C ABI:
the matrix-core GEMM, the diagonal-block inversion, and the whole blocked solve."""
import numpy as np
import pytest

import oracle
import synth
from _gpu_util import (EPS, TOL_LARGE, colmajor_inputs, rel_err, say, scaled_residual, to_dev,
                       views)

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f64", "c64", "c128"]


@pytest.fixture(scope="module")
def hs():
    import torch  # noqa: F401
    import triangular_solve_amd as hs
    return hs


def rand(dtype, shape, rng):
    a = rng.uniform(-1, 1, shape)
    if dtype.startswith("c"):
        a = a + 1j * rng.uniform(-1, 1, shape)
    return a.astype(synth.NP_DTYPE[dtype])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N,K,lower", [(128, 128, 16, 0), (130, 70, 45, 0), (1, 1, 1, 0),
                                         (300, 257, 513, 0), (200, 33, 200, 1), (64, 64, 64, 1),
                                         (517, 129, 517, 1), (31, 200, 0, 0)])
def test_gemm(hs, dtype, M, N, K, lower):
    import torch
    rng = np.random.default_rng(M * 7 + N + K)
    lda, ldb, ldc = M + 3, K + 1, M + 2
    A = rand(dtype, (K, lda), rng)          # column-major: [k, :M] is column k
    if lower:
        Af = A[:, :M].T.copy()
        Af[np.triu_indices(M, 1)] = np.nan  # must never be read
        A[:, :M] = Af.T
    B = rand(dtype, (N, ldb), rng)
    C = rand(dtype, (N, ldc), rng)
    for alpha, beta in [(1.0, 0.0), (-1.0, 1.0)]:
        say("gemm", dtype, M, N, K, lower, alpha, beta)
        dA, dB, dC = to_dev(A), to_dev(B), to_dev(C)
        st = hs.entry("gemm", dtype)(M, N, K, alpha, dA, lda, dB, ldb, beta, dC, ldc, lower)
        torch.cuda.synchronize()
        assert st == hs.SUCCESS
        Cg = dC.cpu().numpy()
        Am = A[:, :M].T
        if lower:
            Am = np.tril(np.nan_to_num(Am))
        ref = alpha * oracle.gemm(np.ascontiguousarray(Am), np.ascontiguousarray(B[:, :K].T))
        if beta:
            ref = ref + C[:, :M].T
        got = Cg[:, :M].T
        scale = np.linalg.norm(ref) if ref.size else 1.0
        tol = 1e-5 if dtype in ("f32", "c64") else 1e-13
        assert np.linalg.norm(got - ref) <= tol * max(scale, 1e-30) * max(1, np.sqrt(K) / 8)
        assert np.array_equal(Cg[:, M:], C[:, M:])   # ldc padding untouched


@pytest.mark.parametrize("dtype", DTYPES)
def test_gemm_integer_exact(hs, dtype):
    import torch
    rng = np.random.default_rng(5)
    M, N, K = 256, 192, 160
    A = rng.integers(-4, 4, (K, M)).astype(synth.NP_DTYPE[dtype])
    B = rng.integers(-4, 4, (N, K)).astype(synth.NP_DTYPE[dtype])
    if dtype.startswith("c"):
        A = A + 1j * rng.integers(-4, 4, A.shape)
        B = B + 1j * rng.integers(-4, 4, B.shape)
        A, B = A.astype(synth.NP_DTYPE[dtype]), B.astype(synth.NP_DTYPE[dtype])
    C = np.zeros((N, M), dtype=synth.NP_DTYPE[dtype])
    dA, dB, dC = to_dev(A), to_dev(B), to_dev(C)
    assert hs.entry("gemm", dtype)(M, N, K, 1.0, dA, M, dB, K, 0.0, dC, M, 0) == hs.SUCCESS
    torch.cuda.synchronize()
    ref = oracle.gemm(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T))
    assert np.array_equal(dC.cpu().numpy().T.astype(ref.dtype), ref)


@pytest.mark.parametrize("dtype,real", [("c64", "f32"), ("c128", "f64")])
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 1024), (300, 130, 70), (1024, 256, 512)])
def test_complex_gemm_equals_its_real_form_bitwise(hs, dtype, real, M, N, K):
    """The blocked solve runs large complex trailing products as real ones on A's panel expanded
    to 2 x 2 real blocks [[re, -im], [im, re]]. The complex GEMM builds the same blocks on its way
    into LDS and takes each output's products in the same order, so C -= A B must give the same
    bits both ways (the real form may run another tile: the order within a wave is the same)."""
    import torch
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    A = rand(dtype, (K, M), rng)             # column-major: [k, :] is column k
    B = rand(dtype, (N, K), rng)
    C = rand(dtype, (N, M), rng)
    rdt = synth.NP_DTYPE[real]
    Ar = A.view(rdt)                          # (K, 2M): column k as (re, im) pairs
    E = np.empty((2 * K, 2 * M), dtype=rdt)   # the real form, column-major 2M x 2K
    E[0::2] = Ar
    E[1::2, 0::2] = -Ar[:, 1::2]
    E[1::2, 1::2] = Ar[:, 0::2]
    say("complex vs real form", dtype, M, N, K)
    dA, dB, dC1 = to_dev(A), to_dev(B), to_dev(C)
    dE, dC2 = to_dev(E), to_dev(C)
    assert hs.entry("gemm", dtype)(M, N, K, -1.0, dA, M, dB, K, 1.0, dC1, M, 0) == hs.SUCCESS
    assert hs.entry("gemm", real)(2 * M, N, 2 * K, -1.0, dE, 2 * M, dB.view(torch.float32 if real == "f32" else torch.float64),
                                  2 * K, 1.0, dC2.view(torch.float32 if real == "f32" else torch.float64), 2 * M, 0) == hs.SUCCESS
    torch.cuda.synchronize()
    assert torch.equal(dC1.view(torch.uint8), dC2.view(torch.uint8))


@pytest.mark.parametrize("dtype,real", [("c64", "f32"), ("c128", "f64")])
@pytest.mark.parametrize("M,N", [(1024, 4096), (300, 130), (2048, 512)])
def test_complex_lower_gemm_equals_its_real_form_bitwise(hs, dtype, real, M, N):
    """The inverse multiply with a complex lower-triangular block runs as a real product on the
    block's real form, which is lower triangular in 2 x 2 blocks (a_lower = 2: entry (i, k) used
    when k <= i | 1). The upper part holds NaN in both forms and must never be read; the result
    must match the complex product (a_lower = 1) bit for bit."""
    import torch
    rng = np.random.default_rng(M + 5 * N)
    A = rand(dtype, (M, M), rng)             # column-major: [k, :] is column k
    L = A.T.copy()
    L[np.triu_indices(M, 1)] = np.nan
    A = np.ascontiguousarray(L.T)
    B = rand(dtype, (N, M), rng)
    C = rand(dtype, (N, M), rng)
    rdt = synth.NP_DTYPE[real]
    Ar = A.view(rdt)
    E = np.empty((2 * M, 2 * M), dtype=rdt)
    E[0::2] = Ar
    E[1::2, 0::2] = -Ar[:, 1::2]
    E[1::2, 1::2] = Ar[:, 0::2]
    say("complex lower vs real form", dtype, M, N)
    dA, dB, dC1 = to_dev(A), to_dev(B), to_dev(C)
    dE, dC2 = to_dev(E), to_dev(C)
    tr = torch.float32 if real == "f32" else torch.float64
    assert hs.entry("gemm", dtype)(M, N, M, 1.0, dA, M, dB, M, 0.0, dC1, M, 1) == hs.SUCCESS
    assert hs.entry("gemm", real)(2 * M, N, 2 * M, 1.0, dE, 2 * M, dB.view(tr), 2 * M, 0.0, dC2.view(tr),
                                  2 * M, 2) == hs.SUCCESS
    torch.cuda.synchronize()
    assert torch.equal(dC1.view(torch.uint8), dC2.view(torch.uint8))
    assert not torch.isnan(dC1.view(tr)).any()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("m,nb", [(100, 64), (256, 128), (1000, 256), (700, 512), (48, 64)])
def test_diag_inv(hs, dtype, m, nb):
    import torch
    if dtype == "c128" and nb > 512:
        pytest.skip("nb > 512 not offered for c128")
    say("diag_inv", dtype, m, nb)
    A = synth.tri(dtype, m, seed=m + nb)                     # (1, m, m) column-major
    nt = (m + nb - 1) // nb
    dA = to_dev(A)
    dI = torch.full((nt * nb * nb,), float("nan"), device="cuda",
                    dtype={"f32": torch.float32, "f64": torch.float64, "c64": torch.complex64,
                           "c128": torch.complex128}[dtype])
    st = hs.entry("diag_inv", dtype)(m, nb, nb // 8, dA, m, dI)
    torch.cuda.synchronize()
    assert st == hs.SUCCESS
    inv = dI.cpu().numpy().reshape(nt, nb, nb)              # [t, col, row]
    L = A[0].T                                              # [i, j]
    for t in range(nt):
        r0 = t * nb
        rb = min(nb, m - r0)
        Dt = np.ascontiguousarray(L[r0:r0 + rb, r0:r0 + rb])
        ref = oracle.trsm(Dt, np.eye(rb, dtype=Dt.dtype))
        got = inv[t].T                                      # [row, col]
        assert rel_err(got[None, :rb, :rb], ref[None]) <= TOL_LARGE[dtype]
        assert np.all(got[np.triu_indices(nb, 1)] == 0)     # explicit zeros above the diagonal
        if rb < nb:                                         # identity padding
            assert np.all(got[rb:, :rb] == 0) and np.all(got[:rb, rb:] == 0)
            assert np.array_equal(got[rb:, rb:], np.eye(nb - rb))


def test_diag_inv_bidiagonal_exact(hs):
    """A bidiagonal (1, -1) block has the all-ones lower triangle as inverse, exactly."""
    import torch
    m, nb = 300, 128
    L = np.full((m, m), np.nan)
    L[np.tril_indices(m, -1)] = 0
    L[np.diag_indices(m)] = 1
    L[np.arange(1, m), np.arange(m - 1)] = -1
    dA = to_dev(np.ascontiguousarray(L.T))
    nt = 3
    dI = torch.zeros(nt * nb * nb, dtype=torch.float64, device="cuda")
    assert hs.hsma_diag_inv_d(m, nb, 16, dA, m, dI) == hs.SUCCESS
    torch.cuda.synchronize()
    inv = dI.cpu().numpy().reshape(nt, nb, nb)
    for t in range(nt):
        rb = min(nb, m - t * nb)
        assert np.array_equal(inv[t].T[:rb, :rb], np.tril(np.ones((rb, rb))))


def blocked_solve(hs, dtype, m, n, nb, alpha=1.0, seed=0, lda=None, ldb=None, ib=0):
    import torch
    lda, ldb = lda or m, ldb or m
    A, B = colmajor_inputs(dtype, m, n, 1, lda=lda, ldb=ldb, seed=seed)
    dA, dB = to_dev(A), to_dev(B)
    st = hs.entry("ex", dtype)(m, n, alpha, dA, lda, dB, ldb,
                               {"nb": nb, "ib": ib, "path": hs.PATH_BLOCKED})
    torch.cuda.synchronize()
    assert st == hs.SUCCESS, hs.status_string(st)
    return A, B, dB.cpu().numpy()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("m,n", [(65, 1), (100, 64), (1000, 37), (1024, 200), (1500, 64)])
@pytest.mark.parametrize("nb", [64, 128, 256, 512])
def test_blocked_trsm(hs, dtype, m, n, nb):
    say("blocked", dtype, m, n, nb)
    A, B, X = blocked_solve(hs, dtype, m, n, nb, seed=m + n + nb)
    Av, Bv = views(A, B, m)
    Xo = oracle.trsm(Av, Bv)
    Xg = X[:, :, :m].transpose(0, 2, 1)
    assert rel_err(Xg, Xo) <= TOL_LARGE[dtype]
    assert scaled_residual(np.ascontiguousarray(Av), Xg, Bv, 1.0) <= 10 * m * EPS[dtype]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("m,n,nb", [(2048, 100, 1024), (3000, 70, 1024), (4096, 64, 2048),
                                    (2048, 33, 2048)])
def test_blocked_trsm_large_blocks(hs, dtype, m, n, nb):
    """N_B = 1024 / 2048: the blocked-inverse formula (m a multiple of N_B) and,
    for m = 3000 with N_B = 1024 in the real and c64 types, the column
    substitution kernel with its short last block; c128 above 512 and any
    type above 1024 need m to be a multiple of N_B."""
    if (nb > 1024 or dtype == "c128") and m % nb != 0:
        pytest.skip("N_B above the column-substitution limit needs m % N_B == 0")
    say("blocked large nb", dtype, m, n, nb)
    A, B, X = blocked_solve(hs, dtype, m, n, nb, seed=m + n + nb)
    Av, Bv = views(A, B, m)
    Xo = oracle.trsm(Av, Bv)
    Xg = X[:, :, :m].transpose(0, 2, 1)
    assert rel_err(Xg, Xo) <= TOL_LARGE[dtype]
    assert scaled_residual(np.ascontiguousarray(Av), Xg, Bv, 1.0) <= 10 * m * EPS[dtype]


@pytest.mark.parametrize("dtype", DTYPES)
def test_blocked_alpha_and_padding(hs, dtype):
    alpha = 0.3 + 0.7j if dtype.startswith("c") else -1.5
    say("blocked alpha", dtype)
    A, B, X = blocked_solve(hs, dtype, 300, 90, 128, alpha=alpha, lda=311, ldb=305)
    Av, Bv = views(A, B, 300)
    Xo = oracle.trsm(Av, Bv, alpha)
    assert rel_err(X[:, :, :300].transpose(0, 2, 1), Xo) <= TOL_LARGE[dtype]
    assert np.array_equal(X[:, :, 300:], B[:, :, 300:])


def test_blocked_exact_integer_all_nb(hs):
    """Bidiagonal (1, -1) system with integer B: X = running sums exactly, for every N_B
    (m = 700: short last blocks; m = 4096 for the blocks above 512 rows)."""
    import torch
    n = 48
    rng = np.random.default_rng(1)
    for m, nbs in ((700, (64, 128, 256, 512)), (4096, (1024, 2048))):
        L = np.full((m, m), np.nan)
        L[np.tril_indices(m, -1)] = 0
        L[np.diag_indices(m)] = 1
        L[np.arange(1, m), np.arange(m - 1)] = -1
        Bm = rng.integers(-30, 30, (m, n)).astype(np.float64)
        for nb in nbs:
            say("exact blocked", m, nb)
            dA = to_dev(np.ascontiguousarray(L.T))
            dB = to_dev(np.ascontiguousarray(Bm.T))
            assert hs.hsma_trsm_ex_d(m, n, 1.0, dA, m, dB, m, {"nb": nb, "path": 2}) == hs.SUCCESS
            torch.cuda.synchronize()
            assert np.array_equal(dB.cpu().numpy().T, np.cumsum(Bm, axis=0))


@pytest.mark.parametrize("dtype", DTYPES)
def test_default_path_large(hs, dtype):
    """Auto dispatch (table N_B) at m = 2048 through the plain entry point."""
    import torch
    m, n = 2048, 96
    say("auto", dtype, m, n)
    A, B = colmajor_inputs(dtype, m, n, 1, seed=3)
    dA, dB = to_dev(A), to_dev(B)
    assert hs.entry("trsm", dtype)(m, n, 1.0, dA, m, dB, m) == hs.SUCCESS
    torch.cuda.synchronize()
    Av, Bv = views(A, B, m)
    assert rel_err(dB.cpu().numpy()[:, :, :m].transpose(0, 2, 1), oracle.trsm(Av, Bv)) <= TOL_LARGE[dtype]


@pytest.mark.parametrize("dtype", DTYPES)
def test_full_size_sampled_columns(hs, dtype):
    """m = n = 8192 as the benchmark runs it (table N_B, one call), checked on 64
    seeded columns that the oracle solves one by one."""
    import torch
    m = n = 8192
    say("full 8192", dtype)
    A = synth.tri(dtype, m, seed=0x5EED0003)
    B = synth.rhs(dtype, m, n, seed=0x5EED0003 + 1)
    dA, dB = to_dev(A), to_dev(B)
    assert hs.entry("trsm", dtype)(m, n, 1.0, dA, m, dB, m) == hs.SUCCESS
    torch.cuda.synchronize()
    cols = synth.pick_columns(n, 64, seed=0x5EED0003)
    Xg = dB[0, torch.from_numpy(cols).cuda()].cpu().numpy()          # (64, m)
    del dA, dB
    Av = A[0].T
    Bs = B[0, cols].T
    Xo = oracle.trsm(Av, Bs)                                         # (m, 64)
    assert rel_err(Xg.T[None], Xo[None]) <= TOL_LARGE[dtype]


@pytest.mark.parametrize("dtype", ["f32", "f64", "c128"])
def test_largest_size_sampled_columns_and_residual(hs, dtype):
    """m = n = 16384 (the largest blocked size), one call with the table N_B:
    64 seeded columns against the oracle, and the scaled residual of the whole
    solution ||tril(A) X - B||_F / (||tril(A)||_F ||X||_F) <= 10 m eps, formed
    with plain torch products in double precision on the GPU."""
    import torch
    m = n = 16384
    say("full 16384", dtype)
    A = synth.tri(dtype, m, seed=0x5EED0004)
    B = synth.rhs(dtype, m, n, seed=0x5EED0004 + 1)
    dA, dB = to_dev(A), to_dev(B)
    assert hs.entry("trsm", dtype)(m, n, 1.0, dA, m, dB, m) == hs.SUCCESS
    torch.cuda.synchronize()
    cols = synth.pick_columns(n, 64, seed=0x5EED0004)
    Xg = dB[0, torch.from_numpy(cols).cuda()].cpu().numpy()          # (64, m)
    # residual: storage is column-major, so dA[0] holds A^T and dB[0] holds X^T
    wide = torch.complex128 if dtype.startswith("c") else torch.float64
    AT = torch.nan_to_num(dA[0].to(wide), nan=0.0)
    del dA
    AT = torch.triu(AT)                                              # tril(A)^T
    XT = dB[0].to(wide)
    del dB
    RT = XT @ AT                                                     # (tril(A) X)^T
    RT -= torch.from_numpy(B[0]).cuda().to(wide)
    num = torch.linalg.vector_norm(RT).item()
    den = torch.linalg.vector_norm(AT).item() * torch.linalg.vector_norm(XT).item()
    del AT, XT, RT
    torch.cuda.empty_cache()
    say("residual", num / den)
    assert num / den <= 10 * m * EPS[dtype]
    Xo = oracle.trsm(A[0].T, B[0, cols].T)                           # (m, 64)
    assert rel_err(Xg.T[None], Xo[None]) <= TOL_LARGE[dtype]
