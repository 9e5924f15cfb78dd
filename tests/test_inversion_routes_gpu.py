"""GPU parity of the three diagonal-block inversion routes against the
oracle's inverse (the oracle solve with the identity as right-hand side):
the blocked-inverse formula from 64 x 64 sub-blocks, the fused route (each
2*I_B x 2*I_B block inverted whole in LDS, then the same merges) and the
column-level substitution; and whole blocked solves through each route."""
import numpy as np
import pytest

import oracle
import synth
from _gpu_util import TOL_LARGE, colmajor_inputs, rel_err, say, to_dev, views

pytestmark = pytest.mark.gpu

TORCH = {"f32": "float32", "f64": "float64", "c64": "complex64", "c128": "complex128"}


@pytest.fixture(scope="module")
def hs():
    import torch  # noqa: F401
    import triangular_solve_amd as hs
    return hs


def routes(hs, dt, nb):
    out = [("blocked", {"inv": hs.INV_BLOCKED})]
    for ib in (32, 64):
        if ib == 64 and dt == "c128":
            continue
        if nb % (2 * ib) == 0:
            out.append(("fused%d" % ib, {"inv": hs.INV_FUSED, "ib": ib}))
    if nb <= 1024:
        out.append(("column", {"inv": hs.INV_COLUMN}))
    return out


@pytest.mark.parametrize("dt", ["f32", "f64", "c64", "c128"])
@pytest.mark.parametrize("m,nb", [(256, 128), (1024, 256), (2048, 1024)])
def test_inverse_routes(hs, dt, m, nb):
    import torch
    if dt == "c128" and nb > 512 and m % nb:
        pytest.skip("not offered")
    A = synth.tri(dt, m, seed=m + nb)
    dA = to_dev(A)
    nt = m // nb
    L = A[0].T
    refs = []
    for t in range(nt):
        Dt = np.ascontiguousarray(L[t * nb:(t + 1) * nb, t * nb:(t + 1) * nb])
        refs.append(oracle.trsm(Dt, np.eye(nb, dtype=Dt.dtype)))
    for name, o in routes(hs, dt, nb):
        say("inverse route", dt, m, nb, name)
        dI = torch.full((nt * nb * nb,), float("nan"), device="cuda", dtype=getattr(torch, TORCH[dt]))
        st = hs.entry("diag_inv_ex", dt)(m, dict(o, nb=nb), dA, m, dI)
        torch.cuda.synchronize()
        assert st == hs.SUCCESS, (name, st)
        inv = dI.cpu().numpy().reshape(nt, nb, nb)
        for t in range(nt):
            got = inv[t].T
            assert rel_err(got[None], refs[t][None]) <= TOL_LARGE[dt], (name, t)
            assert np.all(got[np.triu_indices(nb, 1)] == 0), name


def test_fused_bidiagonal_exact(hs):
    """A bidiagonal (1, -1) matrix: every route gives the all-ones lower
    triangle, exactly (every intermediate is a small integer)."""
    import torch
    m, nb = 512, 256
    L = np.full((m, m), np.nan)
    L[np.tril_indices(m, -1)] = 0
    L[np.diag_indices(m)] = 1
    L[np.arange(1, m), np.arange(m - 1)] = -1
    dA = to_dev(np.ascontiguousarray(L.T))
    for o in ({"inv": hs.INV_FUSED, "ib": 64}, {"inv": hs.INV_FUSED, "ib": 32},
              {"inv": hs.INV_BLOCKED}, {"inv": hs.INV_COLUMN}):
        dI = torch.zeros(2 * nb * nb, dtype=torch.float64, device="cuda")
        assert hs.hsma_diag_inv_ex_d(m, dict(o, nb=nb), dA, m, dI) == hs.SUCCESS
        torch.cuda.synchronize()
        inv = dI.cpu().numpy().reshape(2, nb, nb)
        for t in range(2):
            assert np.array_equal(inv[t].T, np.tril(np.ones((nb, nb)))), o


@pytest.mark.parametrize("dt", ["f32", "f64", "c64", "c128"])
def test_solve_through_each_route(hs, dt):
    import torch
    m, n, nb = 1024, 96, 256
    A, B = colmajor_inputs(dt, m, n, 1, seed=5)
    Av, Bv = views(A, B, m)
    Xo = oracle.trsm(Av, Bv)
    for name, o in routes(hs, dt, nb):
        dA, dB = to_dev(A), to_dev(B)
        st = hs.entry("ex", dt)(m, n, 1.0, dA, m, dB, m, dict(o, nb=nb, path=hs.PATH_BLOCKED))
        torch.cuda.synchronize()
        assert st == hs.SUCCESS, (name, st)
        Xg = dB.cpu().numpy()[:, :, :m].transpose(0, 2, 1)
        assert rel_err(Xg, Xo) <= TOL_LARGE[dt], name


def test_route_checks(hs):
    BAD = 0xDEAD000
    f = hs.hsma_diag_inv_ex_z
    assert f(512, {"nb": 256, "ib": 64, "inv": hs.INV_FUSED}, BAD, 512, BAD) == hs.INVALID_VALUE
    assert hs.hsma_diag_inv_ex_d(500, {"nb": 128, "ib": 64, "inv": hs.INV_FUSED}, BAD, 500, BAD) == \
        hs.INVALID_VALUE    # m not a multiple of nb
    assert hs.hsma_diag_inv_ex_d(512, {"nb": 128, "inv": 9}, BAD, 512, BAD) == hs.INVALID_VALUE
    assert hs.hsma_trsm_ex_d(2048, 4, 1, BAD, 2048, BAD, 2048,
                             {"nb": 2048, "inv": hs.INV_COLUMN}) == hs.INVALID_VALUE


@pytest.mark.parametrize("dt,m,nb,auto_is", [("f64", 1024, 128, "column"), ("f32", 1024, 256, "blocked"),
                                               ("f64", 1024, 256, "blocked"), ("c128", 1024, 256, "column"),
                                               ("c128", 1024, 512, "blocked"), ("c64", 1024, 128, "column"),
                                               ("c64", 2048, 512, "blocked")])
def test_each_route_runs_its_own_arithmetic(hs, dt, m, nb, auto_is):
    """An explicit route is the route that runs (the three give results that
    differ in rounding), and AUTO is bitwise the route it is documented to
    take for this dtype and block size."""
    import torch
    dA = to_dev(synth.tri(dt, m, seed=3))
    nt = m // nb
    got = {}
    for name, o in routes(hs, dt, nb) + [("auto", {"inv": hs.INV_AUTO})]:
        say("route dispatch", dt, m, nb, name)
        dI = torch.zeros(nt * nb * nb, device="cuda", dtype=getattr(torch, TORCH[dt]))
        assert hs.entry("diag_inv_ex", dt)(m, dict(o, nb=nb), dA, m, dI) == hs.SUCCESS, name
        torch.cuda.synchronize()
        got[name] = dI.cpu().numpy()
    assert not np.array_equal(got["blocked"], got["column"])
    assert not np.array_equal(got["blocked"], got["fused32"])
    assert np.array_equal(got["auto"], got[auto_is])
