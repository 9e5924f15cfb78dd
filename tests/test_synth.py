"""CPU checks of the seeded input generator shared by oracle and library tests."""
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_reference_vector():
    vals = [int(l) for l in open(os.path.join(GOLDEN, "splitmix64_seed1234567.txt"))
            if l.strip() and not l.startswith("#")]
    state = 1234567
    for v in vals:
        state = (state + 0x9E3779B97F4A7C15) & ((1 << 64) - 1)
        assert synth.mix64(state) == v


@pytest.mark.parametrize("dtype", synth.DTYPES)
def test_distributions(dtype):
    m = 64
    A = synth.tri(dtype, m, batch=3, seed=1)
    for b in range(3):
        L = A[b].T  # [i, j]
        low = L[np.tril_indices(m, -1)]
        d = np.diag(L)
        up = L[np.triu_indices(m, 1)]
        parts = [low.real, low.imag] if dtype.startswith("c") else [low]
        for p in parts:
            assert np.all(np.abs(p) <= 1.0 / m)
            assert p.std() > 0.3 / m
        dparts = [d.real, d.imag] if dtype.startswith("c") else [d]
        for p in dparts:
            assert np.all((p >= 1) & (p <= 2))
        assert np.all(np.isnan(up.real))
    B = synth.rhs(dtype, m, 64, batch=2, seed=2)
    parts = [B.real, B.imag] if dtype.startswith("c") else [B]
    for p in parts:
        assert np.all((p >= -1) & (p <= 1))
        assert abs(p.mean()) < 0.05
    if dtype.startswith("c"):
        assert abs(np.corrcoef(B.real.ravel(), B.imag.ravel())[0, 1]) < 0.05


def test_deterministic_and_layout_independent():
    a1 = synth.tri("f32", 40, 2, seed=5, ld=45)
    a2 = synth.tri("f32", 40, 2, seed=5)
    assert np.array_equal(np.nan_to_num(a1[:, :, :40]), np.nan_to_num(a2))
    r = synth.tri("f32", 40, 2, seed=5, layout="row")
    assert np.array_equal(np.nan_to_num(r.transpose(0, 2, 1)), np.nan_to_num(a2))
    b1 = synth.rhs("c128", 33, 7, 2, seed=8)
    b2 = synth.rhs("c128", 33, 7, 2, seed=8, layout="row")
    assert np.array_equal(b1.transpose(0, 2, 1), b2)
    assert not np.array_equal(synth.rhs("f64", 8, 8, seed=1), synth.rhs("f64", 8, 8, seed=2))


def test_column_subset():
    full = synth.rhs("f64", 50, 300, seed=3)[0]
    cols = synth.pick_columns(300, 64, seed=3)
    assert len(set(cols.tolist())) == 64 and np.all(np.diff(cols) > 0)
    assert cols.min() >= 0 and cols.max() < 300
    sub = synth.rhs("f64", 50, 0, seed=3, cols=cols)[0]
    assert np.array_equal(sub, full[cols])
