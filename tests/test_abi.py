"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsma_trsm.h")


@pytest.fixture(scope="module")
def hs():
    import triangular_solve_amd as hs
    return hs


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hsma_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(hs):
    lib = ctypes.CDLL(hs.LIB_PATH)
    names = declared_functions()
    assert len(names) == 36
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(names) == hs.EXPORTS


def test_status_strings(hs):
    assert hs.hsma_status_string(0) == "success"
    assert hs.hsma_status_string(hs.NOT_SUPPORTED) == "not supported"
    assert hs.hsma_status_string(12345) == "unknown status"


BAD = 0xDEAD000  # never dereferenced: every call below returns before any GPU work


@pytest.mark.parametrize("t", ["f32", "f64", "c64", "c128"])
def test_trsm_argument_checks(hs, t):
    f = hs.entry("trsm", t)
    assert f(-1, 4, 1, BAD, 4, BAD, 4, 0) == hs.INVALID_SIZE
    assert f(4, -1, 1, BAD, 4, BAD, 4, 0) == hs.INVALID_SIZE
    assert f(4, 4, 1, BAD, 3, BAD, 4, 0) == hs.INVALID_SIZE       # lda < m
    assert f(4, 4, 1, BAD, 4, BAD, 3, 0) == hs.INVALID_SIZE       # ldb < m
    assert f(0, 4, 1, BAD, 0, BAD, 0, 0) == hs.INVALID_SIZE       # lda < 1
    assert f(0, 4, 1, None, 1, None, 1, 0) == hs.SUCCESS          # empty: nothing touched
    assert f(4, 0, 1, None, 4, None, 4, 0) == hs.SUCCESS
    assert f(4, 4, 1, BAD, 4, None, 4, 0) == hs.INVALID_POINTER   # B NULL
    assert f(4, 4, 1, None, 4, BAD, 4, 0) == hs.INVALID_POINTER   # A NULL, alpha != 0


@pytest.mark.parametrize("t", ["f32", "c128"])
def test_batched_argument_checks(hs, t):
    f = hs.entry("strided_batched", t)
    assert f(8, 8, 1, BAD, 8, 64, BAD, 8, 63, 2, 0) == hs.INVALID_SIZE   # overlapping B blocks
    assert f(8, 8, 1, BAD, 8, -1, BAD, 8, 64, 2, 0) == hs.INVALID_SIZE
    assert f(8, 8, 1, BAD, 8, 64, BAD, 8, 64, -1, 0) == hs.INVALID_SIZE
    assert f(8, 8, 1, BAD, 8, 64, BAD, 8, 64, 0, 0) == hs.SUCCESS
    assert f(8, 8, 1, None, 8, 0, BAD, 8, 64, 3, 0) == hs.INVALID_POINTER


def test_ex_option_checks(hs):
    f = hs.entry("ex", "f64")
    assert f(100, 4, 1, BAD, 100, BAD, 100, {"path": 7}, 0) == hs.INVALID_VALUE
    assert f(100, 4, 1, BAD, 100, BAD, 100, {"path": hs.PATH_SMALL}, 0) == hs.INVALID_VALUE
    assert f(513, 4, 1, BAD, 513, BAD, 513, {"path": hs.PATH_ROWS64}, 0) == hs.INVALID_VALUE
    assert f(100, 4, 1, BAD, 100, BAD, 100, {"path": 4}, 0) == hs.INVALID_VALUE
    assert f(100, 4, 1, BAD, 100, BAD, 100, {"nb": 100}, 0) == hs.INVALID_VALUE   # not a multiple of 16
    assert f(100, 4, 1, BAD, 100, BAD, 100, {"nb": 2048}, 0) == hs.INVALID_VALUE
    assert f(100, 4, 1, BAD, 100, BAD, 100, {"nb": 128, "ib": 3}, 0) == hs.INVALID_VALUE
    assert f(100, 4, 1, BAD, 100, BAD, 100, {"nb": 128, "ib": 1}, 0) == hs.INVALID_VALUE  # nb/ib > 64
    assert hs.entry("ex", "c128")(600, 4, 1, BAD, 600, BAD, 600, {"nb": 1024}, 0) == hs.INVALID_VALUE
    # blocks above 1024 rows (512 for c128) need m to be a multiple of nb
    assert f(3000, 4, 1, BAD, 3000, BAD, 3000, {"nb": 2048}, 0) == hs.INVALID_VALUE
    assert f(3000, 4, 1, BAD, 3000, BAD, 3000, {"nb": 4096}, 0) == hs.INVALID_VALUE  # above 2048
    assert hs.entry("ex", "c128")(3000, 4, 1, BAD, 3000, BAD, 3000, {"nb": 1024}, 0) == hs.INVALID_VALUE
    assert hs.entry("diag_inv", "f32")(3000, 2048, 0, BAD, 3000, BAD, 0) == hs.INVALID_VALUE


def test_solve_tri_checks(hs):
    f = hs.hsma_solve_tri_f32
    # n <= 256 is handled (in blocks of 64 above 64); larger n is not supported
    assert f(257, 8, BAD, BAD, BAD, 4, 1, 257, 257 * 257, 4 * 257 * 257, 8, 8 * 257, 4 * 8 * 257,
             8, 8 * 257, 4 * 8 * 257, 0) == hs.NOT_SUPPORTED
    assert f(128, 8, BAD, BAD, BAD, 4, 1, 127, 128 * 128, 4 * 128 * 128, 8, 8 * 128, 4 * 8 * 128,
             8, 8 * 128, 4 * 8 * 128, 0) == hs.INVALID_SIZE    # row stride below n
    assert f(128, 8, BAD, None, BAD, 4, 1, 128, 128 * 128, 4 * 128 * 128, 8, 8 * 128, 4 * 8 * 128,
             8, 8 * 128, 4 * 8 * 128, 0) == hs.INVALID_POINTER
    assert f(64, 6, BAD, BAD, BAD, 4, 2, 63, 4096, 16384, 6, 384, 1536, 6, 384, 1536, 0) == hs.INVALID_SIZE
    assert f(64, 6, BAD, None, BAD, 4, 2, 64, 4096, 16384, 6, 384, 1536, 6, 384, 1536, 0) == hs.INVALID_POINTER
    assert f(64, 0, None, None, None, 4, 2, 64, 4096, 16384, 6, 384, 1536, 6, 384, 1536, 0) == hs.SUCCESS
    assert f(-1, 6, BAD, BAD, BAD, 4, 2, 64, 4096, 16384, 6, 384, 1536, 6, 384, 1536, 0) == hs.INVALID_SIZE


def test_gemm_and_diag_inv_checks(hs):
    g = hs.entry("gemm", "f32")
    assert g(4, 4, 5, 1, BAD, 4, BAD, 5, 0, BAD, 4, 1, 0) == hs.INVALID_SIZE   # lower needs M == K
    assert g(4, 4, 4, 1, BAD, 4, BAD, 4, 0.5, BAD, 4, 0, 0) == hs.INVALID_VALUE
    assert g(4, 4, 4, 1, BAD, 3, BAD, 4, 0, BAD, 4, 0, 0) == hs.INVALID_SIZE
    assert g(0, 4, 4, 1, None, 1, None, 4, 0, None, 1, 0, 0) == hs.SUCCESS
    # a_lower: 0, 1 or (real types, M even) 2 = lower triangular in 2 x 2 blocks
    assert g(4, 4, 4, 1, BAD, 4, BAD, 4, 0, BAD, 4, 3, 0) == hs.INVALID_VALUE
    assert g(4, 4, 4, 1, BAD, 4, BAD, 4, 0, BAD, 4, -1, 0) == hs.INVALID_VALUE
    assert g(5, 4, 5, 1, BAD, 5, BAD, 5, 0, BAD, 5, 2, 0) == hs.INVALID_SIZE
    assert g(0, 4, 0, 1, None, 1, None, 1, 0, None, 1, 2, 0) == hs.SUCCESS
    assert hs.entry("gemm", "c64")(4, 4, 4, 1, BAD, 4, BAD, 4, 0, BAD, 4, 2, 0) == hs.INVALID_VALUE
    d = hs.entry("diag_inv", "f64")
    assert d(100, 100, 0, BAD, 100, BAD, 0) == hs.INVALID_VALUE
    assert d(100, 128, 1, BAD, 100, BAD, 0) == hs.INVALID_VALUE
    assert d(100, 128, 16, BAD, 99, BAD, 0) == hs.INVALID_SIZE
    assert d(100, 128, 16, None, 100, BAD, 0) == hs.INVALID_POINTER
    assert d(0, 128, 16, None, 1, None, 0) == hs.SUCCESS


def nb_table():
    """The built-in N_B table as {dtype code: [(m, n, nb), ...]}."""
    text = open(os.path.join(ROOT, "triangular_solve_amd", "csrc", "nb_table.inc")).read()
    out = {}
    for code, name in enumerate(["kNbF32", "kNbF64", "kNbC64", "kNbC128"]):
        body = re.search(r"static const NbEntry %s\[\] = \{(.*)\};" % name, text).group(1)
        out[code] = [tuple(int(v) for v in t) for t in re.findall(r"\{(\d+), (\d+), (\d+)\}", body)]
    return out


def expected_nb(entries, code, m, n):
    """The lookup rule: nearest tested shape by |log2 m - log2 m_i| + |log2 n - log2 n_i|
    (first entry on ties), halved until blocks above 1024 rows (512 for c128)
    divide m, clamped to m rounded up to a multiple of 16."""
    import math
    best, bd = None, 1e300
    for (mi, ni, nb) in entries:
        d = abs(math.log2(m) - math.log2(mi)) + abs(math.log2(max(n, 1)) - math.log2(ni))
        if d < bd - 1e-12:
            best, bd = nb, d
    nb = best
    while not (nb <= (512 if code == 3 else 1024) or m % nb == 0):
        nb //= 2
    cap = (m + 15) // 16 * 16
    return min(nb, max(cap, 16))


def test_block_size_table(hs):
    tab = nb_table()
    for code in range(4):
        assert hs.hsma_trsm_block_size(code, 64, 64) == 0
        assert len({(m, n) for m, n, _ in tab[code]}) == len(tab[code]) > 5
        for (m, n, nb) in tab[code]:       # every tested shape returns its own entry
            assert hs.hsma_trsm_block_size(code, m, n) == expected_nb(tab[code], code, m, n) == nb
        for m in (65, 100, 1000, 1024, 3000, 8192, 12000, 16384, 50000):
            for n in (1, 8, 64, 100, 700, 5000, 16384, 100000):
                nb = hs.hsma_trsm_block_size(code, m, n)
                assert nb == expected_nb(tab[code], code, m, n), (code, m, n)
                assert nb % 16 == 0 and 16 <= nb <= 2048
                assert nb <= ((m + 15) // 16) * 16
                assert nb <= (512 if code == 3 else 1024) or m % nb == 0
    assert hs.hsma_trsm_block_size(7, 100, 100) == -1


@pytest.mark.parametrize("t", ["f32", "f64", "c64", "c128"])
def test_alloc_failure_injection(hs, t, monkeypatch):
    """HSMA_TEST_FAIL_ALLOC=1 makes the workspace allocation fail: the blocked
    path and the diagonal inversion return ALLOC_FAILED before any GPU work
    (the pointers below are never dereferenced)."""
    monkeypatch.setenv("HSMA_TEST_FAIL_ALLOC", "1")
    assert hs.entry("trsm", t)(300, 8, 1, BAD, 300, BAD, 300, 0) == hs.ALLOC_FAILED
    assert hs.entry("ex", t)(300, 8, 1, BAD, 300, BAD, 300, {"nb": 128, "path": hs.PATH_BLOCKED},
                             0) == hs.ALLOC_FAILED
    assert hs.entry("strided_batched", t)(600, 8, 1, BAD, 600, 0, BAD, 600, 4800, 3, 0) == hs.ALLOC_FAILED
    assert hs.entry("diag_inv_ex", t)(1024, {"nb": 512, "inv": hs.INV_BLOCKED}, BAD, 1024, BAD,
                                      0) == hs.ALLOC_FAILED
    assert hs.hsma_status_string(hs.ALLOC_FAILED) == "workspace allocation failed"


def test_phase_event_checks(hs):
    """Phase-event options are validated before any GPU work: too few events
    returns INVALID_VALUE with the count needed."""
    import ctypes
    used = ctypes.c_int32(-5)
    phases = (ctypes.c_int32 * 4)()
    evs = (ctypes.c_void_p * 4)()
    o = hs.TrsmOpts(128, 0, hs.PATH_BLOCKED, 0, 4, evs, phases, ctypes.pointer(used))
    # m = 1000, nb = 128: 8 diagonal blocks -> 3*8 + 1 events (+1 with alpha != 1)
    assert hs.entry("ex", "f64")(1000, 4, 1, BAD, 1000, BAD, 1000, o, 0) == hs.INVALID_VALUE
    assert used.value == 25
    assert hs.entry("ex", "f64")(1000, 4, 2, BAD, 1000, BAD, 1000, o, 0) == hs.INVALID_VALUE
    assert used.value == 26
    bad = hs.TrsmOpts(128, 0, hs.PATH_BLOCKED, 0, 4, evs, None, ctypes.pointer(used))
    assert hs.entry("ex", "f64")(1000, 4, 1, BAD, 1000, BAD, 1000, bad, 0) == hs.INVALID_POINTER
    neg = hs.TrsmOpts(128, 0, hs.PATH_BLOCKED, 0, -1, None, None, None)
    assert hs.entry("ex", "f64")(1000, 4, 1, BAD, 1000, BAD, 1000, neg, 0) == hs.INVALID_VALUE


def test_noalloc_checks(hs, monkeypatch):
    """hsma_trsm_noalloc validates arguments and rejects problems beyond its
    scratch before any GPU work."""
    f = hs.hsma_trsm_noalloc
    assert f(7, 10, 10, 1.0, BAD, 10, BAD, 10, 0) == hs.INVALID_VALUE
    assert f(1, -1, 10, 1.0, BAD, 10, BAD, 10, 0) == hs.INVALID_SIZE
    assert f(1, 10, 10, 1.0, BAD, 9, BAD, 10, 0) == hs.INVALID_SIZE
    assert f(1, 0, 10, 1.0, None, 1, None, 1, 0) == hs.SUCCESS
    assert f(1, 10, 10, 1.0, BAD, 10, None, 10, 0) == hs.INVALID_POINTER
    # 16 * m * 8 bytes > 32 MiB
    assert f(1, 1 << 19, 4, 1.0, BAD, 1 << 19, BAD, 1 << 19, 0) == hs.SCRATCH_TOO_SMALL
    assert f(3, 200000, 4, 1.0, BAD, 200000, BAD, 200000, 0) == hs.SCRATCH_TOO_SMALL
    monkeypatch.setenv("HSMA_NOALLOC_LIMIT", "4096")
    assert f(0, 100, 4, 1.0, BAD, 100, BAD, 100, 0) == hs.SCRATCH_TOO_SMALL
    assert hs.hsma_status_string(hs.SCRATCH_TOO_SMALL) == "problem exceeds the no-allocation scratch"
