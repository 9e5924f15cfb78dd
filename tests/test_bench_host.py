"""CPU checks of the benchmark's accounting (no GPU needed)."""
import os

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_ggml_byte_convention():
    """The SOLVE_TRI perf line counts full A + B + X bytes, in KiB and GiB/s."""
    kv = {}
    for l in open(os.path.join(GOLDEN, "ggml_solve_tri_perf_line.txt")):
        if l.strip() and not l.startswith("#"):
            k, *v = l.split()
            kv[k] = [float(x) for x in v]
    n, _, b2, b3 = kv["ne_lhs"]
    k, _, _, _ = kv["ne_rhs"]
    nbytes = bench.ggml_bytes(int(n), int(k), int(b2 * b3), 4)
    assert round(nbytes / 1024) == kv["kB_per_run"][0]
    assert round(nbytes / (kv["us_per_run"][0] * 1e-6) / 2 ** 30, 2) == kv["GB_per_s"][0]


def test_flop_and_byte_counts():
    # LAPACK count: m^2 n real, 4 m^2 n complex
    assert bench.lapack_flops("f32", 64, 64) == 262144
    assert bench.lapack_flops("c128", 64, 64) == 1048576
    # triangle (2080 elements) + B read + X write
    assert bench.small_bytes("f32", 64, 64) == 41088
    assert bench.small_bytes("c128", 64, 64) == 164352


def test_multi_gpu_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cpu_baseline_repeats_to_its_time_budget():
    """The CPU baseline times the oracle on the step's problems, repeated until
    its time budget is spent, and reports the repeats and thread count."""
    host = {dt: bench.batched_inputs(dt, 64, 64, 8, seed=7) for dt in bench.DTYPES}
    out = bench.cpu_baseline(host, min_seconds=0.2)
    assert out["kind"] == "oracle" and out["unit"] == "GFLOPS"
    assert out["seconds"] >= 0.2 and out["repeats"] >= 1 and out["cores"] >= 1
    flops = sum(bench.lapack_flops(dt, 64, 64) * 8 for dt in bench.DTYPES) * out["repeats"]
    assert abs(out["value"] - flops / out["seconds"] / 1e9) <= 1e-9 * out["value"]
    assert "%d times" % out["repeats"] in out["sample"]
