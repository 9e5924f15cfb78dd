#!/usr/bin/env python3
"""Benchmark of the MI355X triangular-solve library (left, lower, no-transpose,
non-unit TRSM), printing one JSON line.

Default workload (one "step"): the batched small regime, 4096 column-major
64 x 64 systems with 64 right-hand sides each, solved in f32, f64, c64 and
c128 (four launches of the library's small-regime kernel, one per dtype).
value = LAPACK-count GFLOPS of the whole step (m^2 n per real problem,
4 m^2 n per complex one). Inputs are resident in HBM before timing starts;
every step solves distinct copies of A and B (a ring larger than the 256 MB
MALL), so no step reads another step's data from cache.

The same line carries the blocked regime at m = n = 8192 (f32, f64, c64, c128)
and m = n = 16384 (f32, f64, c128): one solve per dtype, LAPACK GFLOPS, the
MFMA-peak fraction, the time split between diagonal inversion, GEMMs and the
rest measured inside one solve, 64-column parity and the oracle's time on
those columns. Then the SOLVE_TRI shape
(8 systems of 64 x 64 with 6 right-hand sides, ggml layout, us per call), the
roofline of the dominant kernel, and the CPU oracle timed on the same step.

  python bench.py [--steps K] [--warmup W] [--no-blocked] [--no-cpu]
  python bench.py --workload blocked --m 16384 --dtypes f32,f64,c128
"""
import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TRSM GFLOPS (m=64 batched; m=8192/16384 blocked) + % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f32": 157.3, "c64": 157.3, "f64": 78.6, "c128": 78.6}
ITEMSIZE = {"f32": 4, "f64": 8, "c64": 8, "c128": 16}
DTYPES = ["f32", "f64", "c64", "c128"]
SEED_CFG0, SEED_CFG1, SEED_CFG3 = 0x5EED0000, 0x5EED0001, 0x5EED0003


def lapack_flops(dtype, m, n):
    """LAPACK operation count of one m x m TRSM with n right-hand sides."""
    return (4 if dtype.startswith("c") else 1) * m * m * n


def small_bytes(dtype, m, n):
    """Algorithmic HBM bytes of one in-place small solve: triangle of A, read B, write X."""
    return (m * (m + 1) // 2 + 2 * m * n) * ITEMSIZE[dtype]


def ggml_bytes(n, k, nbatch, itemsize):
    """test-backend-ops byte count for SOLVE_TRI: full A + B + X."""
    return (n * n + 2 * n * k) * nbatch * itemsize


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------

def batched_inputs(dtype, m, n, batch, seed):
    import synth
    A = synth.tri(dtype, m, batch, seed=seed, offdiag_div=m)
    B = synth.rhs(dtype, m, n, batch, seed=seed + 1)
    return A, B


def bench_batched(hs, torch, steps, warmup, m=64, n=64, batch=4096, check=True):
    """Timed steps of the batched small regime over all four dtypes."""
    stream = torch.cuda.current_stream()
    nslot = 2  # each slot (all dtypes) is > 1 GB, so alternating slots defeats the MALL
    host, slots = {}, {}
    for dt in DTYPES:
        A, B = batched_inputs(dt, m, n, batch, SEED_CFG1)
        host[dt] = (A, B)
        dA = torch.from_numpy(A).cuda()
        dB = torch.from_numpy(B).cuda()
        slots[dt] = [(dA.clone(), dB.clone()) for _ in range(nslot)]
    f = {dt: hs.entry("strided_batched", dt) for dt in DTYPES}

    def launch(dt, slot):
        dA, dB = slots[dt][slot]
        st = f[dt](m, n, 1.0, dA, m, m * m, dB, m, m * n, batch, stream)
        if st != hs.SUCCESS:
            raise hs.HsmaError(st, "strided_batched_" + dt)

    parity = {}
    if check:
        import oracle
        for dt in DTYPES:
            launch(dt, 0)
        torch.cuda.synchronize()
        for dt in DTYPES:
            A, B = host[dt]
            sel = np.arange(0, batch, max(1, batch // 64))          # 64 problems, spread out
            Xg = slots[dt][0][1].cpu().numpy()[sel][:, :, :m].transpose(0, 2, 1)
            Xo = oracle.trsm(A[sel][:, :, :m].transpose(0, 2, 1), B[sel][:, :, :m].transpose(0, 2, 1))
            num = np.sqrt(np.sum(np.abs(Xg.astype(Xo.dtype) - Xo) ** 2, axis=(1, 2)))
            den = np.sqrt(np.sum(np.abs(Xo) ** 2, axis=(1, 2)))
            parity[dt] = float(np.max(num / den))
            slots[dt][0][1].copy_(torch.from_numpy(B).cuda())

    for s in range(warmup):
        for dt in DTYPES:
            launch(dt, s % nslot)
    torch.cuda.synchronize()
    ev = {dt: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)] for dt in DTYPES}
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for s in range(steps):
        for dt in DTYPES:
            ev[dt][s][0].record(stream)
            launch(dt, (warmup + s) % nslot)
            ev[dt][s][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    per = {}
    for dt in DTYPES:
        ms = [a.elapsed_time(b) for a, b in ev[dt]]
        avg = float(np.mean(ms))
        flops = lapack_flops(dt, m, n) * batch
        nbytes = small_bytes(dt, m, n) * batch
        per[dt] = {"ms_per_launch": avg, "gflops": flops / avg / 1e6,
                   "hbm_gbs": nbytes / avg / 1e6, "hbm_frac": nbytes / avg / 1e6 / HBM_PEAK_GBS,
                   "bytes_per_launch": nbytes, "rel_err": parity.get(dt)}
    step_flops = sum(lapack_flops(dt, m, n) * batch for dt in DTYPES)
    ms_per_step = total_ms / steps
    return {"ms_per_step": ms_per_step, "gflops": step_flops / ms_per_step / 1e6, "per_dtype": per,
            "wall_s": wall, "host": host}


def bench_batched_alone(hs, torch, host, m=64, n=64, batch=4096, launches=20):
    """Each dtype's batched launches back to back, with no other dtype in between (in the step,
    every launch follows another dtype's launch and measures slower). A ring of copies larger than
    the 256 MB last-level cache keeps every launch reading from HBM; HIP events around the
    group of launches on the launch stream, mean per launch."""
    stream = torch.cuda.current_stream()
    out = {}
    for dt in DTYPES:
        A, B = host[dt]
        dA = torch.from_numpy(A).cuda()
        dB = torch.from_numpy(B).cuda()
        set_bytes = (dA.numel() + dB.numel()) * dA.element_size()
        ns = max(2, -(-640 * 2 ** 20 // set_bytes))
        ring = [(dA.clone(), dB.clone()) for _ in range(ns)]
        del dA, dB
        f = hs.entry("strided_batched", dt)

        def launch(i):
            a, b = ring[i % ns]
            st = f(m, n, 1.0, a, m, m * m, b, m, m * n, batch, stream)
            if st != hs.SUCCESS:
                raise hs.HsmaError(st, "strided_batched_" + dt)

        for i in range(ns):
            launch(i)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(launches):
            launch(i)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / launches
        nbytes = small_bytes(dt, m, n) * batch
        out[dt] = {"ms_per_launch": ms, "gflops": lapack_flops(dt, m, n) * batch / ms / 1e6,
                   "hbm_gbs": nbytes / ms / 1e6, "hbm_frac": nbytes / ms / 1e6 / HBM_PEAK_GBS,
                   "launches": launches, "ring_copies": ns}
        del ring
        torch.cuda.empty_cache()
    return out


def bench_solve_tri(hs, torch, runs=2000, n=64, k=6, e2=4, e3=2):
    """A SOLVE_TRI shape of the llama.cpp PR, f32, ggml layout: by default its
    performance shape A [64,64,4,2], B [6,64,4,2]; with n = 128, k = 8, e2 = 4,
    e3 = 1 the [128,128,4,1] case its kernel reports as not supported."""
    import oracle
    import synth
    nb = e2 * e3
    A = synth.tri("f32", n, nb, seed=SEED_CFG0, offdiag_div=n, layout="row")
    B = synth.rhs("f32", n, k, nb, seed=SEED_CFG0 + 1, layout="row")
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    dX = torch.empty_like(dB)
    stream = torch.cuda.current_stream()
    args = (n, k, dA, dB, dX, e2, e3, n, n * n, e2 * n * n, k, n * k, e2 * n * k, k, n * k, e2 * n * k,
            stream.cuda_stream)
    assert hs.hsma_solve_tri_f32(*args) == hs.SUCCESS
    torch.cuda.synchronize()
    Xo = oracle.trsm(A, B)
    X = dX.cpu().numpy()
    err = float(np.sqrt(np.sum((X - Xo) ** 2) / np.sum(Xo ** 2)))
    nmse = err ** 2
    for _ in range(50):
        hs.hsma_solve_tri_f32(*args)
    samples = []
    for rep in range(10):   # 10 samples, the first one a warm-up, mean of the last 9
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(runs // 10):
            hs.hsma_solve_tri_f32(*args)
        b.record(stream)
        torch.cuda.synchronize()
        samples.append(a.elapsed_time(b) * 1e3 / (runs // 10))
    us = float(np.mean(samples[1:]))
    nbytes = ggml_bytes(n, k, nb, 4)
    return {"shape": "A[%d,%d,%d,%d] B[%d,%d,%d,%d] f32 (ggml layout, out of place)" % (n, n, e2, e3, k, n, e2, e3),
            "us_per_call": us, "ggml_kB_per_run": nbytes / 1024, "ggml_GiB_per_s": nbytes / (us * 1e-6) / 2 ** 30,
            "gflops": lapack_flops("f32", n, k) * nb / (us * 1e-6) / 1e9, "rel_err": err, "nmse": nmse,
            "launches_timed": runs}


def phase_split(hs, torch, f, m, dt, dA, dB, nbu, stream):
    """One blocked solve with the library's phase events: ms per phase, in
    the solve's own launch order (events recorded by the library between
    its launches on the stream)."""
    import ctypes
    nt = (m + nbu - 1) // nbu
    cap = 3 * nt + 2
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(cap)]
    for e in evs:            # creates the underlying HIP events
        e.record(stream)
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * cap)(*[e.cuda_event for e in evs])
    phases = (ctypes.c_int32 * cap)()
    used = ctypes.c_int32(0)
    opts = hs.TrsmOpts(nbu, 0, hs.PATH_BLOCKED, 0, cap, handles, phases, ctypes.pointer(used))
    hs.check(f(m, m, 1.0, dA, m, dB, m, opts, stream), "trsm_ex_" + dt + " (timed phases)")
    torch.cuda.synchronize()
    out = {name: 0.0 for name in hs.PHASE_NAMES.values()}
    for k in range(used.value - 1):
        out[hs.PHASE_NAMES[phases[k]]] += evs[k].elapsed_time(evs[k + 1])
    total = evs[0].elapsed_time(evs[used.value - 1])
    gemm = out["inv_gemm"] + out["trailing_gemm"]
    other = total - gemm - out["diag_inv"]
    return {"ms_with_events": total, "phase_ms": out, "events": used.value,
            "share": {"diag_inv": out["diag_inv"] / total, "gemm": gemm / total,
                      "other": other / total},
            "share_note": "gemm = inverse-block multiplies + trailing updates; other = W->B copies, "
                          "scaling and launch gaps"}


def bench_blocked(hs, torch, m, dtypes, runs=4, nb=0, cpu=True):
    """One blocked solve per dtype at m = n, B restored between runs (untimed);
    the phase split from a separate run with the library's phase events; 64
    seeded columns against the oracle, whose time on those columns is the
    configuration's CPU baseline."""
    import oracle
    import synth
    out = {}
    stream = torch.cuda.current_stream()
    for dt in dtypes:
        log("blocked", dt, m)
        A = synth.tri(dt, m, seed=SEED_CFG3)
        B = synth.rhs(dt, m, m, seed=SEED_CFG3 + 1)
        dA, dB0 = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        dB = dB0.clone()
        f = hs.entry("ex", dt)
        nbu = nb or hs.hsma_trsm_block_size(hs.DTYPE_CODE[dt], m)
        opts = {"nb": nbu, "path": hs.PATH_BLOCKED}
        times = []
        for r in range(runs + 1):     # first run is a warm-up
            dB.copy_(dB0)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            st = f(m, m, 1.0, dA, m, dB, m, opts, stream)
            b.record(stream)
            torch.cuda.synchronize()
            if st != hs.SUCCESS:
                raise hs.HsmaError(st, "trsm_ex_" + dt)
            times.append(a.elapsed_time(b))
        ms = float(np.mean(times[1:]))
        # sampled parity: 64 seeded columns against the oracle
        cols = synth.pick_columns(m, 64, seed=SEED_CFG3)
        Xg = dB[0, torch.from_numpy(cols).cuda()].cpu().numpy().T
        threads = oracle.default_threads()
        t0 = time.perf_counter()
        Xo = oracle.trsm(A[0].T, B[0, cols].T, threads=threads)
        osec = time.perf_counter() - t0
        err = float(np.linalg.norm(Xg.astype(Xo.dtype) - Xo) / np.linalg.norm(Xo))
        dB.copy_(dB0)
        split = phase_split(hs, torch, f, m, dt, dA, dB, nbu, stream)
        flops = lapack_flops(dt, m, m)
        out[dt] = {"ms": ms, "gflops": flops / ms / 1e6, "nb": nbu,
                   "mfma_peak_frac": flops / ms / 1e9 / MFMA_PEAK_TFLOPS[dt],
                   "phases": split, "rel_err_64cols": err,
                   "cpu_baseline": {
                       "value": lapack_flops(dt, m, 64) / osec / 1e9, "unit": "GFLOPS",
                       "cores": threads, "kind": "oracle",
                       "sample": "64 seeded right-hand-side columns of the m=n=%d %s solve, plain C "
                                 "double-precision forward substitution, %d threads on %s"
                                 % (m, dt, threads, cpu_model()),
                       "seconds_64cols": osec,
                       "extrapolated_full_n_seconds": osec * m / 64,
                       "extrapolation_note": "seconds_64cols x n/64, not measured"}}
        log("  %.3f ms, %.1f%% of MFMA peak, split %s" % (
            ms, 100 * out[dt]["mfma_peak_frac"],
            {k: round(v, 3) for k, v in split["share"].items()}))
        del dA, dB0, dB, A, B
        torch.cuda.empty_cache()
    return out


VARIANTS = [(s, u, t, d) for s in "LR" for u in "LU" for t in "NTC" for d in "NU"]


def bench_variants(hs, torch, m=8192, dtypes=("f32", "f64"), runs=2, nvec=8):
    """Every TRSM variant (side, triangle, op, diagonal) at m = n, one solve
    each after a warm-up: ms, LAPACK GFLOPS, MFMA fraction, and nvec sampled
    right-hand-side vectors (columns for the left side, rows for the right
    side) against the oracle's variant solve. For real types op C equals T
    and is not repeated."""
    import oracle
    import synth
    out = {}
    stream = torch.cuda.current_stream()
    for dt in dtypes:
        log("variants", dt, m)
        host = {"L": synth.tri(dt, m, seed=SEED_CFG3), "U": synth.tri(dt, m, seed=SEED_CFG3, layout="row")}
        B = synth.rhs(dt, m, m, seed=SEED_CFG3 + 1)
        dAs = {u: torch.from_numpy(a).cuda() for u, a in host.items()}
        dB0 = torch.from_numpy(B).cuda()
        dB = dB0.clone()
        f = hs.entry("general", dt)
        Bv = B[0].T                      # [i, c]
        sel = synth.pick_columns(m, nvec, seed=SEED_CFG3 + 7)
        for (side, uplo, trans, diag) in VARIANTS:
            if trans == "C" and not dt.startswith("c"):
                continue
            if diag == "U":
                continue     # same kernels as the non-unit case (the diagonal reads a constant)
            codes = (hs.SIDE[side], hs.UPLO[uplo], hs.OP[trans], hs.DIAG[diag])
            times = []
            for r in range(runs + 1):
                dB.copy_(dB0)
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                st = f(*codes, m, m, 1.0, dAs[uplo], m, dB, m, stream)
                b.record(stream)
                torch.cuda.synchronize()
                hs.check(st, "general_" + dt)
                times.append(a.elapsed_time(b))
            ms = float(np.mean(times[1:]))
            Xg = dB[0].cpu().numpy().T           # [i, c]
            Av = host[uplo][0].T
            if side == "L":
                Xo = oracle.trsm_general(Av, np.ascontiguousarray(Bv[:, sel]), side, uplo, trans, diag)
                got = Xg[:, sel]
            else:
                Xo = oracle.trsm_general(Av, np.ascontiguousarray(Bv[sel, :]), side, uplo, trans, diag)
                got = Xg[sel, :]
            err = float(np.linalg.norm(got.astype(Xo.dtype) - Xo) / np.linalg.norm(Xo))
            flops = lapack_flops(dt, m, m)
            out["%s %s%s%s%s" % (dt, side, uplo, trans, diag)] = {
                "ms": ms, "gflops": flops / ms / 1e6, "mfma_peak_frac": flops / ms / 1e9 / MFMA_PEAK_TFLOPS[dt],
                "rel_err_%d" % nvec: err}
        del dAs, dB0, dB, host, B
        torch.cuda.empty_cache()
    return out


def bench_inversion(hs, torch, cases=((8192, 2048), (8192, 1024), (2048, 512), (1024, 256), (1024, 128)),
                    dtypes=DTYPES, runs=5):
    """The diagonal-block inversion alone, per route (blocked-inverse formula
    from 64 x 64 sub-blocks; fused 2*I_B blocks in LDS then merges; column
    substitution), ms per call (mean of `runs` after a warm-up)."""
    import synth
    out = {}
    stream = torch.cuda.current_stream()
    tdt = {"f32": torch.float32, "f64": torch.float64, "c64": torch.complex64, "c128": torch.complex128}
    for dt in dtypes:
        for m in sorted({m for m, _ in cases}):
            A = torch.from_numpy(synth.tri(dt, m, seed=SEED_CFG3)).cuda()
            for (mm, nb) in cases:
                if mm != m or (dt == "c128" and nb > 512 and m % nb):
                    continue
                inv = torch.empty(m // nb * nb * nb, dtype=tdt[dt], device="cuda")
                routes = [("blocked", {"inv": hs.INV_BLOCKED})]
                for ib in (64, 32):
                    if not (ib == 64 and dt == "c128") and nb % (2 * ib) == 0:
                        routes.append(("fused_ib%d" % ib, {"inv": hs.INV_FUSED, "ib": ib}))
                if nb <= 1024:
                    routes.append(("column", {"inv": hs.INV_COLUMN}))
                res = {}
                for name, o in routes:
                    f = hs.entry("diag_inv_ex", dt)
                    hs.check(f(m, dict(o, nb=nb), A, m, inv, stream), "diag_inv_ex " + name)
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    for _ in range(runs):
                        f(m, dict(o, nb=nb), A, m, inv, stream)
                    b.record(stream)
                    torch.cuda.synchronize()
                    res[name] = a.elapsed_time(b) / runs
                out["%s m=%d nb=%d" % (dt, m, nb)] = res
                del inv
            del A
            torch.cuda.empty_cache()
    return out


def bench_few_rhs(hs, torch, m=8192, n=64, dtypes=DTYPES, runs=5):
    """Few right-hand sides (m x m, n columns), N_B from the (m, n) table."""
    import oracle
    import synth
    out = {}
    stream = torch.cuda.current_stream()
    for dt in dtypes:
        A = synth.tri(dt, m, seed=SEED_CFG3)
        B = synth.rhs(dt, m, n, seed=SEED_CFG3 + 1)
        dA, dB0 = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        dB = dB0.clone()
        f = hs.entry("trsm", dt)
        times = []
        for r in range(runs + 1):
            dB.copy_(dB0)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            hs.check(f(m, n, 1.0, dA, m, dB, m, stream), "trsm_" + dt)
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        ms = float(np.mean(times[1:]))
        Xg = dB[0].cpu().numpy().T[:, :8]
        Xo = oracle.trsm(A[0].T, np.ascontiguousarray(B[0].T[:, :8]))
        flops = lapack_flops(dt, m, n)
        out[dt] = {"ms": ms, "gflops": flops / ms / 1e6, "nb": hs.hsma_trsm_block_size(hs.DTYPE_CODE[dt], m, n),
                   "rel_err_8cols": float(np.linalg.norm(Xg.astype(Xo.dtype) - Xo) / np.linalg.norm(Xo))}
        del dA, dB0, dB
    return out


def medium_workload(hs, torch, m=128, n=64, batch=1024, reps=5):
    """Strided batches in the 64 < m <= 256 band (block rows of 64 over the
    whole batch): ms per batched call and GFLOPS per dtype, plus 64-problem
    parity against the oracle."""
    import oracle
    import synth
    out = {}
    stream = torch.cuda.current_stream()
    for dt in DTYPES:
        A = synth.tri(dt, m, batch, seed=SEED_CFG1)
        B = synth.rhs(dt, m, n, batch, seed=SEED_CFG1 + 1)
        dA, dB0 = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        dB = dB0.clone()
        f = hs.entry("strided_batched", dt)
        times = []
        for r in range(reps + 1):
            dB.copy_(dB0)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            hs.check(f(m, n, 1.0, dA, m, m * m, dB, m, m * n, batch, stream), "strided_batched_" + dt)
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        ms = float(np.mean(times[1:]))
        Xg = dB[:64].cpu().numpy()[:, :, :m].transpose(0, 2, 1)
        Xo = oracle.trsm(A[:64, :, :m].transpose(0, 2, 1), B[:64, :, :m].transpose(0, 2, 1))
        err = float(np.max([np.linalg.norm(Xg[i] - Xo[i]) / np.linalg.norm(Xo[i]) for i in range(64)]))
        out[dt] = {"ms": ms, "gflops": lapack_flops(dt, m, n) * batch / (ms * 1e6), "rel_err_64": err}
        del dA, dB, dB0
    return out


def gemm_workload(hs, torch, shapes=((7168, 8192, 1024), (6144, 8192, 2048)), reps=5):
    """The library GEMM at trailing-update shapes of the blocked solve
    (C -= A B, beta = 1), per dtype, against torch's own matmul on the same
    shapes for context (not part of any path); for the complex types also
    the real form of the product, which the blocked solve's trailing updates
    run."""
    out = {}
    stream = torch.cuda.current_stream()
    tdt = {"f32": torch.float32, "f64": torch.float64, "c64": torch.complex64, "c128": torch.complex128}
    torch.backends.cuda.matmul.allow_tf32 = False
    for dt in DTYPES:
        for (M, N, K) in shapes:
            g = torch.Generator(device="cuda").manual_seed(M + K)
            A = torch.rand(K, M, device="cuda", generator=g, dtype=tdt[dt])   # column-major M x K
            Bm = torch.rand(N, K, device="cuda", generator=g, dtype=tdt[dt])  # column-major K x N
            C = torch.rand(N, M, device="cuda", generator=g, dtype=tdt[dt])
            f = hs.entry("gemm", dt)

            def timed(fn):
                fn()
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(reps):
                    fn()
                b.record(stream)
                torch.cuda.synchronize()
                return a.elapsed_time(b) / reps

            ms = timed(lambda: hs.check(f(M, N, K, -1.0, A, M, Bm, K, 1.0, C, M, 0, stream), "gemm_" + dt))
            Ct, At, Bt = C.t(), A.t(), Bm.t()
            ms_t = timed(lambda: Ct.addmm_(At, Bt, alpha=-1))
            flops = (8 if dt.startswith("c") else 2) * M * N * K
            peak = MFMA_PEAK_TFLOPS[dt]
            row = {"ms": ms, "tflops": flops / ms / 1e9, "mfma_peak_frac": flops / ms / 1e9 / peak,
                   "torch_ms": ms_t, "torch_mfma_peak_frac": flops / ms_t / 1e9 / peak}
            if dt.startswith("c"):
                # the form the blocked solve's trailing updates take: A's panel as 2 x 2
                # real blocks (2M x 2K), B and C read as real matrices, the real product
                rdt = "f32" if dt == "c64" else "f64"
                E = torch.rand(2 * K, 2 * M, device="cuda", generator=g, dtype=tdt[rdt])
                Br, Cr = torch.view_as_real(Bm), torch.view_as_real(C)
                fr = hs.entry("gemm", rdt)
                ms_r = timed(lambda: hs.check(fr(2 * M, N, 2 * K, -1.0, E, 2 * M, Br, 2 * K, 1.0, Cr, 2 * M, 0,
                                                 stream), "gemm_" + rdt))
                row.update({"real_form_ms": ms_r, "real_form_mfma_peak_frac": flops / ms_r / 1e9 / peak})
                del E
            out["%s %dx%dx%d" % (dt, M, N, K)] = row
            del A, Bm, C
    return out


def counter_workload(hs, torch):
    """Three batched solves per dtype (4096 problems, m = n = 64), then a 1 GiB
    device-to-device copy whose byte counts calibrate the HBM counters."""
    for dt in DTYPES:
        A, B = batched_inputs(dt, 64, 64, 4096, SEED_CFG1)
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        f = hs.entry("strided_batched", dt)
        for _ in range(3):
            hs.check(f(64, 64, 1.0, dA, 64, 4096, dB, 64, 4096, 4096), "strided_batched_" + dt)
        torch.cuda.synchronize()
        del dA, dB
    x = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    log("counter workload done")


# HBM bytes per launch of the batched small kernel (4096 problems of 64 x 64),
# from rocprofv3 FETCH_SIZE x 2.00 + WRITE_SIZE x 1.00, the factors a 1 GiB
# device copy reads for the two counters (profiles/colane_batched64_hbm_traffic.md).
# Valid only for the kernel source they were taken on: keyed by the SHA-256 of
# small.hip.
MEASURED_TRAFFIC = {
    "8d6c08ba7b1e55286cf06bd036e3dd6e187fccd161610d579e13e7b3527799f8": {
        "f32": 185325440, "f64": 353134123, "c64": 357223467, "c128": 852528341},
}


def measured_traffic(dtype):
    import hashlib
    src = os.path.join(ROOT, "triangular_solve_amd", "csrc", "small.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()
    entry = MEASURED_TRAFFIC.get(h, {}).get(dtype)
    return entry


def cpu_baseline(host, m=64, n=64, min_seconds=10.0):
    """The CPU oracle (as it stands) on the same step's problems, all host threads it is given,
    repeated until about min_seconds of CPU work have been timed."""
    import oracle
    threads = oracle.default_threads()
    flops = 0
    reps = 0
    t0 = time.perf_counter()
    while True:
        for dt in DTYPES:
            A, B = host[dt]
            oracle.trsm(A[:, :, :m].transpose(0, 2, 1), B[:, :, :m].transpose(0, 2, 1), threads=threads)
            flops += lapack_flops(dt, m, n) * A.shape[0]
        reps += 1
        sec = time.perf_counter() - t0
        if sec >= min_seconds:
            break
    return {"value": flops / sec / 1e9, "unit": "GFLOPS", "cores": threads, "kind": "oracle",
            "sample": "the full step (4096 problems x 4 dtypes, m=n=64) %d times, plain C "
                      "double-precision forward substitution, %d threads on %s"
                      % (reps, threads, cpu_model()),
            "seconds": sec, "repeats": reps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="batched",
                    choices=["batched", "blocked", "counters", "medium", "gemm", "variants", "inversion"],
                    help="counters: only three batched solves per dtype and a 1 GiB copy, for "
                         "rocprofv3 --pmc runs; medium: strided batches of 1024 systems with "
                         "m = 128, n = 64; gemm: the library GEMM at trailing-update shapes")
    ap.add_argument("--m", type=int, default=8192, help="blocked workload size (m = n)")
    ap.add_argument("--dtypes", default="f32,f64,c64,c128")
    ap.add_argument("--nb", type=int, default=0, help="blocked N_B override (0: table)")
    ap.add_argument("--no-blocked", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the work shards by "
              "right-hand-side columns, see the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import triangular_solve_amd as hs
    torch.cuda.set_device(0)

    if args.workload == "counters":
        counter_workload(hs, torch)
        return
    if args.workload in ("medium", "gemm", "variants", "inversion"):
        fn = {"medium": medium_workload, "gemm": gemm_workload, "variants": bench_variants,
              "inversion": bench_inversion}[args.workload]
        print(json.dumps({"workload": args.workload, "results": fn(hs, torch)}), flush=True)
        return
    if args.workload == "blocked":
        dts = args.dtypes.split(",")
        res = bench_blocked(hs, torch, args.m, dts, runs=max(2, args.steps), nb=args.nb)
        tot_flops = sum(lapack_flops(dt, args.m, args.m) for dt in dts)
        tot_ms = sum(r["ms"] for r in res.values())
        dom = max(res, key=lambda d: res[d]["ms"])
        line = {"metric": METRIC, "value": tot_flops / tot_ms / 1e6, "unit": "GFLOPS", "n_gpus": 1,
                "steps": max(2, args.steps), "warmup": 1, "ms_per_step": tot_ms, "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": "+".join(dts), "data": "synthetic",
                "config": {"workload": "blocked trsm m=n=%d, one solve per dtype (%s), column-major, "
                                       "alpha=1, N_B from table" % (args.m, ",".join(dts)),
                           "m": args.m, "n": args.m},
                "roofline": {"bound": "mfma", "achieved": res[dom]["gflops"] / 1e3,
                             "peak": MFMA_PEAK_TFLOPS[dom], "unit": "TFLOP/s",
                             "frac": res[dom]["mfma_peak_frac"], "traffic": None,
                             "kernel": "whole blocked solve, %s (LAPACK flop count)" % dom},
                "blocked": res}
        print(json.dumps(line), flush=True)
        return

    log("batched small regime")
    bt = bench_batched(hs, torch, args.steps, args.warmup)
    per = bt["per_dtype"]
    dom = max(per, key=lambda d: per[d]["ms_per_launch"])
    log("batched launches of one dtype back to back")
    alone = bench_batched_alone(hs, torch, bt["host"])
    log("solve_tri shape")
    st = bench_solve_tri(hs, torch)
    log("solve_tri 128 shape")
    st128 = bench_solve_tri(hs, torch, runs=1000, n=128, k=8, e2=4, e3=1)
    st256 = bench_solve_tri(hs, torch, runs=1000, n=256, k=8, e2=4, e3=1)
    blocked = blocked16 = variants = inversion = few = None
    if not args.no_blocked:
        blocked = bench_blocked(hs, torch, 8192, DTYPES, runs=3)
        blocked16 = bench_blocked(hs, torch, 16384, ["f32", "f64", "c128"], runs=2)
        log("few right-hand sides")
        few = bench_few_rhs(hs, torch)
        variants = bench_variants(hs, torch)
        log("inversion routes")
        inversion = bench_inversion(hs, torch)
    cpu = None if args.no_cpu else cpu_baseline(bt["host"])
    line = {
        "metric": METRIC, "value": bt["gflops"], "unit": "GFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": bt["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32+f64+c64+c128", "data": "synthetic",
        "config": {"workload": "batched trsm, 4096 column-major problems of m=n=64 per dtype, "
                               "f32+f64+c64+c128 (one launch each), left/lower/no-trans/non-unit, alpha=1",
                   "m": 64, "n": 64, "batch": 4096},
        "roofline": {"bound": "hbm", "achieved": per[dom]["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": per[dom]["hbm_frac"], "traffic": measured_traffic(dom),
                     "kernel": "colane_kernel (%s), %d algorithmic bytes per launch" % (dom, per[dom]["bytes_per_launch"])},
        "cpu_baseline": cpu,
        "per_dtype": per,
        "per_dtype_alone": alone,
        "solve_tri": st, "solve_tri_128": st128, "solve_tri_256": st256,
        "blocked_8192": blocked,
        "blocked_16384": blocked16,
        "few_rhs_8192x64": few,
        "variants_8192": variants,
        "inversion_routes_ms": inversion,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
