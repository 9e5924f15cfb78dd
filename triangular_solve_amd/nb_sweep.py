"""Offline sweep of the blocked path's outer block size N_B (inner I_B = N_B/8).

The HSMA-TRSM paper's adaptive blocking section builds its "size x dtype ->
optimal block" table in a pre-build phase: every candidate block size is run
at a set of problem sizes and only the fastest is kept. This script does the
same on the current GPU for problem shapes (m, n) -- the order of A and the
number of right-hand sides, since few and many right-hand sides favour
different blocks -- and prints (or writes) csrc/nb_table.inc; the library then
picks N_B by the nearest tested shape at run time.

    python -m triangular_solve_amd.nb_sweep [--sizes 1024,2048,...] [--rhs 64,512,4096,m] [--write]

Inputs are random well-conditioned lower-triangular systems drawn on the GPU
(timing does not depend on the values); each (size, dtype, N_B) is timed as
the mean of `--reps` solves after one warm-up, with B restored between solves.
"""
import argparse
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
DTYPES = ["f32", "f64", "c64", "c128"]
CANDIDATES = [64, 128, 256, 512, 1024, 2048]


def shapes_of(sizes, rhs):
    """(m, n) pairs: every size with every right-hand-side count ("m" = square)."""
    out = []
    for m in sizes:
        for r in rhs:
            n = m if r == "m" else int(r)
            if (m, n) not in out:
                out.append((m, n))
    return out


def sweep(shapes, dtypes, reps, log=print):
    import torch
    import triangular_solve_amd as hs
    tdt = {"f32": torch.float32, "f64": torch.float64, "c64": torch.complex64, "c128": torch.complex128}
    results = {}
    stream = torch.cuda.current_stream()
    for dt in dtypes:
        for m in sorted({m for m, _ in shapes}):
            g = torch.Generator(device="cuda").manual_seed(m)
            A = torch.rand(m, m, device="cuda", generator=g, dtype=tdt[dt]) * (2.0 / m) - 1.0 / m
            A.diagonal().add_(1.5)
            A = A.t().contiguous()          # column-major storage of the lower triangle
            for (mm, nn) in shapes:
                if mm != m:
                    continue
                B0 = torch.rand(nn, m, device="cuda", generator=g, dtype=tdt[dt])
                B = B0.clone()
                best = None
                for nb in CANDIDATES:
                    if nb > 2 * m or (nb > (512 if dt == "c128" else 1024) and m % nb != 0):
                        continue
                    times = []
                    for r in range(reps + 1):
                        B.copy_(B0)
                        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        a.record(stream)
                        st = hs.entry("ex", dt)(m, nn, 1.0, A, m, B, m, {"nb": nb, "path": hs.PATH_BLOCKED},
                                                stream)
                        b.record(stream)
                        torch.cuda.synchronize()
                        if st != hs.SUCCESS:
                            raise hs.HsmaError(st, "sweep")
                        times.append(a.elapsed_time(b))
                    ms = sum(times[1:]) / reps
                    flops = (4 if dt.startswith("c") else 1) * m * m * nn
                    results[(dt, m, nn, nb)] = ms
                    log("%s m=%d n=%d nb=%d ms=%.3f GFLOPS=%.0f" % (dt, m, nn, nb, ms, flops / ms / 1e6))
                    if best is None or ms < best[1]:
                        best = (nb, ms)
                results[(dt, m, nn, "best")] = best[0]
                del B, B0
            del A
            torch.cuda.empty_cache()
    return results


def table_text(results, shapes, dtypes):
    names = {"f32": "kNbF32", "f64": "kNbF64", "c64": "kNbC64", "c128": "kNbC128"}
    out = ["// nb_table.inc - outer block size N_B of the blocked path, per dtype, at the",
           "// tested problem shapes {m, n} (order of A, right-hand sides): the \"scale x",
           "// data type -> optimal block\" table of the HSMA-TRSM paper's adaptive",
           "// blocking section, over (m, n). Written by nb_sweep.py from timings on",
           "// MI355X; a shape between entries takes the nearest entry by distance",
           "// |log2 m - log2 m_i| + |log2 n - log2 n_i|."]
    for dt in DTYPES:
        if dt in dtypes:
            ent = ", ".join("{%d, %d, %d}" % (m, n, results[(dt, m, n, "best")]) for m, n in shapes)
        else:
            ent = "{1024, 1024, 256}, {8192, 8192, 512}"
        out.append("static const NbEntry %s[] = {%s};" % (names[dt], ent))
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--sizes", default="1024,2048,4096,8192,16384")
    ap.add_argument("--rhs", default="64,512,4096,m", help="right-hand-side counts; m = square")
    ap.add_argument("--dtypes", default=",".join(DTYPES))
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--write", action="store_true", help="write csrc/nb_table.inc")
    args = ap.parse_args()
    sizes = [int(x) for x in args.sizes.split(",")]
    shapes = shapes_of(sizes, args.rhs.split(","))
    dtypes = args.dtypes.split(",")
    res = sweep(shapes, dtypes, args.reps, log=lambda s: print(s, flush=True))
    text = table_text(res, shapes, dtypes)
    print(text)
    if args.write:
        with open(os.path.join(HERE, "csrc", "nb_table.inc"), "w") as f:
            f.write(text)


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(HERE))
    main()
