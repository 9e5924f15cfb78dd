"""Build libhsma_trsm.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhsma_trsm.so")
SOURCES = ["api.cpp", "small.hip", "blocked.hip", "medium.hip", "noalloc.hip", "variants.hip"]
ARCH = os.environ.get("HSMA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # no packed-FP32 instructions are generated (v_pk_* f32 forms are avoided)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wall", "-Wno-unused-function",
]


def _deps_mtime():
    """Newest modification time of the headers every source includes."""
    hdrs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hpp", ".inc"))]
    hdrs.append(os.path.join(ROOT, "include", "hsma_trsm.h"))
    return max(os.path.getmtime(h) for h in hdrs)


def _compile(src, incremental=False):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if incremental and os.path.exists(obj):
        newest = max(os.path.getmtime(os.path.join(CSRC, src)), _deps_mtime())
        if os.path.getmtime(obj) > newest:
            return obj, []
    # the compiler's per-kernel resource remarks (registers, scratch,
    # occupancy) go to <object>.resources.txt next to the object
    cmd = ["hipcc"] + FLAGS + ["-Rpass-analysis=kernel-resource-usage", "-x", "hip", "-c",
                               os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr[-8000:]))
    remarks = [l for l in r.stderr.splitlines() if "kernel-resource-usage" in l]
    with open(obj + ".resources.txt", "w") as f:
        f.write("\n".join(remarks) + "\n")
    warn = [l for l in r.stderr.splitlines()
            if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l and l.strip()]
    return obj, warn


def kernel_resources():
    """{kernel symbol: {"VGPRs", "AGPRs", "ScratchSize" (bytes per lane),
    "Occupancy" (waves per SIMD), "VGPRsSpill", "SGPRsSpill": int}}
    from the remarks of the last build of every source."""
    out = {}
    for src in SOURCES:
        path = os.path.join(BUILD, os.path.basename(src) + ".o.resources.txt")
        if not os.path.exists(path):
            continue
        cur = None
        for line in open(path):
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                cur = out.setdefault(m.group(1), {})
                continue
            m = re.search(r"remark: \s*(VGPRs Spill|SGPRs Spill|VGPRs|AGPRs|ScratchSize|Occupancy)"
                          r"(?: \[[^]]*\])?: (\d+)", line)
            if m and cur is not None:
                cur[m.group(1).replace(" ", "")] = int(m.group(2))
    return out


def build(verbose=False, incremental=False):
    """Compile every source (incremental: only those older than their
    source or a shared header) and link the library in-tree."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda f: _compile(f, incremental), SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, w in results:
            for l in w:
                print(l, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr[-8000:])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv))
