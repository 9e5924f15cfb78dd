"""Register and scratch use of every kernel in the built library, from the
compiler's resource remarks that the build records: no kernel may keep
values in scratch memory (spills, or register arrays the compiler could not
promote), whose per-lane traffic goes to HBM."""
import os

import pytest

from triangular_solve_amd import build as hb


def resources():
    res = hb.kernel_resources()
    if not res:
        pytest.skip("library built without resource remarks")
    return res


def test_no_kernel_uses_scratch():
    # (SGPR spills are allowed: they go to lanes of a VGPR, not to memory)
    bad = {k: v for k, v in resources().items()
           if v.get("ScratchSize", 0) or v.get("VGPRsSpill", 0)}
    assert not bad, "kernels with scratch use: %s" % sorted(bad)


def test_every_kernel_reported_and_resident():
    res = resources()
    names = " ".join(res)
    for kernel in ("rowlane_kernel", "colane_kernel", "gemm_kernel", "diag_inv_kernel",
                   "fused_inv_kernel", "tile_copy_kernel", "solve_tri_128_kernel", "solve_tri_256_kernel",
                   "reduce_kernel"):
        assert kernel in names, kernel
    for k, v in res.items():
        assert v.get("Occupancy", 0) >= 1, k
        assert v.get("VGPRs", 0) <= 512, k


def test_remarks_files_match_sources():
    for src in hb.SOURCES:
        obj = os.path.join(hb.BUILD, os.path.basename(src) + ".o")
        if os.path.exists(obj) and not os.path.exists(obj + ".resources.txt"):
            pytest.skip("objects from a build without resource remarks")
