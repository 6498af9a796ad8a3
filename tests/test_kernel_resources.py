"""Resources of the built kernels (CPU only: read from the library's gfx950
code objects).  The backward kernels form their per-thread addresses in every
chunk instead of keeping them across the state-index loop: kept, they were
spilled, and each reload waited for the atomics, stores and prefetch loads in
flight (and added a third to the backward's HBM traffic).  These tests keep
the backward variants' scratch under recorded caps and within the register
budget of three waves per SIMD."""
import os
import re

import pytest

from kernel_resources import kernel_resources

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "scan_selective_fwd_amd", "libmamba_scan.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


@pytest.fixture(scope="module")
def res():
    r = kernel_resources(LIB)
    assert r, "no gfx950 kernel metadata found in the library"
    return r


# scan_bwd_kernel<T, NT, ZOH, VEC, TINY, RST>: T = float (f) or bf16 (t, uint16)
REAL_BWD = re.compile(r"^_ZN5mscan15scan_bwd_kernelI([ft])Li(16|64)ELb([01])ELb([01])"
                      r"ELb([01])ELb([01])EEEvNS_9BwdParamsE$")
# scan_bwd_complex_kernel<T, ZOH, VEC, RST>
CPLX_BWD = re.compile(r"^_ZN5mscan12_GLOBAL__N_123scan_bwd_complex_kernelI([ft])Lb([01])"
                      r"ELb([01])ELb([01])EEEvNS_13CplxBwdParamsE$")


# Scratch caps (bytes per lane).  The Euler backward has none.  The ZOH
# backward forms the ZOH coefficient and its A-derivative without
# cancellation (a cubic expm1 bound, the psi series and closed form), whose
# temporaries spill a few dwords per lane outside the state loop; the caps
# keep that from growing unnoticed.
BWD_ZOH_SCRATCH_CAP = {"16": 112, "64": 96}


def test_real_backward_main_variants_scratch(res):
    main = {n: (m, v) for n, v in res.items()
            if (m := REAL_BWD.match(n)) and m.group(5) == "0" and m.group(6) == "0"}
    # {f32, bf16} x {N <= 16, N <= 64} x {ZOH, Euler} x {vector, guarded loads}
    assert len(main) == 16, sorted(main)
    over = {n: v for n, (m, v) in main.items()
            if v["scratch"] > (BWD_ZOH_SCRATCH_CAP[m.group(2)] if m.group(3) == "1" else 0)}
    assert not over, over


def test_real_backward_keeps_three_waves_per_simd(res):
    real = {n: v for n, v in res.items() if REAL_BWD.match(n)}
    assert len(real) == 64, len(real)
    over = {n: v for n, v in real.items() if v["vgpr"] > 168}
    assert not over, over


def test_complex_backward_scratch(res):
    # Euler: none; ZOH: the complex psi of the A-derivative spills (cap)
    cplx = {n: (m, v) for n, v in res.items() if (m := CPLX_BWD.match(n))}
    assert len(cplx) == 16, sorted(cplx)
    over = {n: v for n, (m, v) in cplx.items()
            if v["scratch"] > (200 if m.group(2) == "1" else 0)}
    assert not over, over
