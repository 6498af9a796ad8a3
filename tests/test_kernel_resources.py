"""Resources of the built kernels (CPU only: read from the library's gfx950
code objects).  The backward kernels form their per-thread addresses in every
chunk instead of keeping them across the state-index loop: kept, they were
spilled, and each reload waited for the atomics, stores and prefetch loads in
flight (and added a third to the backward's HBM traffic).  These tests keep
the scan kernels' scratch under recorded caps and within the register budget
of three waves per SIMD."""
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


# scan_bwd_kernel<T, NT, ZOH, VEC, TINY, RST, NW>: T = float (f) or bf16 (t,
# uint16); NW = 4 or 12 waves per block
REAL_BWD = re.compile(r"^_ZN5mscan15scan_bwd_kernelI([ft])Li(16|64)ELb([01])ELb([01])"
                      r"ELb([01])ELb([01])ELi(4|12)EEEvNS_9BwdParamsE$")
# scan_fwd_kernel<T, R, K, NT, ZOH, VEC, MODE, RST, EXACT, SEG>
REAL_FWD = re.compile(r"^_ZN5mscan15scan_fwd_kernelI([ft])Li(16|32|64)ELi(\d+)ELi(16|64)"
                      r"ELb([01])ELb([01])ELi([012])ELb([01])ELb([01])ELi([012])EEEv"
                      r"NS_9FwdParamsE$")
# scan_bwd_complex_kernel<T, ZOH, VEC, RST>
CPLX_BWD = re.compile(r"^_ZN5mscan12_GLOBAL__N_123scan_bwd_complex_kernelI([ft])Lb([01])"
                      r"ELb([01])ELb([01])EEEvNS_13CplxBwdParamsE$")


# Scratch caps (bytes per lane).  The Euler backward has none.  The ZOH
# backward forms the ZOH coefficient and its A-derivative without
# cancellation (a cubic expm1 bound, the psi series and closed form), whose
# temporaries spill a few dwords per lane outside the chunk loop (N <= 16)
# or outside the state loop (N <= 64, 64 carried states per channel); the
# caps keep that from growing unnoticed.
BWD_ZOH_SCRATCH_CAP = {"16": 32, "64": 104}


def test_real_backward_main_variants_scratch(res):
    main = {n: (m, v) for n, v in res.items()
            if (m := REAL_BWD.match(n)) and m.group(5) == "0" and m.group(6) == "0"}
    # {f32, bf16} x {N <= 16, N <= 64} x {ZOH, Euler} x {vector, guarded loads}
    # in 4-wave blocks, and the N <= 16 ones in 12-wave blocks too
    assert len(main) == 24, sorted(main)
    over = {n: v for n, (m, v) in main.items()
            if v["scratch"] > (BWD_ZOH_SCRATCH_CAP[m.group(2)] if m.group(3) == "1" else 0)}
    assert not over, over


def test_real_backward_keeps_three_waves_per_simd(res):
    real = {n: v for n, v in res.items() if REAL_BWD.match(n)}
    assert len(real) == 80, len(real)
    over = {n: v for n, v in real.items() if v["vgpr"] > 168}
    assert not over, over


def test_complex_backward_scratch(res):
    # Euler: none; ZOH: the complex psi of the A-derivative spills (cap)
    cplx = {n: (m, v) for n, v in res.items() if (m := CPLX_BWD.match(n))}
    assert len(cplx) == 16, sorted(cplx)
    over = {n: v for n, (m, v) in cplx.items()
            if v["scratch"] > (200 if m.group(2) == "1" else 0)}
    assert not over, over


# Forward scratch caps (bytes per lane).  The spills sit outside the chunk
# loop of the usual case (the copy for blocks with A ~ 0 or A > 0, the set-up,
# the N <= 64 variant's 64 carried states); the caps keep them from growing
# unnoticed.
FWD_SCRATCH_CAP = 360
FWD_HOT_SCRATCH_CAP = 256   # 16 lanes per channel, N = 16, outputs, no reset flags


def test_forward_kernels_scratch_and_registers(res):
    fwd = {n: (m, v) for n, v in res.items() if (m := REAL_FWD.match(n))}
    # lanes {16, 32, 64}: {f32, bf16} x {ZOH, Euler} x {vector, guarded} x modes x
    # variants; the count guards against the regex silently matching nothing
    assert len(fwd) >= 300, len(fwd)
    assert not {n: v for n, (m, v) in fwd.items() if v["vgpr"] > 168}
    assert not {n: v for n, (m, v) in fwd.items() if v["scratch"] > FWD_SCRATCH_CAP}
    hot = {n: v for n, (m, v) in fwd.items()
           if m.group(2) == "16" and m.group(4) == "16" and m.group(7) == "0"
           and m.group(8) == "0" and m.group(9) == "1"}
    assert len(hot) == 24, sorted(hot)   # {f32, bf16} x {ZOH, Euler} x {vec, guarded} x 3 SEG
    assert not {n: v for n, v in hot.items() if v["scratch"] > FWD_HOT_SCRATCH_CAP}
