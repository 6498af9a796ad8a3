"""mamba_scan_bwd_noalloc (the backward without a workspace argument, its
buffers in the library's fixed per-GPU scratch array) against mamba_scan_bwd
on the same inputs, through the C ABI: two calls in a row, the second with a
smaller input, each compared per row at the float32 bound (and with the
oracle).  The first call splits its long sequence into segments, so the
segment buffers live in the scratch array too."""
import numpy as np
import pytest
import torch

import oracle
import scan_selective_fwd_amd as ms
import workloads as W
from parity_utils import RTOL_F32, announce, assert_match, to_device, to_f64

pytestmark = pytest.mark.gpu

CASES = [  # (wid, batch, dim, N, L, dtype, disc): larger first, then smaller
    (111, 2, 520, 16, 4096, "bf16", "zoh"),
    (112, 1, 40, 16, 1000, "f32", "euler"),
]


def test_noalloc_matches_bwd_two_calls_second_smaller():
    for wid, batch, dim, N, L, dtype, disc in CASES:
        announce(f"noalloc bwd wid={wid} ({batch},{dim},{N},{L}) {dtype} {disc}")
        inp = W.make_inputs(wid, batch, dim, N, L, dtype=dtype, bias="uniform", with_dout=True)
        g = to_device(inp, dtype)
        h0 = torch.from_numpy(np.random.default_rng(wid).standard_normal(
            (batch, dim, N)).astype(np.float32)).cuda()
        args = (g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"],
                g["dout"], h0)
        got = ms.scan_bwd_noalloc(*args, disc=disc)
        ref = ms.scan_bwd(*args, disc=disc)
        torch.cuda.synchronize()
        assert set(got) == set(ref)
        for k in ref:
            assert_match(to_f64(got[k]), to_f64(ref[k]), RTOL_F32, k + " noalloc vs bwd")
        f = W.inputs_f64(inp, dtype)
        oref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                               f["delta_bias"], f["dout"], to_f64(h0),
                               disc=oracle.ZOH if disc == "zoh" else oracle.EULER)
        for k in oref:
            assert_match(to_f64(got[k]), oref[k], RTOL_F32, k + " noalloc vs oracle")
