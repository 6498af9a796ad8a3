"""GPU parity of the short causal convolution + SiLU (forward and backward)
against the float64 oracle on identical seeded inputs: tap counts 1..4,
float32 and bfloat16, with and without bias, packed sequences (reset flags
at t = 0, at thread-run and block borders), ragged and tiny lengths."""
import numpy as np
import pytest
import torch

import oracle
import scan_selective_fwd_amd as ms
import workloads as W
from parity_utils import RTOL, announce, assert_match, to_f64

pytestmark = pytest.mark.gpu


def _case(seed, batch, dim, L, width, dtype, with_b=True, reset=None):
    announce(f"conv seed={seed} shape=({batch},{dim},{L}) W={width} {dtype} bias={with_b} "
             f"resets={None if reset is None else int(reset.sum())}")
    inp = W.make_inputs(seed, batch, dim, 1, L, dtype=dtype, with_dout=True)
    g = np.random.default_rng([seed, 10])
    w = (g.standard_normal((dim, width)) * 0.5).astype(np.float32)
    b = (g.standard_normal(dim) * 0.5).astype(np.float32) if with_b else None
    x_bits = inp["u"]                                     # the seeded x, in its dtype
    x64 = W.as_f64(x_bits, dtype)
    du = W.as_f64(inp["dout"], dtype).astype(np.float32)   # a float32 gradient
    if dtype == "bf16":
        xt = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(
            torch.bfloat16).cuda()
    else:
        xt = torch.from_numpy(np.ascontiguousarray(x_bits)).cuda()
    wt = torch.from_numpy(w).cuda()
    bt = torch.from_numpy(b).cuda() if b is not None else None
    rt = torch.from_numpy(reset).cuda() if reset is not None else None
    u = ms.conv1d_silu_fwd(xt, wt, bt, reset=rt)
    grads = ms.conv1d_silu_bwd(xt, wt, bt, torch.from_numpy(du).cuda(), reset=rt)
    torch.cuda.synchronize()
    ref_u = oracle.conv1d_silu_fwd(x64, w, b, reset=reset)
    ref_g = oracle.conv1d_silu_bwd(x64, w, b, du.astype(np.float64), reset=reset)
    rtol = RTOL[dtype]
    assert_match(to_f64(u), ref_u, rtol, "u")
    # the backward computes in float32 from exact inputs: float32 tolerance
    assert_match(to_f64(grads["dx"]), ref_g["dx"], RTOL["f32"], "dx")
    assert_match(to_f64(grads["dw"]), ref_g["dw"], RTOL["f32"], "dw")
    if b is not None:
        assert_match(to_f64(grads["db"]), ref_g["dcb"], RTOL["f32"], "db")
    else:
        assert "db" not in grads


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("width", [4, 3, 1])
def test_conv_widths_dtypes(dtype, width):
    # 4100 steps: two full 2048-step blocks and a ragged third
    _case(60, 2, 37, 4100, width, dtype)


@pytest.mark.parametrize("L", [1, 2, 5, 8, 2047, 2048, 2049])
def test_conv_lengths(L):
    _case(61, 1, 5, L, 4, "f32", with_b=False)
    _case(61, 1, 5, L, 4, "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_packed_sequences(dtype):
    L = 4100
    rs = W.make_resets(62, 2, L, 1, 300, force=(0, 7, 8, 9, 2047, 2048, 2050, L - 1))
    rs[1, 0] = 0
    _case(62, 2, 9, L, 4, dtype, reset=rs)
    _case(63, 2, 9, L, 2, dtype, with_b=False, reset=rs)


def test_conv_over_2e31_elements_sampled_channels():
    # batch 1, D 2064, 2^20 steps: 2.16e9 elements per tensor (64-bit offsets
    # and about a million blocks); sampled channels against the oracle, with
    # packed-sequence flags
    seed, batch, dim, L, width = 94, 1, 2064, 1 << 20, 4
    announce(f"conv over 2^31 elements: bf16 ({batch},{dim},{L}) W={width} sampled channels")
    inp = W.make_inputs(seed, batch, dim, 1, L, dtype="bf16", per_row=True, with_dout=True,
                        with_D=False, with_z=False, with_bias=False)
    g = np.random.default_rng([seed, 10])
    w = (g.standard_normal((dim, width)) * 0.5).astype(np.float32)
    b = (g.standard_normal(dim) * 0.5).astype(np.float32)
    reset = W.make_resets(seed, batch, L, 1000, 300000, force=(0, 2048 * 300))
    xt = torch.from_numpy(np.ascontiguousarray(inp["u"]).view(np.int16)).view(
        torch.bfloat16).cuda()
    dut = torch.from_numpy(np.ascontiguousarray(inp["dout"]).view(np.int16)).view(
        torch.bfloat16).cuda().float()               # bf16 values, exact in float32
    wt, bt, rt = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda(), torch.from_numpy(reset).cuda()
    u = ms.conv1d_silu_fwd(xt, wt, bt, reset=rt)
    grads = ms.conv1d_silu_bwd(xt, wt, bt, dut, reset=rt)
    torch.cuda.synchronize()
    chans = [0, 1031, 2063]
    got_u = to_f64(u[:, chans])
    got = {k: to_f64(grads[k][:, chans]) for k in ("dx",)}
    got.update({k: to_f64(grads[k][chans]) for k in ("dw", "db")})
    del xt, dut, u, grads
    x64 = W.as_f64(inp["u"][:, chans], "bf16")
    du64 = W.as_f64(inp["dout"][:, chans], "bf16")
    ref_u = oracle.conv1d_silu_fwd(x64, w[chans], b[chans], reset=reset)
    ref_g = oracle.conv1d_silu_bwd(x64, w[chans], b[chans], du64, reset=reset)
    assert_match(got_u, ref_u, RTOL["bf16"], "u")
    assert_match(got["dx"], ref_g["dx"], RTOL["f32"], "dx")
    assert_match(got["dw"], ref_g["dw"], RTOL["f32"], "dw")
    assert_match(got["db"], ref_g["dcb"], RTOL["f32"], "db")
