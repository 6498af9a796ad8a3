"""Pins of the float64 oracle's forward and state update against results the
pages and the mathematics fix independently of the oracle's own code.

Pages (web pages about Gu & Dao, "Mamba: Linear-Time Sequence Modeling with
Selective State Spaces"):
  * chapterpal.com page, Knowl 1 (S6 layer: ZOH rule, recurrence) and Knowl 4
    (ZOH selective SSM with N=1, A=-1, B=1, softplus step equals the gated
    recurrence h_t = (1-g_t) h_{t-1} + g_t x_t with g_t = sigmoid(.));
    Knowl 4 also states the limits: large step resets, small step preserves;
  * trishampatil.com essay, Part II §4 "The same SSM is also a convolution"
    (h_0 = 0; time-invariant parameters give y = x * K with K_k = C A^k B)
    and Part III §2 (associative composition of affine pairs);
  * paper-graph-ui.vercel.app summary, section 3.4 (Theorem 1; channel
    independence; chunk boundary carry of the scan state).

Independent routines used: scipy.linalg.expm (matrix-exponential ZOH of the
augmented system [[A, B], [0, 0]]), scipy.special.expit (sigmoid),
numpy.logaddexp (softplus), brute-force O(L^2) convolution and a Blelloch
up-sweep/down-sweep tree scan written here.
"""
import numpy as np
import pytest
import scipy.linalg
from scipy.special import expit

import oracle
import workloads as W


def softplus_ref(r):
    return np.logaddexp(0.0, r)


def zoh_expm(dt, a_n, b_n):
    """(Abar, Bbar) for the scalar system h' = a h + b x held over dt, from the
    matrix exponential of the augmented matrix [[a, b], [0, 0]] * dt."""
    M = np.array([[a_n * dt, b_n * dt], [0.0, 0.0]])
    E = scipy.linalg.expm(M)
    return E[0, 0], E[0, 1]


def rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# Theorem 1: N=1, A=-1, B=1, softplus => gated RNN, exactly.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("with_bias", [False, True])
def test_theorem1_gated_rnn(with_bias):
    g = rng(1)
    batch, dim, L = 2, 3, 64
    x = g.standard_normal((batch, dim, L))
    w = g.standard_normal((batch, dim, L)) * 2.0
    bias = g.standard_normal(dim) if with_bias else None
    A = -np.ones((dim, 1))
    B = np.ones((batch, 1, L))
    C = np.ones((batch, 1, L))
    out, last = oracle.scan_fwd(x, w, A, B, C, None, None, bias, delta_softplus=True)
    # closed form
    wr = w + (bias[None, :, None] if with_bias else 0.0)
    gate = expit(wr)
    h = np.zeros((batch, dim))
    ref = np.zeros_like(x)
    for t in range(L):
        h = (1.0 - gate[..., t]) * h + gate[..., t] * x[..., t]
        ref[..., t] = h
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(last[..., 0], h, rtol=1e-12, atol=1e-13)


def test_softplus_off_uses_biased_step_directly():
    # N=1, A=-1, B=1: with a given positive step dt, ZOH gives
    # Abar = e^{-dt}, Bbar = 1 - e^{-dt} (matrix exponential below).
    g = rng(2)
    L = 40
    x = g.standard_normal((1, 2, L))
    dt_raw = g.uniform(0.01, 1.0, (1, 2, L))
    bias = np.array([0.05, 0.2])
    out, _ = oracle.scan_fwd(x, dt_raw, -np.ones((2, 1)), np.ones((1, 1, L)), np.ones((1, 1, L)),
                             None, None, bias, delta_softplus=False)
    h = np.zeros(2)
    for t in range(L):
        for d in range(2):
            ab, bb = zoh_expm(dt_raw[0, d, t] + bias[d], -1.0, 1.0)
            h[d] = ab * h[d] + bb * x[0, d, t]
        np.testing.assert_allclose(out[0, :, t], h, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# Time-invariant special case == brute-force convolution with K_k = C Abar^k Bbar
# --------------------------------------------------------------------------
@pytest.mark.parametrize("disc", [oracle.ZOH, oracle.EULER])
@pytest.mark.parametrize("softplus_on", [True, False])
def test_lti_equals_bruteforce_convolution(disc, softplus_on):
    g = rng(10 + disc * 2 + int(softplus_on))
    batch, dim, N, L = 2, 3, 5, 96
    A = -np.exp(g.standard_normal((dim, N)))
    x = g.standard_normal((batch, dim, L))
    # constant step per channel, constant B, C along t (per batch row)
    raw = g.standard_normal((batch, dim, 1)) * 0.5 + (0.0 if softplus_on else 1.0)
    raw = np.abs(raw) if not softplus_on else raw
    delta = np.repeat(raw, L, axis=2)
    Bc = g.standard_normal((batch, N, 1))
    Cc = g.standard_normal((batch, N, 1))
    B = np.repeat(Bc, L, axis=2)
    C = np.repeat(Cc, L, axis=2)
    Dv = g.standard_normal(dim)
    out, _ = oracle.scan_fwd(x, delta, A, B, C, Dv, None, None, delta_softplus=softplus_on,
                             disc=disc)
    ref = np.zeros_like(x)
    for b in range(batch):
        for d in range(dim):
            dt = softplus_ref(raw[b, d, 0]) if softplus_on else raw[b, d, 0]
            K = np.zeros(L)
            for n in range(N):
                ab, bb = zoh_expm(dt, A[d, n], Bc[b, n, 0])
                if disc == oracle.EULER:
                    bb = dt * Bc[b, n, 0]
                K += Cc[b, n, 0] * ab ** np.arange(L) * bb
            for t in range(L):
                ref[b, d, t] = np.dot(K[: t + 1], x[b, d, t::-1]) + Dv[d] * x[b, d, t]
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_zoh_limit_at_zero_A_is_cumulative_sum():
    # A = 0: Abar = 1, Bbar = dt*B (the limit of (e^{dt A}-1)/A), so h is a
    # running sum of dt*B*x.
    g = rng(3)
    L = 50
    x = g.standard_normal((1, 1, L))
    raw = g.standard_normal((1, 1, L))
    Bv = g.standard_normal((1, 1, L))
    out, _ = oracle.scan_fwd(x, raw, np.zeros((1, 1)), Bv, np.ones((1, 1, L)), None, None, None)
    dt = softplus_ref(raw)
    np.testing.assert_allclose(out, np.cumsum(dt * Bv * x, axis=2), rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# Reset / preserve limits of the step size
# --------------------------------------------------------------------------
@pytest.mark.parametrize("disc", [oracle.ZOH, oracle.EULER])
def test_large_step_resets_state(disc):
    g = rng(4)
    batch, dim, N, L, ts = 1, 4, 6, 48, 20
    inp = W.make_inputs(101, batch, dim, N, L)
    f = W.inputs_f64(inp, "f32")
    f1 = {k: v.copy() for k, v in f.items()}
    f2 = {k: v.copy() for k, v in f.items()}
    # different prefixes
    f2["u"][..., :ts] = g.standard_normal((batch, dim, ts))
    f2["delta"][..., :ts] = g.standard_normal((batch, dim, ts))
    for f_ in (f1, f2):
        f_["delta"][..., ts] = 60.0   # softplus(60 - 2) ~ 58: Abar ~ e^-58
    o1, _ = oracle.scan_fwd(f1["u"], f1["delta"], f1["A"], f1["B"], f1["C"], f1["D"], f1["z"],
                            f1["delta_bias"], disc=disc)
    o2, _ = oracle.scan_fwd(f2["u"], f2["delta"], f2["A"], f2["B"], f2["C"], f2["D"], f2["z"],
                            f2["delta_bias"], disc=disc)
    assert not np.allclose(o1[..., :ts], o2[..., :ts])
    np.testing.assert_allclose(o1[..., ts:], o2[..., ts:], rtol=1e-13, atol=1e-13)
    # right at the reset the state is Bbar*u only: y = sum_n C Bbar u + D u
    dt = softplus_ref(60.0 + f1["delta_bias"])
    for d in range(dim):
        y = 0.0
        for n in range(N):
            _, bb = zoh_expm(dt[d], f1["A"][d, n], f1["B"][0, n, ts])
            if disc == oracle.EULER:
                bb = dt[d] * f1["B"][0, n, ts]
            y += f1["C"][0, n, ts] * bb * f1["u"][0, d, ts]
        y += f1["D"][d] * f1["u"][0, d, ts]
        zt = f1["z"][0, d, ts]
        np.testing.assert_allclose(o1[0, d, ts], y * zt * expit(zt), rtol=1e-12)


@pytest.mark.parametrize("disc", [oracle.ZOH, oracle.EULER])
def test_zero_step_preserves_state(disc):
    # softplus off, raw step 0, bias 0: Abar = 1, Bbar = 0 exactly, so the
    # state stays h0 and y_t = C_t . h0 + D u_t.
    g = rng(5)
    batch, dim, N, L = 2, 3, 4, 30
    u = g.standard_normal((batch, dim, L))
    A = -np.exp(g.standard_normal((dim, N)))
    B = g.standard_normal((batch, N, L))
    C = g.standard_normal((batch, N, L))
    Dv = g.standard_normal(dim)
    h0 = g.standard_normal((batch, dim, N))
    out, last = oracle.scan_fwd(u, np.zeros_like(u), A, B, C, Dv, None, np.zeros(dim), h0,
                                delta_softplus=False, disc=disc)
    ref = np.einsum("bnt,bdn->bdt", C, h0) + Dv[None, :, None] * u
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(last, h0)


# --------------------------------------------------------------------------
# Associative operator: a Blelloch tree scan of (Abar, Bbar x) pairs gives the
# same states as the sequential oracle.
# --------------------------------------------------------------------------
def _compose(left, right):
    """Apply `left` then `right`: h -> a_r (a_l h + b_l) + b_r."""
    (al, bl), (ar, br) = left, right
    return (ar * al, ar * bl + br)


def blelloch_exclusive(pairs):
    n = len(pairs)
    size = 1
    while size < n:
        size *= 2
    tree = list(pairs) + [(1.0, 0.0)] * (size - n)
    step = 1
    while step < size:  # up-sweep
        for i in range(2 * step - 1, size, 2 * step):
            tree[i] = _compose(tree[i - step], tree[i])
        step *= 2
    tree[size - 1] = (1.0, 0.0)
    step = size // 2
    while step >= 1:  # down-sweep
        for i in range(2 * step - 1, size, 2 * step):
            left = tree[i - step]
            tree[i - step] = tree[i]
            tree[i] = _compose(tree[i], left)
        step //= 2
    return tree[:n]


@pytest.mark.parametrize("disc", [oracle.ZOH, oracle.EULER])
def test_tree_scan_matches_sequential(disc):
    g = rng(6)
    N, L = 3, 37
    A = -np.exp(g.standard_normal((1, N)))
    u = g.standard_normal((1, 1, L))
    raw = g.standard_normal((1, 1, L))
    B = g.standard_normal((1, N, L))
    dt = softplus_ref(raw[0, 0])
    for n in range(N):
        C = np.zeros((1, N, L))
        C[0, n, :] = 1.0   # read out h[n]
        out, last = oracle.scan_fwd(u, raw, A, B, C, None, None, None, disc=disc)
        pairs = []
        for t in range(L):
            ab, bb = zoh_expm(dt[t], A[0, n], B[0, n, t])
            if disc == oracle.EULER:
                bb = dt[t] * B[0, n, t]
            pairs.append((ab, bb * u[0, 0, t]))
        excl = blelloch_exclusive(pairs)
        incl = [_compose(excl[t], pairs[t])[1] for t in range(L)]
        np.testing.assert_allclose(out[0, 0], incl, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(last[0, 0, n], incl[-1], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# Chunk carry / resume, and the state update step
# --------------------------------------------------------------------------
@pytest.mark.parametrize("disc", [oracle.ZOH, oracle.EULER])
def test_split_and_resume(disc):
    inp = W.make_inputs(102, 2, 5, 4, 80, bias="normal")
    f = W.inputs_f64(inp, "f32")
    full, last_full = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                                      f["delta_bias"], disc=disc)
    k = 53
    sl = lambda a, s: None if a is None else a[..., s]
    _, last_k = oracle.scan_fwd(*(sl(f[n], slice(0, k)) for n in ("u", "delta")), f["A"],
                                *(sl(f[n], slice(0, k)) for n in ("B", "C")), f["D"],
                                sl(f["z"], slice(0, k)), f["delta_bias"], disc=disc)
    tail, last_tail = oracle.scan_fwd(*(sl(f[n], slice(k, None)) for n in ("u", "delta")), f["A"],
                                      *(sl(f[n], slice(k, None)) for n in ("B", "C")), f["D"],
                                      sl(f["z"], slice(k, None)), f["delta_bias"], last_k,
                                      disc=disc)
    np.testing.assert_allclose(tail, full[..., k:], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(last_tail, last_full, rtol=1e-13, atol=1e-13)
    # continue with single recurrent steps from the split point
    st = last_k
    for t in range(k, 80):
        y, st = oracle.state_update(st, f["u"][..., t], f["delta"][..., t], f["A"],
                                    f["B"][..., t], f["C"][..., t], f["D"], f["z"][..., t],
                                    f["delta_bias"], disc=disc)
        np.testing.assert_allclose(y, full[..., t], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(st, last_full, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Structure: linearity in u, separability over the state index, C = 0
# --------------------------------------------------------------------------
def test_linear_in_u():
    g = rng(7)
    inp = W.inputs_f64(W.make_inputs(103, 2, 3, 4, 40), "f32")
    u1, u2 = g.standard_normal((2,) + inp["u"].shape)
    args = lambda u: (u, inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], None,
                      inp["delta_bias"])
    o1, _ = oracle.scan_fwd(*args(u1))
    o2, _ = oracle.scan_fwd(*args(u2))
    o3, _ = oracle.scan_fwd(*args(2.5 * u1 - 0.75 * u2))
    np.testing.assert_allclose(o3, 2.5 * o1 - 0.75 * o2, rtol=1e-11, atol=1e-12)


def test_state_dimensions_are_separable():
    inp = W.inputs_f64(W.make_inputs(104, 2, 3, 5, 40, A_mode="random_neg"), "f32")
    full, _ = oracle.scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], None, None,
                              inp["delta_bias"])
    acc = np.zeros_like(full)
    for n in range(5):
        o, _ = oracle.scan_fwd(inp["u"], inp["delta"], inp["A"][:, n:n + 1],
                               inp["B"][:, n:n + 1], inp["C"][:, n:n + 1], None, None,
                               inp["delta_bias"])
        acc += o
    np.testing.assert_allclose(full, acc, rtol=1e-12, atol=1e-13)
    # channels are independent: running one channel alone gives its row
    one, _ = oracle.scan_fwd(inp["u"][:, 1:2], inp["delta"][:, 1:2], inp["A"][1:2], inp["B"],
                             inp["C"], None, None, inp["delta_bias"][1:2])
    np.testing.assert_array_equal(one[:, 0], full[:, 1])


def test_zero_C_gives_gated_skip():
    inp = W.inputs_f64(W.make_inputs(105, 2, 3, 4, 40), "f32")
    out, _ = oracle.scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], np.zeros_like(inp["C"]),
                             inp["D"], inp["z"], inp["delta_bias"])
    z = inp["z"]
    np.testing.assert_allclose(out, inp["D"][None, :, None] * inp["u"] * z * expit(z),
                               rtol=1e-14, atol=1e-15)


def test_workload1_shapes_and_determinism():
    inp = W.workload_inputs(1)
    assert inp["u"].shape == (1, 16, 128) and inp["B"].shape == (1, 4, 128)
    np.testing.assert_array_equal(inp["A"][3], [-1, -2, -3, -4])
    assert np.all(inp["delta_bias"] == -2.0)
    again = W.workload_inputs(1)
    for k in inp:
        np.testing.assert_array_equal(inp[k], again[k])
    f = W.inputs_f64(inp, "f32")
    o1, l1 = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                             f["delta_bias"], threads=1)
    o2, l2 = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                             f["delta_bias"], threads=5)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_per_row_generation_subset_matches_full():
    full = W.make_inputs(4, 1, 6, 4, 64, dtype="bf16", per_row=True)
    sub = W.make_inputs(4, 1, 6, 4, 64, dtype="bf16", per_row=True, dim_subset=[1, 4])
    for k in ("u", "delta", "z"):
        np.testing.assert_array_equal(sub[k], full[k][:, [1, 4]])
    for k in ("B", "C"):
        np.testing.assert_array_equal(sub[k], full[k])
    np.testing.assert_array_equal(sub["A"], full["A"][[1, 4]])


def test_bf16_rounding_is_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e-3],
                 np.float32)
    back = W.bf16_bits_to_f32(W.bf16_round_bits(x))
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa (1.0) wins;
    # 1+3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even (1+2^-6) wins.
    np.testing.assert_array_equal(back[:4], [1.0, 1.0, 1.0 + 2 ** -6, 1.0])
    assert back[4] == -2.5
    assert abs(back[5] - 3.0e-3) <= 3.0e-3 * 2 ** -8


# ---------------------------------------------------------------------------
# Packed variable-length sequences: a reset flag zeroes the state before its
# step, so the packed run must equal independent runs of each segment (the
# first segment keeps the initial state unless it is itself reset).
# ---------------------------------------------------------------------------
def _segments(row):
    starts = [0] + [t for t in range(1, row.size) if row[t]]
    return list(zip(starts, starts[1:] + [row.size]))


def _packed_inputs(seed, batch=2, dim=3, N=4, L=40):
    g = np.random.default_rng(seed)
    p = dict(u=g.standard_normal((batch, dim, L)), delta=g.standard_normal((batch, dim, L)),
             A=-np.exp(g.standard_normal((dim, N))), B=g.standard_normal((batch, N, L)),
             C=g.standard_normal((batch, N, L)), D=g.standard_normal(dim),
             z=g.standard_normal((batch, dim, L)), delta_bias=g.standard_normal(dim) - 1.0,
             h0=g.standard_normal((batch, dim, N)))
    reset = np.zeros((batch, L), np.uint8)
    reset[0, [0, 7, 8, 30]] = 1          # reset at t = 0, two adjacent flags
    reset[1, [13, L - 1]] = 1            # a one-step final segment
    return p, reset, g.standard_normal((batch, dim, L))


def _slice(p, b, s, e):
    q = {}
    for k, v in p.items():
        if k in ("u", "delta", "z", "B", "C"):
            q[k] = v[b:b + 1, :, s:e]
        elif k == "h0":
            q[k] = v[b:b + 1]
        else:
            q[k] = v
    return q


@pytest.mark.parametrize("disc", [oracle.ZOH, oracle.EULER])
def test_reset_forward_equals_independent_segments(disc):
    p, reset, _ = _packed_inputs(5)
    out, last = oracle.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                                p["delta_bias"], p["h0"], disc=disc, reset=reset)
    for b in range(reset.shape[0]):
        for i, (s, e) in enumerate(_segments(reset[b])):
            q = _slice(p, b, s, e)
            h0 = q["h0"] if (i == 0 and not reset[b, 0]) else None
            o, l = oracle.scan_fwd(q["u"], q["delta"], q["A"], q["B"], q["C"], q["D"], q["z"],
                                   q["delta_bias"], h0, disc=disc)
            np.testing.assert_array_equal(out[b, :, s:e], o[0])
        np.testing.assert_array_equal(last[b], l[0])


@pytest.mark.parametrize("disc", [oracle.ZOH, oracle.EULER])
def test_reset_backward_equals_independent_segments(disc):
    p, reset, dout = _packed_inputs(6)
    g = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                        p["delta_bias"], dout, p["h0"], disc=disc, reset=reset)
    sums = dict(dA=0.0, dD=0.0, ddelta_bias=0.0)
    for b in range(reset.shape[0]):
        for i, (s, e) in enumerate(_segments(reset[b])):
            q = _slice(p, b, s, e)
            first = i == 0 and not reset[b, 0]
            gs = oracle.scan_bwd(q["u"], q["delta"], q["A"], q["B"], q["C"], q["D"], q["z"],
                                 q["delta_bias"], dout[b:b + 1, :, s:e],
                                 q["h0"] if first else None, disc=disc)
            for k in ("du", "ddelta", "dz"):
                np.testing.assert_array_equal(g[k][b, :, s:e], gs[k][0], err_msg=k)
            for k in ("dB", "dC"):
                np.testing.assert_allclose(g[k][b, :, s:e], gs[k][0], rtol=1e-12, atol=1e-13)
            for k in sums:
                sums[k] = sums[k] + gs[k]
            if i == 0:
                want = gs["dh0"][0] if first else np.zeros_like(g["dh0"][b])
                np.testing.assert_array_equal(g["dh0"][b], want)
    for k, v in sums.items():
        np.testing.assert_allclose(g[k], v, rtol=1e-12, atol=1e-12, err_msg=k)


def test_oracle_rejects_missing_or_misshaped_arguments():
    # the C code reads through the pointers with the documented sizes: a
    # missing required array or a wrong shape is refused before the call
    inp = W.make_inputs(62, 1, 4, 8, 64, dtype="f32", with_dout=True)
    f = W.inputs_f64(inp, "f32")
    args = [f[k] for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")]
    with pytest.raises(ValueError, match="dout is required"):
        oracle.scan_bwd(*args, None)
    with pytest.raises(ValueError, match="h0 has shape"):
        oracle.scan_fwd(*args, f["dout"])            # (batch, dim, L) where h0 goes
    with pytest.raises(ValueError, match="B has shape"):
        oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"][:, :4], f["C"])
    ci = W.make_complex_inputs(62, 1, 4, 8, 64, dtype="f32", with_dout=True)
    cargs = [ci[k] for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")]
    with pytest.raises(ValueError, match="dout is required"):
        oracle.scan_bwd_complex(*cargs, None)
