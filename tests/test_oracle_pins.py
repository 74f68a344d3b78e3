"""CPU pins of the fp64 oracle against things other than itself.

Each test names what fixes the expected value: a 50-digit mpmath evaluation, a
library routine (numpy.convolve, scipy.signal.lfilter, scipy ODE integration), a
closed form, an invariant, or the mpmath fixture in tests/golden/. Together they are
chosen so that a dropped term, a wrong sign, a shifted index or a transposed
operand anywhere in the oracle fails at least one of them.
"""
import json
import math
import os

import mpmath as mp
import numpy as np
import pytest
from scipy import integrate, signal

import oracle

mp.mp.dps = 50
HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------------------- scalar functions
@pytest.mark.parametrize("v", [-800.0, -60.0, -20.0, -3.5, -1e-3, 0.0, 1e-8, 0.7, 5.0, 33.0, 700.0])
def test_silu_matches_mpmath(v):
    ref = mp.mpf(v) / (1 + mp.exp(-mp.mpf(v)))
    got = float(oracle.silu(np.array([v]))[0])
    assert abs(got - float(ref)) <= 1e-15 * max(1.0, abs(float(ref))) + 1e-300


@pytest.mark.parametrize("v", [-800.0, -40.0, -7.0, -1.0, 0.0, 1e-9, 2.5, 19.0, 31.0, 750.0])
def test_softplus_matches_mpmath(v):
    ref = mp.log(1 + mp.exp(mp.mpf(v)))
    got = float(oracle.softplus(np.array([v]))[0])
    assert abs(got - float(ref)) <= 2e-16 * abs(float(ref)) + 1e-320


def test_rmsnorm_matches_mpmath():
    rng = np.random.default_rng(5)
    v = rng.normal(size=17) * 3.0
    g = rng.uniform(0.5, 1.5, size=17)
    eps = 1e-6
    ms = mp.fsum(mp.mpf(float(e)) ** 2 for e in v) / len(v)
    den = mp.sqrt(ms + mp.mpf(eps))
    ref = [float(mp.mpf(float(e)) / den * mp.mpf(float(gg))) for e, gg in zip(v, g)]
    got = oracle.rmsnorm(v, g, eps)
    np.testing.assert_allclose(got, ref, rtol=1e-15, atol=0)


def test_rmsnorm_constant_vector_and_scale_invariance():
    c, eps = 0.37, 1e-6
    got = oracle.rmsnorm(np.full(8, c), np.full(8, 2.0), eps)
    np.testing.assert_allclose(got, 2.0 * c / math.sqrt(c * c + eps), rtol=1e-15)
    v = np.random.default_rng(1).normal(size=(3, 32))
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * v, 1.0, 0.0), oracle.rmsnorm(v, 1.0, 0.0),
                               rtol=1e-14)
    # RMSNorm of the zero vector is zero (eps > 0 keeps it finite)
    assert np.all(oracle.rmsnorm(np.zeros(5), 1.0, 1e-6) == 0.0)


# ----------------------------------------------------------------------------- convolution
def test_conv_matches_numpy_convolve():
    rng = np.random.default_rng(2)
    L, D, K = 37, 5, 4
    x = rng.normal(size=(L, D))
    w = rng.uniform(-0.5, 0.5, size=(D, K))
    b = rng.uniform(-0.5, 0.5, size=D)
    st = rng.normal(size=(D, K - 1))
    u, _ = oracle.causal_conv1d_silu(x, w, b, st)
    u0, _ = oracle.causal_conv1d_silu(x, w, None, None)
    for i in range(D):
        # correlation with tap K-1 on the current token == convolution with the reversed kernel
        full = np.convolve(np.concatenate([st[i], x[:, i]]), w[i, ::-1])
        pre = full[K - 1:K - 1 + L] + b[i]
        np.testing.assert_allclose(u[:, i], pre / (1 + np.exp(-pre)), rtol=1e-13, atol=1e-15)
        pre0 = np.convolve(x[:, i], w[i, ::-1])[:L]
        np.testing.assert_allclose(u0[:, i], pre0 / (1 + np.exp(-pre0)), rtol=1e-13, atol=1e-15)


def test_conv_identity_tap_is_silu():
    x = np.random.default_rng(3).normal(size=(20, 6))
    w = np.zeros((6, 4))
    w[:, 3] = 1.0
    u, st = oracle.causal_conv1d_silu(x, w)
    np.testing.assert_allclose(u, x / (1 + np.exp(-x)), rtol=1e-15)
    np.testing.assert_array_equal(st, x[-3:].T)


def test_conv_state_continuity_and_short_sequences():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(11, 3))
    w = rng.normal(size=(3, 4))
    st0 = rng.normal(size=(3, 3))
    u, st = oracle.causal_conv1d_silu(x, w, None, st0)
    for split in (1, 2, 5, 10):
        ua, sa = oracle.causal_conv1d_silu(x[:split], w, None, st0)
        ub, sb = oracle.causal_conv1d_silu(x[split:], w, None, sa)
        np.testing.assert_array_equal(np.concatenate([ua, ub]), u)
        np.testing.assert_array_equal(sb, st)
    # L < K-1: the new state keeps the tail of the old one, oldest first
    _, s1 = oracle.causal_conv1d_silu(x[:1], w, None, st0)
    np.testing.assert_array_equal(s1, np.concatenate([st0[:, 1:], x[:1].T], axis=1))


# ----------------------------------------------------------------------------- projections
def test_projections_match_bruteforce_sums():
    rng = np.random.default_rng(6)
    T, D, R, N = 4, 7, 3, 2
    u = rng.normal(size=(T, D))
    wx = rng.normal(size=(R + 2 * N, D))
    got = oracle.x_proj(u, wx)
    for t in range(T):
        for r in range(R + 2 * N):
            assert abs(got[t, r] - math.fsum(wx[r, i] * u[t, i] for i in range(D))) < 1e-14
    a, bb, c = oracle.split_xdbl(got, R, N)
    np.testing.assert_array_equal(a, got[:, :R])
    np.testing.assert_array_equal(bb, got[:, R:R + N])
    np.testing.assert_array_equal(c, got[:, R + N:])
    wdt = rng.normal(size=(5, R))
    bias = rng.normal(size=5)
    dt = oracle.dt_proj_softplus(a, wdt, bias)
    for t in range(T):
        for i in range(5):
            pre = math.fsum(wdt[i, r] * a[t, r] for r in range(R)) + bias[i]
            assert abs(dt[t, i] - math.log1p(math.exp(pre))) < 1e-14


# ----------------------------------------------------------------------------- scan
def _scan_inputs(rng, L, D, N):
    u = rng.normal(size=(L, D))
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(0.5), size=(L, D)))
    A = -rng.uniform(0.5, 4.0, size=(D, N))
    Bm = rng.normal(size=(L, N))
    Cm = rng.normal(size=(L, N))
    Dskip = rng.normal(size=D)
    z = rng.normal(size=(L, D))
    h0 = rng.normal(size=(D, N))
    return u, dt, A, Bm, Cm, Dskip, z, h0


@pytest.mark.parametrize("zoh", [False, True])
def test_scan_matches_unrolled_cumulative_formula(zoh):
    """mpmath, 50 digits: h_t = e^{A S(1,t)} h0 + sum_s e^{A S(s+1,t)} Bbar_s u_s."""
    rng = np.random.default_rng(7)
    L, D, N = 9, 3, 4
    u, dt, A, Bm, Cm, Dskip, z, h0 = _scan_inputs(rng, L, D, N)
    y, hL = oracle.selective_scan(u, dt, A, Bm, Cm, Dskip, z, h0, zoh=zoh)
    M = lambda v: mp.mpf(float(v))  # noqa: E731
    for i in range(D):
        for t in range(L):
            hs = []
            for n in range(N):
                a = M(A[i, n])
                acc = mp.exp(a * mp.fsum(M(dt[r, i]) for r in range(t + 1))) * M(h0[i, n])
                for s in range(t + 1):
                    S = mp.fsum(M(dt[r, i]) for r in range(s + 1, t + 1))
                    bbar = ((mp.exp(M(dt[s, i]) * a) - 1) / a if zoh else M(dt[s, i])) * M(Bm[s, n])
                    acc += mp.exp(a * S) * bbar * M(u[s, i])
                hs.append(acc)
            yref = (mp.fsum(M(Cm[t, n]) * hs[n] for n in range(N)) + M(Dskip[i]) * M(u[t, i])) \
                * M(z[t, i]) / (1 + mp.exp(-M(z[t, i])))
            assert abs(y[t, i] - float(yref)) <= 1e-13 * (1 + abs(float(yref)))
            if t == L - 1:
                for n in range(N):
                    assert abs(hL[i, n] - float(hs[n])) <= 1e-13 * (1 + abs(float(hs[n])))


def test_scan_first_order_matches_lfilter():
    """N = 1, constant dt, B, C: h is a first-order IIR filter of u (scipy.signal.lfilter)."""
    rng = np.random.default_rng(8)
    L = 200
    u = rng.normal(size=(L, 1))
    dtv, a, bv, cv, dv = 0.05, -1.7, 0.8, -1.3, 0.4
    z = rng.normal(size=(L, 1))
    y, hL = oracle.selective_scan(u, np.full((L, 1), dtv), np.array([[a]]), np.full((L, 1), bv),
                                  np.full((L, 1), cv), np.array([dv]), z)
    q = math.exp(dtv * a)
    h = signal.lfilter([dtv * bv], [1.0, -q], u[:, 0])
    yref = (cv * h + dv * u[:, 0]) * z[:, 0] / (1 + np.exp(-z[:, 0]))
    np.testing.assert_allclose(y[:, 0], yref, rtol=1e-11, atol=1e-13)
    assert abs(hL[0, 0] - h[-1]) < 1e-12


@pytest.mark.parametrize("zoh", [False, True])
def test_scan_zoh_is_exact_for_piecewise_constant_input(zoh):
    """The page's ZOH Bbar is the exact solution of dx/dt = A x + B u over a step with u, B held
    constant (scipy ODE integration); the first-order Bbar = dt*B is not, and differs from it by
    a factor expm1(dt A)/(dt A) that tends to 1 as dt -> 0."""
    rng = np.random.default_rng(9)
    L, N = 12, 3
    A = -np.array([[0.7, 1.9, 3.2]])
    dt = rng.uniform(0.05, 0.6, size=(L, 1))
    u = rng.normal(size=(L, 1))
    Bm = rng.normal(size=(L, N))
    h0 = rng.normal(size=(1, N))
    hs = [h0[0].copy()]
    x = h0[0].copy()
    for t in range(L):
        sol = integrate.solve_ivp(lambda _, s: A[0] * s + Bm[t] * u[t, 0], (0.0, dt[t, 0]), x,
                                  rtol=1e-12, atol=1e-14, method="DOP853")
        x = sol.y[:, -1]
        hs.append(x.copy())
    ones = np.ones((L, 1))
    _, h_zoh = oracle.selective_scan(u, dt, A, Bm, np.zeros((L, N)), np.zeros(1), ones * 50.0,
                                     h0, zoh=True)
    np.testing.assert_allclose(h_zoh[0], hs[-1], rtol=1e-9, atol=1e-11)
    if not zoh:
        # first-order input matrix: tends to ZOH as dt -> 0
        small = dt * 1e-4
        _, he = oracle.selective_scan(u, small, A, Bm, np.zeros((L, N)), np.zeros(1), ones,
                                      h0 * 0, zoh=False)
        _, hz = oracle.selective_scan(u, small, A, Bm, np.zeros((L, N)), np.zeros(1), ones,
                                      h0 * 0, zoh=True)
        np.testing.assert_allclose(he, hz, rtol=1e-3)


def test_scan_linear_in_u_and_memoryless_limit():
    rng = np.random.default_rng(10)
    L, D, N = 30, 4, 5
    u, dt, A, Bm, Cm, Dskip, z, _ = _scan_inputs(rng, L, D, N)
    u2 = rng.normal(size=(L, D))
    y1, h1 = oracle.selective_scan(u, dt, A, Bm, Cm, Dskip, z)
    y2, h2 = oracle.selective_scan(u2, dt, A, Bm, Cm, Dskip, z)
    y12, h12 = oracle.selective_scan(u + 3.0 * u2, dt, A, Bm, Cm, Dskip, z)
    np.testing.assert_allclose(y12, y1 + 3.0 * y2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h12, h1 + 3.0 * h2, rtol=1e-12, atol=1e-12)
    # exp(dt A) underflows to 0: the state forgets everything, h_t = dt_t B_t u_t
    yA, hA = oracle.selective_scan(u, dt, np.full((D, N), -1e6), Bm, Cm, Dskip, z)
    g = z / (1 + np.exp(-z))
    yref = ((dt * u) * (Bm * Cm).sum(axis=1)[:, None] + Dskip * u) * g
    np.testing.assert_allclose(yA, yref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hA, (dt[-1] * u[-1])[:, None] * Bm[-1][None, :], rtol=1e-12)


# ----------------------------------------------------------------------------- whole mixer
def _mixer_case(seed, B=2, L=40, D=8, N=4, K=4, R=3, conv_bias=True):
    rng = np.random.default_rng(seed)
    p = dict(conv_w=rng.uniform(-0.5, 0.5, (D, K)),
             conv_b=rng.uniform(-0.5, 0.5, D) if conv_bias else None,
             x_proj_w=rng.normal(size=(R + 2 * N, D)) / math.sqrt(D),
             dt_proj_w=rng.normal(size=(D, R)) / math.sqrt(R),
             dt_proj_b=rng.uniform(-6, -2, D),
             A=-np.tile(np.arange(1, N + 1, dtype=float), (D, 1)),
             Dskip=np.ones(D), dt_norm_w=rng.uniform(0.5, 1.5, R),
             B_norm_w=rng.uniform(0.5, 1.5, N), C_norm_w=rng.uniform(0.5, 1.5, N))
    xz = rng.normal(size=(B, L, 2 * D))
    cs = rng.normal(size=(B, D, K - 1))
    ss = rng.normal(size=(B, D, N))
    return p, xz, cs, ss


def test_zero_input_closed_form():
    """x = 0 and no conv bias: u = 0, B = C = RMSNorm(0) = 0, dt = softplus(bias) for every
    token, so h_L = exp(L dt A) h_0 and y = 0."""
    p, xz, _, ss = _mixer_case(11, conv_bias=False)
    xz[..., :xz.shape[-1] // 2] = 0.0
    L = xz.shape[1]
    y, _, hL = oracle.mixer_prefill(xz, p, None, ss)
    dt = np.log1p(np.exp(p["dt_proj_b"]))
    ref = np.exp(L * dt[:, None] * p["A"])[None] * ss
    np.testing.assert_allclose(hL, ref, rtol=1e-12, atol=1e-300)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("zoh", [False, True])
def test_chunked_equals_sequential(zoh):
    """Associativity of the scan (the page's parallel-scan operator) lets the sequence be cut
    anywhere and resumed from the carried conv and SSM states."""
    p, xz, cs, ss = _mixer_case(12)
    y, c1, s1 = oracle.mixer_prefill(xz, p, cs, ss, zoh=zoh)
    for cuts in ([1], [3], [17, 18], [2, 9, 33, 39]):
        ys, c, s = [], cs, ss
        for a, b in zip([0] + cuts, cuts + [xz.shape[1]]):
            yy, c, s = oracle.mixer_prefill(xz[:, a:b], p, c, s, zoh=zoh)
            ys.append(yy)
        np.testing.assert_allclose(np.concatenate(ys, axis=1), y, rtol=1e-12, atol=1e-14)
        np.testing.assert_array_equal(c, c1)
        np.testing.assert_allclose(s, s1, rtol=1e-12, atol=1e-14)


def test_prefill_equals_repeated_decode_steps():
    p, xz, cs, ss = _mixer_case(13, L=25)
    y, c1, s1 = oracle.mixer_prefill(xz, p, cs, ss)
    c, s = cs, ss
    for t in range(xz.shape[1]):
        yt, c, s = oracle.mixer_decode_step(xz[:, t], p, c, s)
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(c, c1)
    np.testing.assert_allclose(s, s1, rtol=1e-12, atol=1e-14)


def test_batch_independence_channel_subset_and_token_blocks():
    p, xz, cs, ss = _mixer_case(14, B=3)
    y, c, s = oracle.mixer_prefill(xz, p, cs, ss)
    for b in range(3):
        yb, cb, sb = oracle.mixer_prefill(xz[b:b + 1], p, cs[b:b + 1], ss[b:b + 1])
        np.testing.assert_allclose(yb[0], y[b], rtol=1e-13, atol=1e-15)
        np.testing.assert_array_equal(cb[0], c[b])
    sel = np.array([6, 1, 3])
    ysel, csel, ssel = oracle.mixer_prefill(xz, p, cs, ss, channels=sel, token_block=7)
    np.testing.assert_allclose(ysel, y[:, :, sel], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ssel, s[:, sel], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(csel, c)
    # independent token blocks on a thread pool, including blocks shorter than K-1
    for tb in (1, 2, 5):
        for st in ((cs, ss), (None, None)):
            r0 = oracle.mixer_prefill(xz, p, *st)
            r1 = oracle.mixer_prefill(xz, p, *st, token_block=tb, workers=4)
            np.testing.assert_allclose(r1[0], r0[0], rtol=1e-12, atol=1e-14)
            np.testing.assert_array_equal(r1[1], r0[1])
            np.testing.assert_allclose(r1[2], r0[2], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("mode", ["euler", "zoh"])
def test_whole_mixer_matches_mpmath_fixture(mode):
    with open(os.path.join(HERE, "golden", "tiny_mixer_mpmath.json")) as f:
        g = json.load(f)
    arr = lambda v: np.array(v, dtype=float) if not isinstance(v, str) else float(v)  # noqa: E731
    inp = {k: np.vectorize(float)(np.array(v, dtype=object)) for k, v in g["inputs"].items()}
    p = {k: inp[k] for k in ("conv_w", "conv_b", "x_proj_w", "dt_proj_w", "dt_proj_b", "A",
                             "Dskip", "dt_norm_w", "B_norm_w", "C_norm_w")}
    xz = np.concatenate([inp["x"], inp["z"]], axis=1)[None]
    y, cs, ss = oracle.mixer_prefill(xz, p, inp["conv_state0"][None], inp["ssm_state0"][None],
                                     eps=float(g["shape"]["eps"]), zoh=(mode == "zoh"))
    exp = g[mode]
    np.testing.assert_allclose(y[0], np.vectorize(float)(np.array(exp["y"], dtype=object)),
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(cs[0], np.vectorize(float)(np.array(exp["conv_state"], dtype=object)))
    np.testing.assert_allclose(ss[0], np.vectorize(float)(np.array(exp["ssm_state"], dtype=object)),
                               rtol=1e-12, atol=1e-14)
    del arr
