"""Pins of the layer oracle (out = x + W_out . mixer(W_in . RMSNorm(x))), CPU only.

- W_out = 0 gives out = x exactly (the residual path alone).
- out - x is linear in W_out.
- Batch rows are independent.
- With x_proj_w = 0 the mixer's B and C are RMSNorm(0) = 0, so from zero states the SSM adds
  nothing and y = D u SiLU(z): the whole layer is then evaluated in mpmath at 50 digits from
  the definitions (RMSNorm equation, the two projections, the causal conv, SiLU), with no code
  shared with the oracle.
- round_bf16 (the bf16 activation storage of act_round="bf16"): hand-worked values and ties, and
  torch's float32 -> bfloat16 conversion on float32 inputs (a single rounding there); the rounded
  layer applies it at exactly the three stored activations (W_in = I and a D-only mixer make
  each one visible).
"""
import mpmath
import numpy as np
import torch

import oracle
import synth

CFG = synth.MixerConfig("layer_tiny", 2, 7, 8, 16, 3, 8, "f32", d_model=6)


def _setup(seed=5, zero_xproj=False):
    p = synth.make_params(CFG, seed, conv_bias=True, gamma_random=True)
    if zero_xproj:
        p["x_proj_w"] = p["x_proj_w"] * 0
    lay = synth.make_layer(CFG, seed, gamma_random=True)
    x = synth.make_layer_x(CFG, seed)
    p64 = oracle.as_f64_params(p)
    lay64 = {k: v.double().numpy() for k, v in lay.items()}
    return x.double().numpy(), p64, lay64


def test_zero_out_proj_is_identity():
    x, p, lay = _setup()
    lay["out_proj_w"] = np.zeros_like(lay["out_proj_w"])
    out, _, _ = oracle.layer_prefill(x, p, lay)
    assert np.array_equal(out, x)


def test_linear_in_out_proj():
    x, p, lay = _setup()
    rng = np.random.default_rng(3)
    w1 = rng.standard_normal(lay["out_proj_w"].shape)
    w2 = rng.standard_normal(lay["out_proj_w"].shape)
    res = []
    for w in (w1, w2, 2.0 * w1 - 0.5 * w2):
        out, _, _ = oracle.layer_prefill(x, p, dict(lay, out_proj_w=w))
        res.append(out - x)
    np.testing.assert_allclose(res[2], 2.0 * res[0] - 0.5 * res[1], rtol=1e-12, atol=1e-12)


def test_batch_rows_independent():
    x, p, lay = _setup()
    both, _, _ = oracle.layer_prefill(x, p, lay)
    for b in range(x.shape[0]):
        one, _, _ = oracle.layer_prefill(x[b:b + 1], p, lay)
        np.testing.assert_allclose(one[0], both[b], rtol=1e-13, atol=1e-13)


def _mp_layer_without_ssm(x, p, lay, eps=1e-6, norm_eps=1e-6):
    mpmath.mp.dps = 50
    B, L, Dm = x.shape
    D, K = p["conv_w"].shape
    out = np.zeros_like(x)
    sig = lambda v: 1 / (1 + mpmath.exp(-v))  # noqa: E731
    for b in range(B):
        xn = []
        for t in range(L):
            row = [mpmath.mpf(float(v)) for v in x[b, t]]
            r = mpmath.sqrt(sum(v * v for v in row) / Dm + mpmath.mpf(norm_eps))
            xn.append([row[j] / r * mpmath.mpf(float(lay["norm_w"][j])) for j in range(Dm)])
        xz = [[sum(xn[t][j] * mpmath.mpf(float(lay["in_proj_w"][c, j])) for j in range(Dm))
               for c in range(2 * D)] for t in range(L)]
        y = []
        for t in range(L):
            yt = []
            for i in range(D):
                acc = mpmath.mpf(float(p["conv_b"][i]))
                for k in range(K):
                    s = t - (K - 1) + k
                    if s >= 0:
                        acc += mpmath.mpf(float(p["conv_w"][i, k])) * xz[s][i]
                u = acc * sig(acc)
                z = xz[t][D + i]
                yt.append(mpmath.mpf(float(p["Dskip"][i])) * u * z * sig(z))
            y.append(yt)
        for t in range(L):
            for m in range(Dm):
                v = mpmath.mpf(float(x[b, t, m])) + sum(
                    mpmath.mpf(float(lay["out_proj_w"][m, i])) * y[t][i] for i in range(D))
                out[b, t, m] = float(v)
    return out


def test_layer_without_ssm_contribution_matches_mpmath():
    x, p, lay = _setup(seed=9, zero_xproj=True)
    p["Dskip"] = np.linspace(0.5, 1.5, p["Dskip"].shape[0])
    out, _, ss = oracle.layer_prefill(x, p, lay)
    ref = _mp_layer_without_ssm(x, p, lay)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert np.all(ss == 0)


def test_round_bf16_hand_worked():
    u = 2.0 ** -7                                   # bf16 spacing on [1, 2)
    vals = [1.0, 1 + u / 2, 1 + 3 * u / 2, 1 + u / 2 + 2 ** -30, -(1 + 3 * u / 2), 3.0 + 2 ** -9,
            0.0, 2.0 ** -100 * (1 + u / 2)]
    want = [1.0, 1.0, 1 + 2 * u, 1 + u, -(1 + 2 * u), 3.0, 0.0, 2.0 ** -100]
    np.testing.assert_array_equal(oracle.round_bf16(np.array(vals)), np.array(want))


def test_round_bf16_matches_torch_on_float32():
    rng = np.random.default_rng(11)
    a = (rng.standard_normal(200000) * np.exp2(rng.integers(-20, 20, 200000))).astype(np.float32)
    ref = torch.from_numpy(a).bfloat16().double().numpy()
    np.testing.assert_array_equal(oracle.round_bf16(a.astype(np.float64)), ref)
    r = oracle.round_bf16(a.astype(np.float64))
    np.testing.assert_array_equal(oracle.round_bf16(r), r)


def test_rounded_layer_rounds_the_three_activations():
    # d_model = 8 = d_inner with W_in = [I; I]: xz = (xn, xn); x_proj_w = 0 and conv = identity
    # tap make y = D u SiLU(z); W_out = I makes out - x = rounded y. Each stage's rounding shows.
    cfg = synth.MixerConfig("layer_round", 1, 5, 8, 16, 2, 8, "f32", d_model=8)
    p = oracle.as_f64_params(synth.make_params(cfg, 4))
    p["x_proj_w"] = p["x_proj_w"] * 0
    p["conv_w"] = np.zeros_like(p["conv_w"]); p["conv_w"][:, -1] = 1.0
    p["conv_b"] = np.zeros_like(p["conv_w"][:, 0])
    p["Dskip"] = np.full(8, 1.0 / 3.0)
    lay = {"norm_w": np.full(8, 1.1), "in_proj_w": np.vstack([np.eye(8), np.eye(8)]),
           "out_proj_w": np.eye(8)}
    x = np.random.default_rng(2).standard_normal((1, 5, 8))
    out, _, _ = oracle.layer_prefill(x, p, lay, act_round="bf16")
    r = oracle.round_bf16
    silu = lambda v: v / (1 + np.exp(-v))  # noqa: E731
    xn = r(x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-6) * 1.1)
    y = r(silu(xn) * silu(xn) / 3.0)
    np.testing.assert_allclose(out - x, y, rtol=0, atol=1e-15)
    exact, _, _ = oracle.layer_prefill(x, p, lay)
    assert np.max(np.abs(exact - out)) > 1e-5          # the rounding is really applied
