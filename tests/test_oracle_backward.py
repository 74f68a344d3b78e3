"""Pins of the backward oracle (oracle/mixer_bwd_f64.py), CPU only.

Every gradient is checked against central finite differences of the (separately pinned) forward
oracle: for a random direction V of one tensor, (l(theta + e V) - l(theta - e V)) / 2e must equal
<grad, V>, with l = sum(dy * y) in fp64 (e = 1e-5; the truncation and rounding errors are ~1e-10
relative). One direction per tensor, so a wrong term anywhere in that tensor's gradient shows.
Cases: first-order and ZOH Bbar, zero and carried states, with a conv bias and random RMSNorm
gains, and checkpoint blocks shorter than the sequence with a ragged last block.
"""
import numpy as np
import pytest

import oracle
import synth

CFG = synth.MixerConfig("bwd_tiny", 2, 11, 6, 3, 4, 2, "f32")
TENSORS = ["conv_w", "conv_b", "x_proj_w", "dt_proj_w", "dt_proj_b", "A", "Dskip", "dt_norm_w",
           "B_norm_w", "C_norm_w"]


def _setup(seed, states):
    p = oracle.as_f64_params(synth.make_params(CFG, seed, conv_bias=True, gamma_random=True))
    rng = np.random.default_rng(seed)
    # A spread over a wider range than -(n+1) so that dt A covers small and large magnitudes
    p["A"] = -np.exp(rng.uniform(-2.0, 1.5, p["A"].shape))
    p["Dskip"] = rng.uniform(0.5, 1.5, p["Dskip"].shape)
    xz = synth.make_xz(CFG, seed).double().numpy()
    cs = ss = None
    if states:
        cs, ss = (t.double().numpy() for t in synth.make_states(CFG, seed))
    dy = rng.standard_normal((CFG.batch, CFG.seqlen, CFG.d_inner))
    return p, xz, cs, ss, dy


def _loss(p, xz, cs, ss, dy, zoh):
    y, _, _ = oracle.mixer_prefill(xz, p, cs, ss, zoh=zoh)
    return float(np.sum(dy * y))


def _fd(fun, base, V, e=1e-5):
    return (fun(base + e * V) - fun(base - e * V)) / (2 * e)


@pytest.mark.parametrize("zoh", [False, True])
@pytest.mark.parametrize("states", [False, True])
def test_gradients_match_central_differences(zoh, states):
    p, xz, cs, ss, dy = _setup(31 + 2 * zoh + states, states)
    g = oracle.mixer_prefill_backward(xz, p, dy, cs, ss, zoh=zoh, ckpt=4)
    rng = np.random.default_rng(7)
    checks = [(name, p[name]) for name in TENSORS] + [("xz", xz)]
    if states:
        checks += [("conv_state0", cs), ("ssm_state0", ss)]
    for name, base in checks:
        V = rng.standard_normal(base.shape)

        def fun(v, name=name):
            if name in p:
                return _loss(dict(p, **{name: v}), xz, cs, ss, dy, zoh)
            if name == "xz":
                return _loss(p, v, cs, ss, dy, zoh)
            if name == "conv_state0":
                return _loss(p, xz, v, ss, dy, zoh)
            return _loss(p, xz, cs, v, dy, zoh)

        fd = _fd(fun, base, V)
        an = float(np.sum(g[name] * V))
        assert abs(fd - an) <= 1e-7 * max(abs(fd), 1.0), f"{name}: fd {fd!r} vs analytic {an!r}"


def test_zero_states_have_gradients_too():
    # the gradient of the carried states exists (and is what a chunked training step passes
    # back) even when the forward starts from zeros
    p, xz, _, _, dy = _setup(40, False)
    g0 = oracle.mixer_prefill_backward(xz, p, dy)
    zc = np.zeros((CFG.batch, CFG.d_inner, CFG.d_conv - 1))
    zs = np.zeros((CFG.batch, CFG.d_inner, CFG.d_state))
    g1 = oracle.mixer_prefill_backward(xz, p, dy, zc, zs)
    for k in g0:
        if g0[k] is not None:
            np.testing.assert_allclose(g0[k], g1[k], rtol=1e-13, atol=1e-13)
    assert np.any(g0["ssm_state0"] != 0) and np.any(g0["conv_state0"] != 0)


def test_checkpoint_length_changes_nothing():
    p, xz, cs, ss, dy = _setup(41, True)
    ga = oracle.mixer_prefill_backward(xz, p, dy, cs, ss, ckpt=3)
    gb = oracle.mixer_prefill_backward(xz, p, dy, cs, ss, ckpt=64)
    for k in ga:
        if ga[k] is not None:
            np.testing.assert_allclose(ga[k], gb[k], rtol=1e-12, atol=1e-13)


def test_linear_in_dy():
    p, xz, cs, ss, dy = _setup(42, True)
    dy2 = np.random.default_rng(1).standard_normal(dy.shape)
    g1 = oracle.mixer_prefill_backward(xz, p, dy, cs, ss)
    g2 = oracle.mixer_prefill_backward(xz, p, dy2, cs, ss)
    g3 = oracle.mixer_prefill_backward(xz, p, 2 * dy - 3 * dy2, cs, ss)
    for k in g1:
        if g1[k] is not None:
            np.testing.assert_allclose(g3[k], 2 * g1[k] - 3 * g2[k], rtol=1e-10, atol=1e-11)
