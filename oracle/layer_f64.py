"""fp64 oracle of the Mamba layer around the mixer -- TEST INFRASTRUCTURE, not product code.

    out = x + W_out . mixer(W_in . RMSNorm(x))

[Jamba] "RMSNorm definition and placement": RMSNorm at the input of every Mamba module (RMSNorm
equation). "From scalar SSM to vector processing", steps 1 and 4: the hidden state is projected
linearly to the d_inner scalar SSMs, and their concatenated outputs are projected back. The
residual add around the module is the pre-norm block the architecture description implies (a
reading; the pages do not write it out). numpy's matmul is the library primitive for the two
projections; the mixer is mixer_f64.mixer_prefill.

act_round="bf16" models a layer whose activations live in bf16 between its three operations
(the normalised input, the projected x|z and the mixer output y are each stored as bf16, then
read back): each is rounded to the nearest bf16 value, ties to even, and the arithmetic stays in
fp64. That is a reading of a bf16 layer's storage, not a step the pages spell out; the output
itself is not rounded. With act_round=None every step is exact fp64.
"""
from __future__ import annotations

import numpy as np

from .mixer_f64 import mixer_prefill, rmsnorm


def round_bf16(a):
    """Nearest bf16 value (8 significant bits, ties to even, the float32 exponent range) of each
    element, returned as float64. a = m 2^e with 0.5 <= |m| < 1; m 2^8 is rounded to an integer
    with ties to even (numpy's rint) and scaled back. Values here are far from the bf16
    underflow and overflow thresholds, which this does not model."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def layer_prefill(x, p, layer, conv_state0=None, ssm_state0=None, eps=1e-6, norm_eps=1e-6,
                  zoh=False, act_round=None):
    """x: [B, L, d_model]; p: mixer parameters (float64 numpy, as_f64_params); layer: norm_w
    [d_model], in_proj_w [2 d_inner, d_model] (rows: x then z), out_proj_w [d_model, d_inner].
    Returns (out [B, L, d_model], conv_state, ssm_state) as mixer_prefill returns the states."""
    x = np.asarray(x, dtype=np.float64)
    w_in = np.asarray(layer["in_proj_w"], dtype=np.float64)
    w_out = np.asarray(layer["out_proj_w"], dtype=np.float64)
    if act_round not in (None, "bf16"):
        raise ValueError(act_round)
    rnd = round_bf16 if act_round == "bf16" else (lambda a: a)
    xn = rnd(rmsnorm(x, layer["norm_w"], norm_eps))     # over d_model
    xz = rnd(xn @ w_in.T)                                # [B, L, 2 d_inner]
    y, cs, ss = mixer_prefill(xz, p, conv_state0, ssm_state0, eps=eps, zoh=zoh)
    return x + rnd(y) @ w_out.T, cs, ss
