"""GPU parity of the layer entry point (mamba_layer_prefill: out = x + W_out . mixer(W_in .
RMSNorm(x))) against the fp64 layer oracle, through the C ABI.

A bf16 layer stores its normalised input, the in_proj output x|z and the mixer output y as bf16
between its operations. Those roundings are part of what it computes: rounding x|z alone moves
the mixer output by up to 6e-2 (mixed relative) from the exact-activation result, since x feeds
B, C and dt through x_proj. So the parity reference is the oracle with act_round="bf16" (fp64
arithmetic, the three stored activations rounded to nearest bf16); the distance to the
exact-activation oracle is printed alongside.

The layer output `out` and the final SSM and conv states (the latter the last rows of the
in_proj output, rounded once on each side) are held to 2e-2 with the floor of the relative bar at rms(ref) rather than the mixer's 0.01 rms: where
the GPU's value of a stored bf16 activation (x|z after in_proj, y before out_proj) and the
oracle's fall on two sides of a rounding boundary they round one ulp (2^-8 relative) apart,
and each such flip feeds sums over thousands of channels (out_proj; x_proj, hence B, C and dt,
hence every state). The two results then differ by ~3e-4 of their RMS wherever a value itself
is small: 3e-2 relative at 0.01 rms, from the rounding the r17 reading prescribes rather than
from the kernels. The floor-0.01 figure is still measured and printed for every check
(tests/conftest.py); the mixer's own tests keep the 0.01 rms floor."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import BF16_REL_TOL, check, mixed_rel_err, to64

pytestmark = pytest.mark.gpu

mm = pytest.importorskip("mamba_selective_scan_02_amd")


def check_residual_branch(out, x, ref):
    """The bf16 bar applied to the module's contribution out - x rather than to out: the GPU adds
    x to the fp32 out_proj accumulator and rounds once to bf16, so |out - ref| may exceed the
    branch error by at most half a bf16 ulp of the result; the excess over that half ulp is held
    to 2e-2 * max(|ref - x|, rms(ref - x)) element by element."""
    o, xx = to64(out), to64(x)
    d_ref = ref - xx
    rms = float(np.sqrt(np.mean(d_ref * d_ref)))
    mag = np.maximum(np.abs(o), np.abs(ref))
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 1e-30))) - 8)
    excess = np.maximum(np.abs(o - ref) - half_ulp, 0.0)
    e = float(np.max(excess / np.maximum(np.abs(d_ref), rms)))
    assert e <= BF16_REL_TOL, f"out - x: error {e:.3e} > {BF16_REL_TOL}"
    return e


def _layer_case(cfg, seed, *, states=False, conv_bias=False, gamma_random=False, zoh=False):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"[layer] {cfg.name} B={cfg.batch} L={cfg.seqlen} D={cfg.d_inner} R={cfg.dt_rank} "
          f"d_model={cfg.d_model} seed={seed} states={states} zoh={zoh}", flush=True)
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev, conv_bias=conv_bias, gamma_random=gamma_random)
    lay = synth.make_layer(cfg, seed, dev, gamma_random=gamma_random)
    x = synth.make_layer_x(cfg, seed, dev)
    if states:
        cs, ss = synth.make_states(cfg, seed, dev)
    else:
        cs = torch.zeros(cfg.batch, cfg.d_inner, cfg.d_conv - 1, dtype=cfg.torch_dtype, device=dev)
        ss = torch.zeros(cfg.batch, cfg.d_inner, cfg.d_state, dtype=torch.float32, device=dev)
    cs_in, ss_in = cs.clone(), ss.clone()
    out = mm.layer_prefill(x, p, lay, conv_state=cs, ssm_state=ss, states_valid=states,
                           eps=cfg.rms_eps, zoh=zoh)
    torch.cuda.synchronize()
    lay64 = {k: to64(v) for k, v in lay.items()}
    args = (to64(x), oracle.as_f64_params(p), lay64, to64(cs_in) if states else None,
            to64(ss_in) if states else None)
    outr, csr, ssr = oracle.layer_prefill(*args, eps=cfg.rms_eps, zoh=zoh, act_round="bf16")
    oute, _, sse = oracle.layer_prefill(*args, eps=cfg.rms_eps, zoh=zoh)
    print(f"[layer] vs exact-activation oracle: out {mixed_rel_err(out, oute):.3e} "
          f"ssm_state {mixed_rel_err(ss, sse):.3e}", flush=True)
    errs = {"out": check(out, outr, "bf16", "layer out", bf16_floor=1.0),
            "out-x": check_residual_branch(out, x, outr),
            "ssm_state": check(ss, ssr, "bf16", "layer ssm_state", bf16_floor=1.0),
            "conv_state": check(cs, csr, "bf16", "layer conv_state", bf16_floor=1.0)}
    print(f"[layer] errors {errs}", flush=True)
    return out


BASE = synth.MixerConfig("layer_small", 2, 300, 256, 16, 4, 64, "bf16", d_model=256)


def test_layer_small_ragged_states():
    # 600 tokens: four full 128-row GEMM tiles and a ragged fifth
    _layer_case(BASE, 201, states=True, conv_bias=True, gamma_random=True)


def test_layer_zero_states_zoh_three_column_tiles():
    _layer_case(BASE.with_(seqlen=129, d_model=384, name="layer_dm384"), 202, zoh=True)


@pytest.mark.parametrize("L", [1, 2])
def test_layer_single_tokens(L):
    _layer_case(BASE.with_(batch=3, seqlen=L, name=f"layer_L{L}"), 203 + L, states=True)


def test_layer_fused_projection_path():
    # >= 32768 tokens: the fused conv + x_proj + RMSNorm kernel inside the mixer; in_proj
    # (N = 512, 129 x 2 tiles of 256, ragged last row) runs the 256-tile GEMM
    cfg = synth.MixerConfig("layer_fused", 1, 32768 + 77, 256, 16, 4, 64, "bf16", d_model=128)
    _layer_case(cfg, 207, states=True, conv_bias=True, gamma_random=True)


def test_layer_full_width_short_sequence():
    # the d_model 4096 / d_inner 8192 / dt_rank 256 layer on a short ragged sequence: in_proj
    # (N = 16384, 320 tiles of 256 x 256, the last row of tiles 76 rows deep) runs the 256-tile
    # GEMM, out_proj (K = 8192, 80 tiles) the 128-tile one
    cfg = synth.MixerConfig("layer_full_width", 1, 1100, 8192, 16, 4, 256, "bf16", d_model=4096)
    _layer_case(cfg, 208, states=True, conv_bias=True, gamma_random=True)


def test_layer_zero_out_proj_returns_x_bit_exact():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = BASE
    p = synth.make_params(cfg, 209, "cuda")
    lay = synth.make_layer(cfg, 209, "cuda")
    lay["out_proj_w"].zero_()
    x = synth.make_layer_x(cfg, 209, "cuda")
    out = mm.layer_prefill(x, p, lay)
    torch.cuda.synchronize()
    assert torch.equal(out, x)
