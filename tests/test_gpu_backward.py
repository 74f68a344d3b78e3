"""GPU parity of the prefill backward (mamba_mixer_prefill_backward, through the C ABI) against
the fp64 backward oracle, on the same seeded inputs.

Bars: dxz is an I/O-dtype output and meets the forward's bar (fp32: max abs 1e-4; bf16: mixed
relative 2e-2, here only the output rounding as the arithmetic is fp32). The other gradients are fp32 sums over tokens and channels;
each tensor is held to a normwise bar, max |g - r| <= 1e-4 * max |r|: fp32 rounding (2^-24)
accumulated over the reverse recurrence and the token reductions stays orders of magnitude
below it, while a wrong term anywhere moves the result by O(1) of the largest entry.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import check, normwise_err, to64

pytestmark = pytest.mark.gpu

mm = pytest.importorskip("mamba_selective_scan_02_amd")

GRAD_TOL = 1e-4
PARAMS = ["conv_w", "conv_b", "x_proj_w", "dt_proj_w", "dt_proj_b", "A", "Dskip", "dt_norm_w",
          "B_norm_w", "C_norm_w"]


def _case(cfg, seed, *, states=True, conv_bias=True, zoh=False, spread_A=True):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"[bwd] {cfg.name} B={cfg.batch} L={cfg.seqlen} D={cfg.d_inner} R={cfg.dt_rank} "
          f"K={cfg.d_conv} io={cfg.io_dtype} seed={seed} states={states} zoh={zoh}", flush=True)
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev, conv_bias=conv_bias, gamma_random=True)
    if spread_A:   # A over a wider range than -(n+1): dt A spans small and large magnitudes
        g = torch.Generator(device="cpu").manual_seed(seed)
        p["A"] = (-torch.exp(torch.rand(p["A"].shape, generator=g) * 3.5 - 2.0)).to(dev)
    xz = synth.make_xz(cfg, seed, dev)
    dy = torch.randn(cfg.batch, cfg.seqlen, cfg.d_inner,
                     generator=torch.Generator(device="cpu").manual_seed(seed + 1)).to(cfg.torch_dtype).to(dev)
    cs = ss = None
    if states:
        cs, ss = synth.make_states(cfg, seed, dev)
    got = mm.prefill_backward(xz, p, dy, conv_state=cs, ssm_state=ss, states_valid=states,
                              eps=cfg.rms_eps, zoh=zoh)
    torch.cuda.synchronize()
    ref = oracle.mixer_prefill_backward(
        to64(xz), oracle.as_f64_params(p), to64(dy), to64(cs) if states else None,
        to64(ss) if states else None, eps=cfg.rms_eps, zoh=zoh)
    errs = {"dxz": check(got["dxz"], ref["xz"], cfg.io_dtype, "dxz")}
    names = [n for n in PARAMS if ref[n] is not None] + ["conv_state0", "ssm_state0"]
    for n in names:
        key = {"conv_state0": "conv_state", "ssm_state0": "ssm_state"}.get(n, n)
        gv = to64(got[key])
        assert np.all(np.isfinite(gv)), n
        e = normwise_err(gv, ref[n])
        errs[n] = e
        assert e <= GRAD_TOL, f"{n}: normwise error {e:.3e} > {GRAD_TOL}"
    print("[bwd] errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)


F32 = synth.MixerConfig("bwd_f32", 2, 77, 64, 16, 4, 8, "f32")


def test_f32_short_ragged_sub_blocks():
    _case(F32, 301)


def test_f32_zero_states_no_bias():
    _case(F32, 302, states=False, conv_bias=False)


@pytest.mark.parametrize("zoh", [False, True])
def test_f32_three_ranges(zoh):
    # 1100 tokens: two full 512-token ranges and a ragged third (76 tokens, 3 sub-blocks)
    _case(F32.with_(batch=1, seqlen=1100, d_inner=128, dt_rank=16, name="bwd_f32_1100"),
          303 + zoh, zoh=zoh)


@pytest.mark.parametrize("K", [2, 3])
def test_f32_d_conv(K):
    _case(F32.with_(d_conv=K, seqlen=40, name=f"bwd_f32_K{K}"), 310 + K)


def test_f32_single_token():
    _case(F32.with_(batch=3, seqlen=1, name="bwd_f32_L1"), 315)


def test_bf16_ragged():
    _case(synth.MixerConfig("bwd_bf16", 2, 600, 256, 16, 4, 64, "bf16"), 320)


def test_bf16_zoh():
    _case(synth.MixerConfig("bwd_bf16_zoh", 1, 530, 128, 16, 4, 64, "bf16"), 321, zoh=True)


def test_bf16_full_width():
    _case(synth.MixerConfig("bwd_bf16_wide", 1, 700, 8192, 16, 4, 256, "bf16"), 322)


def test_backward_is_deterministic():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = synth.MixerConfig("bwd_det", 1, 600, 256, 16, 4, 64, "bf16")
    p = synth.make_params(cfg, 330, "cuda", conv_bias=True)
    xz = synth.make_xz(cfg, 330, "cuda")
    dy = torch.randn(1, 600, 256, device="cuda").bfloat16()
    g1 = mm.prefill_backward(xz, p, dy)
    g2 = mm.prefill_backward(xz, p, dy)
    torch.cuda.synchronize()
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k


def test_bf16_long_sequence_split_k():
    # 8192 tokens: 16 ranges; the weight gradients' products (K = tokens) are split 4 ways
    _case(synth.MixerConfig("bwd_bf16_8k", 1, 8192, 256, 16, 4, 64, "bf16"), 323)
