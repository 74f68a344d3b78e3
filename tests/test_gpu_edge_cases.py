"""GPU parity on the method's edge cases, on every forward scan kernel and the decode kernels,
against the fp64 oracle (bars in tests/parity.py).

The workloads draw A = -(n + 1), D = 1 and dt in [1e-3, 1e-1]. Here instead:
  * general A: A[i, n] = -exp(U(-2, 3)) per (channel, state), with random D (Jamba analysis page,
    "The Mamba Layer", continuous SSM equation: A, D are parameters; ZOH equation: the decay
    exp(dt A) depends on both);
  * large steps: dt0 in [12, 40], so dt_proj's pre-activation crosses softplus's linear-branch
    threshold (20 in the kernels) and dt A reaches -800: exp(dt A) underflows to 0 and the
    recurrence becomes memoryless (h = Bbar u);
  * tiny steps: dt0 in [1e-7, 1e-5] (pre-activation near -16 .. -11.5);
  * zero input x = 0 with a carried SSM state: u = 0 and B = C = RMSNorm(0) = 0, so y = 0
    exactly and the state decays in closed form, h_L = exp(L dt A) h_0 with dt = softplus(bias)
    (recurrence equation with zero input);
  * a bf16 dt_rank (192) outside the tiled dt_proj kernel's instantiations.
Kernels: "sequential" forces the one-lane-per-channel scan (d_state 16) or the general
time-parallel scan (other d_state), "chunked" the tuned time-parallel scan; decode runs the
fused decode kernels (bf16, d_conv 4) and the general path (d_conv 3).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import check, to64

pytestmark = pytest.mark.gpu

mm = pytest.importorskip("mamba_selective_scan_02_amd")

BASE = synth.MixerConfig("edge", 2, 300, 256, 16, 4, 64, "bf16")

INPUTS = {
    "general_A": dict(a_random=True, d_random=True),
    "large_dt": dict(a_random=True, dt_range=(12.0, 40.0)),
    "tiny_dt": dict(a_random=True, dt_range=(1e-7, 1e-5), d_random=True),
}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _prefill_case(cfg, seed, kw, *, zoh=False, scan=None, x_zero=False, conv_bias=True,
                  general_a=False):
    _need_gpu()
    print(f"[edge] {cfg.name} B={cfg.batch} L={cfg.seqlen} D={cfg.d_inner} N={cfg.d_state} "
          f"R={cfg.dt_rank} io={cfg.io_dtype} seed={seed} {kw} zoh={zoh} scan={scan} "
          f"x_zero={x_zero}", flush=True)
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev, conv_bias=conv_bias, gamma_random=True, **kw)
    xz = synth.make_xz(cfg, seed, dev)
    cs, ss = synth.make_states(cfg, seed, dev)
    if x_zero:
        xz[..., :cfg.d_inner] = 0
        cs.zero_()
    cs_in, ss_in = cs.clone(), ss.clone()
    y = mm.prefill(xz, p, conv_state=cs, ssm_state=ss, states_valid=True, zoh=zoh, scan=scan,
                   general_a=general_a)
    torch.cuda.synchronize()
    p64 = oracle.as_f64_params(p)
    yr, csr, ssr = oracle.mixer_prefill(to64(xz), p64, to64(cs_in), to64(ss_in), zoh=zoh)
    # edge inputs reach outputs far above order one (large steps, decay rates up to 20, 64
    # states): the fp32 bar is taken relative to the largest output there (tests/parity.py)
    check(y, yr, cfg.io_dtype, f"{cfg.name} y", f32_large_outputs=True)
    check(ss, ssr, cfg.io_dtype, f"{cfg.name} ssm_state", f32_large_outputs=True)
    np.testing.assert_array_equal(to64(cs), csr)
    return y, ss, p64, to64(ss_in)


@pytest.mark.parametrize("scan", ["sequential", "chunked"])
@pytest.mark.parametrize("inp", list(INPUTS))
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_edge_inputs_d_state_16(io, inp, scan):
    cfg = BASE.with_(io_dtype=io, name=f"edge_{io}_{inp}_{scan}")
    _prefill_case(cfg, 600 + list(INPUTS).index(inp), INPUTS[inp], scan=scan)


@pytest.mark.parametrize("zoh", [False, True])
@pytest.mark.parametrize("inp", ["general_A", "large_dt"])
def test_edge_inputs_zoh_both_scans(inp, zoh):
    for scan in ("sequential", "chunked"):
        cfg = BASE.with_(name=f"edge_zoh{int(zoh)}_{inp}_{scan}")
        _prefill_case(cfg, 610 + zoh, INPUTS[inp], zoh=zoh, scan=scan)


@pytest.mark.parametrize("N", [8, 32, 64])
@pytest.mark.parametrize("inp", list(INPUTS))
def test_edge_inputs_other_state_sizes(N, inp):
    # "sequential": the general time-parallel scan (1100 tokens: two full ranges and a ragged
    # third); "chunked": the tuned kernel's state groups
    for scan in ("sequential", "chunked"):
        cfg = BASE.with_(batch=1, seqlen=1100, d_state=N, name=f"edge_N{N}_{inp}_{scan}")
        _prefill_case(cfg, 620 + N, INPUTS[inp], scan=scan)


@pytest.mark.parametrize("scan", ["sequential", "chunked"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_zero_input_closed_form(io, scan):
    """x = 0: y is exactly 0 and h_L = exp(L dt A) h_0 with dt = softplus(dt_proj bias)."""
    cfg = BASE.with_(io_dtype=io, name=f"edge_zero_x_{io}_{scan}")
    y, ss, p64, ss0 = _prefill_case(cfg, 630, dict(a_random=True, dt_range=(1e-3, 1e-2)),
                                    scan=scan, x_zero=True, conv_bias=False)
    assert torch.count_nonzero(y).item() == 0, "y must be exactly zero for zero input"
    b = p64["dt_proj_b"]
    dt = np.maximum(b, 0.0) + np.log1p(np.exp(-np.abs(b)))        # softplus, fp64
    h_closed = np.exp(cfg.seqlen * dt[None, :, None] * p64["A"][None]) * ss0
    check(ss, h_closed, io, f"{cfg.name} ssm_state vs exp(L dt A) h0")


def test_bf16_generic_dt_rank():
    # dt_rank 192: the bf16 dt_proj runs on the generic split-precision GEMM
    cfg = BASE.with_(dt_rank=192, name="edge_R192")
    _prefill_case(cfg, 640, INPUTS["general_A"])
    _prefill_case(cfg.with_(seqlen=1, name="edge_R192_L1"), 641, INPUTS["large_dt"])


DEC = [("fast_k4", 4), ("general_k3", 3)]


@pytest.mark.parametrize("inp", list(INPUTS))
@pytest.mark.parametrize("dec", DEC, ids=[d[0] for d in DEC])
@pytest.mark.parametrize("zoh", [False, True])
def test_edge_inputs_decode(dec, inp, zoh):
    _need_gpu()
    name, K = dec
    cfg = synth.MixerConfig(f"edge_dec_{name}_{inp}", 70, 1, 512, 16, K, 64, "bf16")
    seed = 650 + K + 3 * list(INPUTS).index(inp)
    print(f"[edge] {cfg.name} B=70 D=512 K={K} seed={seed} zoh={zoh}", flush=True)
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev, conv_bias=True, gamma_random=True, **INPUTS[inp])
    cs, ss = synth.make_states(cfg, seed, dev)
    csr, ssr = to64(cs), to64(ss)
    p64 = oracle.as_f64_params(p)
    for step in range(3):
        xt = synth.make_xz(cfg, seed, dev, seqlen=1, tensor="decode_xz", step=step)[:, 0]
        y = mm.decode_step(xt, p, cs, ss, zoh=zoh)
        torch.cuda.synchronize()
        yr, csr, ssr = oracle.mixer_decode_step(to64(xt), p64, csr, ssr, zoh=zoh)
        check(y, yr, "bf16", f"{cfg.name} y step {step}")
        check(ss, ssr, "bf16", f"{cfg.name} ssm_state step {step}")
        np.testing.assert_array_equal(to64(cs), csr)


def test_zero_input_decode_closed_form():
    """Decode steps with x = 0 and a zero conv state: y = 0 exactly and each step scales the
    state by exp(dt A)."""
    _need_gpu()
    cfg = synth.MixerConfig("edge_dec_zero", 70, 1, 512, 16, 4, 64, "bf16")
    dev = "cuda"
    p = synth.make_params(cfg, 660, dev, a_random=True, dt_range=(1e-3, 1e-1))
    cs, ss = synth.make_states(cfg, 660, dev)
    cs.zero_()
    ss0 = to64(ss)
    steps = 5
    for step in range(steps):
        xt = synth.make_xz(cfg, 660, dev, seqlen=1, tensor="decode_xz", step=step)[:, 0]
        xt[:, :cfg.d_inner] = 0
        y = mm.decode_step(xt, p, cs, ss)
        torch.cuda.synchronize()
        assert torch.count_nonzero(y).item() == 0, f"y must be zero at step {step}"
    p64 = oracle.as_f64_params(p)
    b = p64["dt_proj_b"]
    dt = np.maximum(b, 0.0) + np.log1p(np.exp(-np.abs(b)))
    h_closed = np.exp(steps * dt[None, :, None] * p64["A"][None]) * ss0
    check(ss, h_closed, "bf16", "decode ssm_state vs exp(steps dt A) h0")


@pytest.mark.parametrize("N", [16, 32, 64])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_paired_decay_and_general_paths(io, N):
    """A = -(n + 1): the lane kernel's paired-decay path (the default) and the path that
    evaluates every exp(dt A) (MM_FLAG_SCAN_GENERAL_A) both match the oracle, and each other
    to fp32 rounding; random A (no arithmetic progression) takes the general path either way."""
    cfg = BASE.with_(io_dtype=io, batch=1, seqlen=700, d_state=N, name=f"edge_paired_{io}_N{N}")
    y1, s1, _, _ = _prefill_case(cfg, 670 + N, {}, scan="chunked")
    y2, s2, _, _ = _prefill_case(cfg, 670 + N, {}, scan="chunked", general_a=True)
    assert float((s1 - s2).abs().max()) <= 1e-5 * max(1.0, float(s2.abs().max()))
    _prefill_case(cfg.with_(name=f"edge_unpaired_{io}_N{N}"), 680 + N, INPUTS["general_A"],
                  scan="chunked")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_mixed_paired_and_general_channels(io):
    """A = -(n + 1) on the first half of the channels and random A on the rest, default flags:
    the time-parallel d_state-16 scan runs the workgroups with paired decay and the others in
    two launches (each exits on the other's); every channel matches the oracle."""
    _need_gpu()
    cfg = BASE.with_(io_dtype=io, name=f"edge_mixed_A_{io}")
    seed = 690
    print(f"[edge] {cfg.name} seed={seed} mixed A, scan=chunked", flush=True)
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev, conv_bias=True, gamma_random=True,
                          **INPUTS["general_A"])
    half = cfg.d_inner // 2
    p["A"][:half] = -torch.arange(1, cfg.d_state + 1, dtype=torch.float32, device=dev)
    xz = synth.make_xz(cfg, seed, dev)
    cs, ss = synth.make_states(cfg, seed, dev)
    cs_in, ss_in = cs.clone(), ss.clone()
    y = mm.prefill(xz, p, conv_state=cs, ssm_state=ss, states_valid=True, scan="chunked")
    torch.cuda.synchronize()
    yr, csr, ssr = oracle.mixer_prefill(to64(xz), oracle.as_f64_params(p), to64(cs_in),
                                        to64(ss_in))
    check(y, yr, cfg.io_dtype, f"{cfg.name} y", f32_large_outputs=True)
    check(ss, ssr, cfg.io_dtype, f"{cfg.name} ssm_state", f32_large_outputs=True)
    np.testing.assert_array_equal(to64(cs), csr)
