"""GPU parity of the fused dt_proj (MM_FLAG_FUSED_DTPROJ): dt_proj + bias + softplus formed
inside the two-pass scan (Jamba analysis page, "The selective mechanism": the step Delta is a
function of the token through a small linear layer) instead of a separate kernel writing dt to
HBM.

The fused scan forms dt with the separate dt_proj kernel's MFMA sequence, so y and both states
must equal the unfused path's bit for bit; each case is also held to the oracle's bar
(tests/parity.py). Shapes span several 96-token blocks with a ragged tail, two sequences (the
per-sequence offset of dt_low), every conv width, paired (A = -(n + 1)) and general A, the
large- and tiny-step inputs, and the 128K workload.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import check, to64

pytestmark = pytest.mark.gpu

mm = pytest.importorskip("mamba_selective_scan_02_amd")

BASE = synth.MixerConfig("fused_dt", 2, 1000, 256, 16, 4, 256, "bf16")

INPUTS = {
    "workload": dict(),                                   # A = -(n + 1): the paired-decay kernel
    "general_A": dict(a_random=True, d_random=True),
    "large_dt": dict(a_random=True, dt_range=(12.0, 40.0)),
    "tiny_dt": dict(a_random=True, dt_range=(1e-7, 1e-5), d_random=True),
}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(cfg, p, xz, cs, ss, **kw):
    cs, ss = cs.clone(), ss.clone()
    y = mm.prefill(xz, p, conv_state=cs, ssm_state=ss, states_valid=True, **kw)
    torch.cuda.synchronize()
    return y, cs, ss


def _case(cfg, seed, kw, *, general_a=False, oracle_check=True):
    _need_gpu()
    print(f"[fused_dt] {cfg.name} B={cfg.batch} L={cfg.seqlen} D={cfg.d_inner} K={cfg.d_conv} "
          f"seed={seed} {kw} general_a={general_a}", flush=True)
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev, conv_bias=True, gamma_random=True, **kw)
    xz = synth.make_xz(cfg, seed, dev)
    cs, ss = synth.make_states(cfg, seed, dev)
    y0, cs0, ss0 = _run(cfg, p, xz, cs, ss, scan="chunked", general_a=general_a)
    y1, cs1, ss1 = _run(cfg, p, xz, cs, ss, scan="chunked", general_a=general_a, fused_dt=True)
    assert torch.equal(y1, y0), f"{cfg.name}: fused y differs from the unfused path"
    assert torch.equal(ss1, ss0), f"{cfg.name}: fused ssm_state differs from the unfused path"
    assert torch.equal(cs1, cs0), f"{cfg.name}: fused conv_state differs from the unfused path"
    if oracle_check:
        p64 = oracle.as_f64_params(p)
        yr, csr, ssr = oracle.mixer_prefill(to64(xz), p64, to64(cs), to64(ss))
        check(y1, yr, cfg.io_dtype, f"{cfg.name} y", f32_large_outputs=True)
        check(ss1, ssr, cfg.io_dtype, f"{cfg.name} ssm_state", f32_large_outputs=True)
        np.testing.assert_array_equal(to64(cs1), csr)


@pytest.mark.parametrize("inp", list(INPUTS))
@pytest.mark.parametrize("K", [2, 3, 4])
def test_fused_dt_matches_unfused_and_oracle(K, inp):
    cfg = BASE.with_(d_conv=K, name=f"fused_dt_k{K}_{inp}")
    _case(cfg, 700 + 10 * K + list(INPUTS).index(inp), INPUTS[inp])


@pytest.mark.parametrize("general_a", [False, True])
def test_fused_dt_declared_general_a(general_a):
    cfg = BASE.with_(name=f"fused_dt_general_a{int(general_a)}")
    _case(cfg, 740, INPUTS["workload"], general_a=general_a)


@pytest.mark.parametrize("L", [1, 7, 33, 95, 96, 97, 192, 289])
def test_fused_dt_lengths(L):
    # a single token, less than one segment, one block and less, exactly one and two blocks,
    # one token past a block (the chunked scan is forced, so the fused path runs at every L)
    cfg = BASE.with_(batch=1, seqlen=L, name=f"fused_dt_L{L}")
    _case(cfg, 750 + L, INPUTS["general_A"])


def test_fused_dt_workspace_and_where_it_applies():
    _need_gpu()
    dev = "cuda"
    cfg = BASE
    p = synth.make_params(cfg, 760, dev, conv_bias=True)
    xz = synth.make_xz(cfg, 760, dev)
    T, D = cfg.batch * cfg.seqlen, cfg.d_inner
    plain = mm.prefill_workspace_bytes(mm.shape_of(xz, p, scan="chunked"))
    fused = mm.prefill_workspace_bytes(mm.shape_of(xz, p, scan="chunked", fused_dt=True))
    assert plain - fused == -(-4 * T * D // 256) * 256, (plain, fused)
    # shapes the fused path does not take: the flag changes nothing (same workspace, same y)
    for name, c, kw in [("zoh", cfg, dict(zoh=True, scan="chunked")),
                        ("f32", cfg.with_(io_dtype="f32"), dict(scan="chunked")),
                        ("dt_rank_64", cfg.with_(dt_rank=64), dict(scan="chunked")),
                        ("sequential", cfg, dict(scan="sequential"))]:
        print(f"[fused_dt] flag ignored: {name}", flush=True)
        pc = synth.make_params(c, 761, dev, conv_bias=True)
        xzc = synth.make_xz(c, 761, dev)
        cs, ss = synth.make_states(c, 761, dev)
        assert (mm.prefill_workspace_bytes(mm.shape_of(xzc, pc, fused_dt=True, **kw)) ==
                mm.prefill_workspace_bytes(mm.shape_of(xzc, pc, **kw))), name
        y0, _, s0 = _run(c, pc, xzc, cs, ss, **kw)
        y1, _, s1 = _run(c, pc, xzc, cs, ss, fused_dt=True, **kw)
        assert torch.equal(y0, y1) and torch.equal(s0, s1), name


def test_fused_dt_long_prefill_128k():
    """The 128K workload (B=1, L=131072, d_inner 8192, dt_rank 256) in the launch configuration
    the benchmark times: the fused path equals the unfused one bit for bit (the unfused path is
    held to the oracle at this size by tests/test_gpu_fullsize.py)."""
    _need_gpu()
    cfg = synth.CONFIGS["long_prefill_128k"]
    print(f"[fused_dt] {cfg.name}", flush=True)
    dev = "cuda"
    p = synth.make_params(cfg, 770, dev)
    xz = synth.make_xz(cfg, 770, dev)
    ss = torch.zeros(cfg.batch, cfg.d_inner, cfg.d_state, device=dev)
    y0 = mm.prefill(xz, p, ssm_state=ss)
    s0 = ss.clone()
    y1 = mm.prefill(xz, p, ssm_state=ss, fused_dt=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y0) and torch.equal(ss, s0)
    del y0, y1
    # paired and general-A instances of the fused kernel at full size
    ya = mm.prefill(xz, p, general_a=True, fused_dt=True)
    yb = mm.prefill(xz, p, general_a=True)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb)
