"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle, element by
element, on the same seeded inputs. Sizes here finish in seconds on the oracle while
spanning several tiles of every kernel and a ragged tail; the full workload sizes are in
test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import check, to64

pytestmark = pytest.mark.gpu

mm = pytest.importorskip("mamba_selective_scan_02_amd")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(cfg, seed, *, states=False, conv_bias=False, gamma_random=False, zoh=False,
          channels=None, check_y=True, scan=None):
    _need_gpu()
    print(f"[case] {cfg.name} B={cfg.batch} L={cfg.seqlen} D={cfg.d_inner} R={cfg.dt_rank} "
          f"io={cfg.io_dtype} seed={seed} states={states} bias={conv_bias} zoh={zoh} scan={scan}",
          flush=True)
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev, conv_bias=conv_bias, gamma_random=gamma_random)
    xz = synth.make_xz(cfg, seed, dev)
    if states:
        cs, ss = synth.make_states(cfg, seed, dev)
    else:
        cs = torch.zeros(cfg.batch, cfg.d_inner, cfg.d_conv - 1, dtype=cfg.torch_dtype, device=dev)
        ss = torch.zeros(cfg.batch, cfg.d_inner, cfg.d_state, dtype=torch.float32, device=dev)
    cs_in, ss_in = cs.clone(), ss.clone()
    y = mm.prefill(xz, p, conv_state=cs, ssm_state=ss, states_valid=states, eps=cfg.rms_eps,
                   zoh=zoh, scan=scan)
    torch.cuda.synchronize()
    yr, csr, ssr = oracle.mixer_prefill(
        to64(xz), oracle.as_f64_params(p), to64(cs_in) if states else None,
        to64(ss_in) if states else None, eps=cfg.rms_eps, zoh=zoh, channels=channels)
    sel = slice(None) if channels is None else channels
    errs = {}
    if check_y:
        errs["y"] = check(y[:, :, sel], yr, cfg.io_dtype, "y")
    errs["ssm_state"] = check(ss[:, sel], ssr, cfg.io_dtype, "ssm_state")
    np.testing.assert_array_equal(to64(cs), csr)
    print(f"[case] errors {errs}", flush=True)
    return y, cs, ss


TINY = synth.CONFIGS["tiny_f32"]


def test_tiny_f32_zero_states():
    _case(TINY, synth.seed_for("tiny_f32"))


def test_tiny_f32_carried_states_bias_gamma():
    _case(TINY, 7, states=True, conv_bias=True, gamma_random=True)


def test_tiny_f32_zoh():
    _case(TINY, 8, states=True, zoh=True)


@pytest.mark.parametrize("L", [1, 2, 3, 77])
def test_f32_ragged_and_short_sequences(L):
    _case(TINY.with_(batch=3, seqlen=L, name=f"f32_L{L}"), 20 + L, states=True, conv_bias=True)


def test_f32_d_conv_variants():
    for K in (2, 3):
        _case(TINY.with_(d_conv=K, seqlen=50, name=f"f32_K{K}"), 30 + K, states=True)


BF16_SMALL = synth.MixerConfig("bf16_small", 2, 300, 256, 16, 4, 64, "bf16")


def test_bf16_small_ragged_tiles():
    _case(BF16_SMALL, 41, states=True, conv_bias=True, gamma_random=True)


def test_bf16_small_zero_states_zoh():
    _case(BF16_SMALL, 42, zoh=True)


@pytest.mark.parametrize("L", [1, 2, 129])
def test_bf16_short_sequences(L):
    _case(BF16_SMALL.with_(seqlen=L, name=f"bf16_L{L}"), 50 + L, states=True)


def test_bf16_mini_prefill_4k_full():
    cfg = synth.CONFIGS["mini_prefill_4k"]
    _case(cfg, synth.seed_for("mini_prefill_4k"))


@pytest.mark.parametrize("scan", ["sequential", "chunked"])
@pytest.mark.parametrize("zoh", [False, True])
def test_both_scan_kernels_f32(scan, zoh):
    # L = 300: two full 128-token blocks and a ragged tail of 44 for the time-parallel kernel
    _case(TINY.with_(batch=2, seqlen=300, name="f32_L300"), 90, states=True, conv_bias=True,
          gamma_random=True, zoh=zoh, scan=scan)


@pytest.mark.parametrize("scan", ["sequential", "chunked"])
@pytest.mark.parametrize("L", [5, 128, 129, 300])
def test_both_scan_kernels_bf16(scan, L):
    _case(BF16_SMALL.with_(seqlen=L, name=f"bf16_L{L}"), 91 + L, states=True, conv_bias=True,
          scan=scan)


@pytest.mark.parametrize("B,L,R,N", [(1, 32768 + 77, 64, 16), (2, 16448, 128, 16),
                                     (1, 32768 + 77, 64, 8), (1, 32768 + 77, 128, 32)])
def test_bf16_fused_projection_path(B, L, R, N):
    # >= 32768 tokens selects the fused conv + x_proj + RMSNorm kernel (128-token tiles, ragged
    # last tile) and the token-stationary dt_proj kernel; d_state 8 / 32 take it with the
    # time-parallel scan of d_state 16 (B|C in one, or two, 16-row blocks of the product)
    cfg = synth.MixerConfig(f"bf16_fused_R{R}_N{N}", B, L, 256, N, 4, R, "bf16")
    _case(cfg, 111 + R + N, states=True, conv_bias=True, gamma_random=True)


def test_chunked_prefill_equals_whole_on_gpu_and_oracle():
    """Prefill over L1 tokens, then L2 more from the returned states, equals one prefill
    (associativity of the page's scan operator); checked against the oracle."""
    _need_gpu()
    cfg = BF16_SMALL.with_(seqlen=257, name="bf16_chunked")
    dev = "cuda"
    p = synth.make_params(cfg, 61, dev, conv_bias=True)
    xz = synth.make_xz(cfg, 61, dev)
    cs0, ss0 = synth.make_states(cfg, 61, dev)
    cs, ss = cs0.clone(), ss0.clone()
    y1 = mm.prefill(xz[:, :100].contiguous(), p, conv_state=cs, ssm_state=ss, states_valid=True)
    y2 = mm.prefill(xz[:, 100:].contiguous(), p, conv_state=cs, ssm_state=ss, states_valid=True)
    torch.cuda.synchronize()
    yr, csr, ssr = oracle.mixer_prefill(to64(xz), oracle.as_f64_params(p), to64(cs0), to64(ss0))
    check(torch.cat([y1, y2], dim=1), yr, "bf16", "y (chunked)")
    check(ss, ssr, "bf16", "ssm_state (chunked)")
    np.testing.assert_array_equal(to64(cs), csr)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_steps_match_oracle(io):
    _need_gpu()
    cfg = (TINY if io == "f32" else BF16_SMALL).with_(batch=4, seqlen=1, name=f"decode_{io}")
    dev = "cuda"
    p = synth.make_params(cfg, 71, dev, conv_bias=True)
    cs, ss = synth.make_states(cfg, 71, dev)
    csr, ssr = to64(cs), to64(ss)
    p64 = oracle.as_f64_params(p)
    for step in range(6):
        xt = synth.make_xz(cfg, 71, dev, seqlen=1, tensor="decode_xz", step=step)[:, 0]
        y = mm.decode_step(xt, p, cs, ss)
        torch.cuda.synchronize()
        yr, csr, ssr = oracle.mixer_decode_step(to64(xt), p64, csr, ssr)
        check(y, yr, io, f"y step {step}")
        check(ss, ssr, io, f"ssm_state step {step}")
        np.testing.assert_array_equal(to64(cs), csr)


# bf16 decode with d_conv 4 runs the decode kernels (x_proj split over channel ranges, fused
# state update); d_conv 3 the general path. Batches span several 64-sequence tiles with a
# ragged one; d_inner spans several channel ranges; each supported dt_rank instantiation.
DECODE_CASES = [
    # name, batch, d_inner, dt_rank, d_conv, conv_bias, zoh, gamma_random
    ("dec_b1_r64", 1, 256, 64, 4, True, False, False),
    ("dec_b130_r128", 130, 1024, 128, 4, False, False, True),
    ("dec_b65_r256_zoh", 65, 2048, 256, 4, True, True, True),
    ("dec_b200_r512", 200, 512, 512, 4, True, False, False),
    ("dec_b70_k3", 70, 512, 64, 3, True, False, False),
    # 5 sequence tiles x 38 ranges of 3 chunks (the last of 1): a grid of 190 workgroups, not a
    # multiple of the 8 XCDs, so the XCD mapping of the x_proj workgroups has a tail
    ("dec_b300_d7168_r64", 300, 7168, 64, 4, True, False, True),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_kernels_match_oracle(case):
    _need_gpu()
    name, B, D, R, K, bias, zoh, gam = case
    cfg = synth.MixerConfig(name, B, 1, D, 16, K, R, "bf16")
    seed = 90 + DECODE_CASES.index(case)
    print(f"[case] {name} B={B} D={D} R={R} K={K} bias={bias} zoh={zoh} seed={seed}", flush=True)
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev, conv_bias=bias, gamma_random=gam)
    cs, ss = synth.make_states(cfg, seed, dev)
    csr, ssr = to64(cs), to64(ss)
    p64 = oracle.as_f64_params(p)
    for step in range(4):
        xt = synth.make_xz(cfg, seed, dev, seqlen=1, tensor="decode_xz", step=step)[:, 0]
        y = mm.decode_step(xt, p, cs, ss, zoh=zoh)
        torch.cuda.synchronize()
        yr, csr, ssr = oracle.mixer_decode_step(to64(xt), p64, csr, ssr, zoh=zoh)
        check(y, yr, "bf16", f"y step {step}")
        check(ss, ssr, "bf16", f"ssm_state step {step}")
        np.testing.assert_array_equal(to64(cs), csr)


def test_prefill_then_decode_equals_longer_prefill():
    """Decoding the last tokens one at a time continues a prefill exactly as a prefill over
    all tokens would (to rounding): the carried states are the whole history."""
    _need_gpu()
    cfg = synth.MixerConfig("dec_continue", 96, 40, 1024, 16, 4, 128, "bf16")
    seed = 97
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev, conv_bias=True)
    xz = synth.make_xz(cfg, seed, dev)
    y_full = mm.prefill(xz, p)
    cs = torch.zeros(cfg.batch, cfg.d_inner, 3, dtype=cfg.torch_dtype, device=dev)
    ss = torch.zeros(cfg.batch, cfg.d_inner, 16, dtype=torch.float32, device=dev)
    n0 = 32
    y_pre = mm.prefill(xz[:, :n0].contiguous(), p, conv_state=cs, ssm_state=ss)
    ys = [y_pre]
    for t in range(n0, cfg.seqlen):
        ys.append(mm.decode_step(xz[:, t].contiguous(), p, cs, ss)[:, None])
    torch.cuda.synchronize()
    yr, _, ssr = oracle.mixer_prefill(to64(xz), oracle.as_f64_params(p))
    check(torch.cat(ys, dim=1), yr, "bf16", "y (prefill + decode)")
    check(y_full, yr, "bf16", "y (prefill)")
    check(ss, ssr, "bf16", "ssm_state (prefill + decode)")


def test_outputs_are_deterministic():
    _need_gpu()
    cfg = BF16_SMALL
    p = synth.make_params(cfg, 81, "cuda")
    xz = synth.make_xz(cfg, 81, "cuda")
    y1 = mm.prefill(xz, p)
    y2 = mm.prefill(xz, p)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# d_state other than 16 with the default kernel selection: fp32 at 77 tokens takes the general
# path (conv, x_proj, RMSNorm, dt_proj kernels and the general time-parallel scan); bf16 at 1100
# tokens the time-parallel scan of d_state 16 (half the state lanes idle for 8, one launch per
# 16 states for 32 / 64)
@pytest.mark.parametrize("N", [8, 32, 64])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_state_size_sweep_prefill(N, io):
    if io == "f32":
        cfg = TINY.with_(batch=2, seqlen=77, d_state=N, name=f"f32_N{N}")
    else:
        # 1100 tokens: 8 full 128-token blocks and a ragged ninth
        cfg = BF16_SMALL.with_(batch=1, seqlen=1100, d_state=N, name=f"bf16_N{N}")
    _case(cfg, 400 + N, states=True, conv_bias=True, gamma_random=True)


# d_state 32 / 64 on the time-parallel kernel: one launch per group of 16 states (state offset
# and stride N), each writing its part of y in fp32, then the combine with D u and the gate;
# d_state 8: one launch with the upper state half of every channel idle
@pytest.mark.parametrize("N", [8, 32, 64])
@pytest.mark.parametrize("io,zoh", [("f32", False), ("f32", True), ("bf16", False), ("bf16", True)])
def test_state_groups_on_the_time_parallel_kernel(N, io, zoh):
    if io == "f32":   # two full 128-token blocks and a ragged tail of 44
        cfg = TINY.with_(batch=2, seqlen=300, d_state=N, name=f"f32_grp_N{N}")
    else:             # 8 blocks and a ragged tail
        cfg = BF16_SMALL.with_(batch=1, seqlen=1100, d_state=N, name=f"bf16_grp_N{N}")
    _case(cfg, 470 + N + 2 * zoh, states=True, conv_bias=True, gamma_random=True, zoh=zoh,
          scan="chunked")


# the general time-parallel scan (csrc/scan_n.hip) where the tuned kernel would be chosen by
# default: "sequential" selects it for d_state != 16; 1100 tokens = two full 512-token ranges and
# a ragged third, with carried states
@pytest.mark.parametrize("N", [8, 32, 64])
@pytest.mark.parametrize("zoh", [False, True])
def test_general_scan_multiple_ranges(N, zoh):
    cfg = BF16_SMALL.with_(batch=1, seqlen=1100, d_state=N, name=f"bf16_general_N{N}")
    _case(cfg, 480 + N + zoh, states=True, conv_bias=True, gamma_random=True, zoh=zoh,
          scan="sequential")


@pytest.mark.parametrize("N", [8, 64])
def test_state_size_sweep_zoh(N):
    _case(BF16_SMALL.with_(seqlen=600, d_state=N, name=f"bf16_zoh_N{N}"), 450 + N, states=True,
          zoh=True)


@pytest.mark.parametrize("N", [8, 32, 64])
def test_state_size_sweep_decode_continues_prefill(N):
    """Prefill, then decode steps one token at a time, at d_state N: equals the oracle's
    prefill over all tokens."""
    _need_gpu()
    cfg = synth.MixerConfig(f"dec_N{N}", 8, 40, 256, N, 4, 64, "bf16")
    seed = 460 + N
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev, conv_bias=True)
    xz = synth.make_xz(cfg, seed, dev)
    cs = torch.zeros(cfg.batch, cfg.d_inner, 3, dtype=cfg.torch_dtype, device=dev)
    ss = torch.zeros(cfg.batch, cfg.d_inner, N, dtype=torch.float32, device=dev)
    n0 = 30
    ys = [mm.prefill(xz[:, :n0].contiguous(), p, conv_state=cs, ssm_state=ss)]
    for t in range(n0, cfg.seqlen):
        ys.append(mm.decode_step(xz[:, t].contiguous(), p, cs, ss)[:, None])
    torch.cuda.synchronize()
    yr, csr, ssr = oracle.mixer_prefill(to64(xz), oracle.as_f64_params(p))
    check(torch.cat(ys, dim=1), yr, "bf16", f"y (N={N}, prefill + decode)")
    check(ss, ssr, "bf16", f"ssm_state (N={N})")
    np.testing.assert_array_equal(to64(cs), csr)
