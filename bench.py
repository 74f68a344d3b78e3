"""Benchmark of the gfx950 Mamba-1 mixer core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]

One step = one mamba_mixer_prefill over the long-context workload (B=1, L=131072,
d_inner=8192, d_state=16, d_conv=4, dt_rank=256, bf16 I/O, fp32 state): conv1d+SiLU,
x_proj, RMSNorm, dt_proj+softplus, selective scan with D feed-through and SiLU(z) gate,
final conv/SSM states. The headline evaluates every exp(dt A) of the scan directly
(MM_FLAG_SCAN_GENERAL_A), as for an arbitrary A. Inputs are synthetic, seeded, resident in HBM
before timing. Further legs, reported beside the headline: the same prefill with the library's
default, which detects that A = -(n + 1) has equally spaced decay rates and forms the decays
from fewer exps ("paired_decay"); dt_proj fused into the scan (MM_FLAG_FUSED_DTPROJ, no dt
buffer); the ZOH input matrix; the 4K and 2 x 256K prefills; 512
batched decode steps (B=256) at d_inner 8192 and 16384 after a 1024-token prefill seeds the
states; mamba_layer_prefill (pre-RMSNorm, in_proj 4096 -> 16384, the mixer, out_proj 8192 ->
4096 with the residual) and mamba_mixer_prefill_backward on the 128K tokens; the prefill at
d_state 8, 16, 32 and 64; and the fp64 oracle on the host's cores. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PREFILL_WORKLOAD = "long_prefill_128k"
DECODE_WORKLOAD = "decode_b256"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor peak
CU, CLOCK_HZ = 256, 2.4e9
# MI355X published fp32 vector peak 157.3 TFLOP/s = 256 CUs x 2.4 GHz x 128 lanes x 2 (an FMA
# is two flops): 128 fp32 VALU lane-operations per clock per CU
VALU_LANE_OPS_PER_S = 157.3e12 / 2
# v_exp_f32 issue rate, measured on gfx950 (profiles/valu_rates_probe.md): ~30 lanes/clk/CU
EXP_LANE_OPS_PER_S = 30.0 * CU * CLOCK_HZ


def scan_alu_peak_updates_per_s() -> float:
    """ALU roofline of the selective scan in state updates (token, channel, state) per second.
    Each update needs 4 fp32 VALU operations (dt*A, (dt*u)*B, the h FMA, the y FMA) at the
    published VALU rate and one v_exp_f32 at its measured rate, which do not overlap
    (profiles/valu_rates_probe.md): 1 / (4 / VALU + 1 / EXP) updates per second."""
    return 1.0 / (4.0 / VALU_LANE_OPS_PER_S + 1.0 / EXP_LANE_OPS_PER_S)


def scan_algorithmic_bytes(cfg) -> int:
    """Bytes the scan kernel must move per launch: read x and z (the two halves of xz, bf16),
    dt (fp32), B and C (fp32, 2N per token); write y (bf16); plus the SSM state in/out."""
    T, D, N = cfg.batch * cfg.seqlen, cfg.d_inner, cfg.d_state
    return T * D * (2 + 2 + 4 + 2) + T * 2 * N * 4 + 2 * cfg.batch * D * N * 4


def scan_source_sha256() -> str:
    """Hash of the scan kernel's source: scan.hip, common.h and the ScanArgs definition in
    kernels.h (the rest of kernels.h declares other kernels)."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "mamba_selective_scan_02_amd", "csrc")
    h = hashlib.sha256()
    for f in ("scan.hip", "common.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    hdr = open(os.path.join(csrc, "kernels.h")).read()
    m = re.search(r"struct ScanArgs \{.*?\n\};", hdr, re.S)
    h.update(m.group(0).encode() if m else b"")
    return h.hexdigest()


def measured_scan_traffic():
    """HBM bytes per launch of the scan kernel from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (profiles/selective_scan_traffic.json), or None when the scan kernel's
    sources have changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "selective_scan_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))["selective_scan"]
    if scan_source_sha256() != rec["source_sha256"] or rec["workload"] != PREFILL_WORKLOAD:
        return None
    return rec["read_bytes"] + rec["write_bytes"]


MFMA_BF16_PEAK_FLOPS = 2.5e15  # MI355X dense bf16 MFMA, vendor peak


def copy_ceiling_gbs() -> float:
    """Measured device-copy bandwidth (read + write) on this GPU: the practical HBM ceiling
    against which the bandwidth-bound stages are also reported."""
    a = torch.empty(1 << 29, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbs = 5 * 2 * a.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbs


def stage_view(ms, nbytes=None, flops=None, copy_gbs=None):
    """One stage's time with its algorithmic bytes (GB/s, fraction of the HBM peak and of the
    measured copy ceiling) and, for the projections, algorithmic flops (MFMA utilisation)."""
    out = {"ms": ms}
    if nbytes is not None:
        gbs = nbytes / (ms * 1e-3) / 1e9
        out.update({"algorithmic_bytes": nbytes, "GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS})
        if copy_gbs:
            out["copy_frac"] = gbs / copy_gbs
    if flops is not None:
        out.update({"algorithmic_flops": flops,
                    "mfma_util": flops / (ms * 1e-3) / MFMA_BF16_PEAK_FLOPS})
    return out


def prefill_leg(args, mm, workload=PREFILL_WORKLOAD, general_a=True, zoh=False, steps=None,
                warmup=None, fused_dt=False):
    """Time mamba_mixer_prefill on a prefill workload; per-stage times from HIP events on the
    launch stream (the *_timed entry point)."""
    cfg = synth.CONFIGS[workload]
    seed = synth.seed_for(workload)
    dev = "cuda"
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    p = synth.make_params(cfg, seed, dev)
    xz = synth.make_xz(cfg, seed, dev)
    y = torch.empty(cfg.batch, cfg.seqlen, cfg.d_inner, dtype=cfg.torch_dtype, device=dev)
    cs = torch.zeros(cfg.batch, cfg.d_inner, cfg.d_conv - 1, dtype=cfg.torch_dtype, device=dev)
    ss = torch.zeros(cfg.batch, cfg.d_inner, cfg.d_state, dtype=torch.float32, device=dev)
    shape = mm.shape_of(xz, p, eps=cfg.rms_eps, zoh=zoh, general_a=general_a, fused_dt=fused_dt)
    ws = mm.alloc_workspace(mm.prefill_workspace_bytes(shape), dev)
    timer = mm.StageTimer()

    def step(t=None):
        mm.prefill(xz, p, conv_state=cs, ssm_state=ss, states_valid=False, y=y, workspace=ws,
                   eps=cfg.rms_eps, timer=t, zoh=zoh, general_a=general_a, fused_dt=fused_dt)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    timer.reset()
    print(f"[bench] prefill {workload} general_a={general_a} zoh={zoh} fused_dt={fused_dt}: "
          f"{warmup} warmup done, "
          f"timing {steps}", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = timer.read()
    ms_per_step = wall * 1e3 / steps
    tokens = cfg.batch * cfg.seqlen
    scan_ms, scan_n = stages["selective_scan"]
    scan_avg_s = scan_ms / max(scan_n, 1) * 1e-3
    updates = tokens * cfg.d_inner * cfg.d_state
    sbytes = scan_algorithmic_bytes(cfg)
    out = {
        "value": tokens / (ms_per_step * 1e-3),
        "ms_per_step": ms_per_step,
        "steps": steps,
        "config": {"workload": workload, "batch": cfg.batch, "seq_len": cfg.seqlen,
                   "d_inner": cfg.d_inner, "d_state": cfg.d_state, "d_conv": cfg.d_conv,
                   "dt_rank": cfg.dt_rank, "io_dtype": cfg.io_dtype, "state_dtype": "f32",
                   "scan_exps": "every exp(dt A)" if (general_a or zoh) else
                                "paired decay (A = -(n + 1) detected)",
                   "bbar": "zoh" if zoh else "first-order",
                   "dt_proj": "fused into the scan" if fused_dt else "own kernel, dt via HBM",
                   "workspace_bytes": mm.prefill_workspace_bytes(shape)},
        "scan": {"ms": scan_avg_s * 1e3, "state_updates_per_s": updates / scan_avg_s,
                 "algorithmic_bytes": sbytes, "GBs": sbytes / scan_avg_s / 1e9,
                 "hbm_frac": sbytes / scan_avg_s / 1e9 / HBM_PEAK_GBS},
        "stages_ms_per_step": {k: v[0] / max(v[1], 1) for k, v in stages.items() if v[1]},
    }
    # per-stage rooflines: the fused conv + x_proj + RMSNorm reads x and writes dt_low (hi, lo)
    # and B|C; dt_proj reads dt_low and writes dt (fp32); weights are counted once
    T, D, R, N = tokens, cfg.d_inner, cfg.dt_rank, cfg.d_state
    sm = out["stages_ms_per_step"]
    copy_gbs = args.copy_gbs
    xproj_bytes = T * D * 2 + T * R * 4 + T * 2 * N * 4 + (R + 2 * N) * D * 2 + D * cfg.d_conv * 2
    dtproj_bytes = T * R * 4 + T * D * 4 + D * R * 2
    out["stages"] = {
        "selective_scan": stage_view(sm["selective_scan"], sbytes, None, copy_gbs)}
    if "x_proj" in sm:
        out["stages"]["x_proj"] = stage_view(sm["x_proj"], xproj_bytes, 2 * T * D * (R + 2 * N),
                                             copy_gbs)
    if "dt_proj_softplus" in sm:
        out["stages"]["dt_proj_softplus"] = stage_view(sm["dt_proj_softplus"], dtproj_bytes,
                                                       2 * T * D * R, copy_gbs)
    mixer_min = T * D * (4 + 2)            # xz in, y out: the mixer's own I/O
    unfused = scan_algorithmic_bytes(cfg) + T * D * 4 + xproj_bytes + dtproj_bytes
    out["mixer"] = {"min_bytes": mixer_min, "unfused_design_bytes": unfused,
                    "min_bytes_hbm_frac": mixer_min / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "copy_ceiling_GBs": copy_gbs}
    del xz, y, ws
    return out, (p, cfg)


def headline_roofline(pre):
    """The dominant kernel (the selective scan) against its ALU roofline, with its fraction of
    the HBM peak beside it."""
    sc = pre["scan"]
    peak = scan_alu_peak_updates_per_s()
    return {"bound": "alu", "kernel": "selective_scan (every exp(dt A) evaluated)",
            "achieved": sc["state_updates_per_s"], "peak": peak, "unit": "state-updates/s",
            "frac": sc["state_updates_per_s"] / peak,
            "hbm_frac": sc["hbm_frac"], "hbm_GBs": sc["GBs"], "hbm_peak_GBs": HBM_PEAK_GBS,
            "algorithmic_bytes": sc["algorithmic_bytes"],
            "peak_derivation": "1 / (4 / 7.865e13 + 1 / 1.843e13) updates/s: 4 fp32 VALU ops "
                               "per update at the published 157.3 TFLOP/s fp32 vector rate, one "
                               "v_exp_f32 at its measured 30 lanes/clk/CU, not overlapped",
            "traffic": measured_scan_traffic(), "traffic_unit": "bytes/launch"}


def decode_leg(args, mm, steps=None, workload=DECODE_WORKLOAD):
    cfg = synth.CONFIGS[workload]
    seed = synth.seed_for(workload)
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev)
    cs = torch.zeros(cfg.batch, cfg.d_inner, cfg.d_conv - 1, dtype=cfg.torch_dtype, device=dev)
    ss = torch.zeros(cfg.batch, cfg.d_inner, cfg.d_state, dtype=torch.float32, device=dev)
    # seeded random prefill of 1024 tokens per sequence gives the carried states
    pre = synth.make_xz(cfg, seed, dev, seqlen=cfg.decode_prefix)
    mm.prefill(pre, p, conv_state=cs, ssm_state=ss, states_valid=False, eps=cfg.rms_eps)
    del pre
    steps = cfg.decode_steps if steps is None else steps
    xs = synth.make_xz(cfg, seed, dev, seqlen=steps, tensor="decode_xz")  # [B, steps, 2D]
    xs = xs.transpose(0, 1).contiguous()                                   # [steps, B, 2D]
    y = torch.empty(cfg.batch, cfg.d_inner, dtype=cfg.torch_dtype, device=dev)
    shape = mm.shape_of(xs[0], p, decode=True, eps=cfg.rms_eps)
    ws = mm.alloc_workspace(mm.decode_workspace_bytes(shape), dev)
    timer = mm.StageTimer()
    for i in range(min(8, steps)):
        mm.decode_step(xs[i], p, cs, ss, y=y, workspace=ws, eps=cfg.rms_eps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        mm.decode_step(xs[i], p, cs, ss, y=y, workspace=ws, eps=cfg.rms_eps, timer=timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = timer.read()
    # the same steps captured once in a HIP graph and replayed (no per-step host launches)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(steps):
                mm.decode_step(xs[i], p, cs, ss, y=y, workspace=ws, eps=cfg.rms_eps)
    torch.cuda.current_stream().wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    gwall = time.perf_counter() - t0
    # state read + write (fp32), conv state read + write, xz in, y out, weights once per step
    D, N, K, R, B = cfg.d_inner, cfg.d_state, cfg.d_conv, cfg.dt_rank, cfg.batch
    step_bytes = (B * D * N * 4 * 2 + B * D * (K - 1) * 2 * 2 + B * 2 * D * 2 + B * D * 2
                  + (R + 2 * N) * D * 2 + D * R * 2)
    return {"metric": "decode steps/sec", "value": steps / wall, "unit": "steps/s",
            "tokens_per_s": steps * B / wall, "ms_per_step": wall * 1e3 / steps,
            "workload": workload, "batch": B, "d_inner": D, "dt_rank": R, "steps": steps,
            "hbm_frac_of_step": step_bytes / (wall / steps) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes_per_step": step_bytes,
            "stages_ms_per_step": {k: v[0] / max(v[1], 1) for k, v in stages.items() if v[1]},
            # the state update (conv, scan step, gate, conv-state shift): state read + write,
            # conv state read + write, xz, dt (fp32) and y
            "graph_replay": {"steps_per_s": steps / gwall, "tokens_per_s": steps * B / gwall,
                             "ms_per_step": gwall * 1e3 / steps,
                             "hbm_frac_of_step": step_bytes / (gwall / steps) / 1e9 / HBM_PEAK_GBS},
            "update_stage": stage_view(stages["selective_scan"][0] / max(stages["selective_scan"][1], 1),
                                       B * D * (N * 4 * 2 + (K - 1) * 2 * 2 + 2 * 2 + 4 + 2),
                                       None, args.copy_gbs)}


def layer_leg(args, mm, steps=None):
    """mamba_layer_prefill over the 128K workload at d_model 4096 (x ~ N(0, 1), random weights)."""
    cfg = synth.CONFIGS[PREFILL_WORKLOAD]
    seed = synth.seed_for(PREFILL_WORKLOAD)
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev)
    lay = synth.make_layer(cfg, seed, dev)
    x = synth.make_layer_x(cfg, seed, dev)
    out = torch.empty_like(x)
    shape = mm.make_shape(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, cfg.d_conv,
                          cfg.dt_rank, x.dtype, cfg.rms_eps, 0)
    ws = mm.alloc_workspace(mm.layer_workspace_bytes(shape, cfg.d_model), dev)
    timer = mm.StageTimer()
    steps = args.steps if steps is None else steps

    def step(t=None):
        mm.layer_prefill(x, p, lay, out=out, workspace=ws, eps=cfg.rms_eps, timer=t)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = {k: v[0] / max(v[1], 1) for k, v in timer.read().items() if v[1]}
    T, D, Dm = cfg.batch * cfg.seqlen, cfg.d_inner, cfg.d_model
    ms = wall * 1e3 / steps
    return {"metric": "Mamba layer prefill tokens/sec at L=128K", "value": T / (ms * 1e-3),
            "unit": "tokens/s", "ms_per_step": ms, "steps": steps,
            "config": {"workload": PREFILL_WORKLOAD, "d_model": Dm, "d_inner": D,
                       "dt_rank": cfg.dt_rank, "d_state": cfg.d_state, "io_dtype": "bf16"},
            "stages_ms_per_step": st,
            "stages": {
                # x read, xn written, gain once
                "layer_rmsnorm": stage_view(st["layer_rmsnorm"], T * Dm * 2 * 2 + Dm * 4, None,
                                            args.copy_gbs),
                "in_proj": stage_view(st["in_proj"], None, 2 * T * Dm * 2 * D),
                "out_proj": stage_view(st["out_proj"], None, 2 * T * D * Dm)}}


def state_sweep_leg(args, mm, sizes=(8, 16, 32, 64)):
    """The 128K prefill at d_state 8, 16, 32, 64 (same widths; A[i, n] = -(n + 1))."""
    base = synth.CONFIGS[PREFILL_WORKLOAD]
    seed = synth.seed_for(PREFILL_WORKLOAD)
    out = {}
    steps = max(1, min(args.steps, 3))
    for N in sizes:
        cfg = base.with_(d_state=N, name=f"{PREFILL_WORKLOAD}_N{N}")
        p = synth.make_params(cfg, seed, "cuda")
        xz = synth.make_xz(cfg, seed, "cuda")
        y = torch.empty(cfg.batch, cfg.seqlen, cfg.d_inner, dtype=cfg.torch_dtype, device="cuda")
        shape = mm.shape_of(xz, p, eps=cfg.rms_eps)
        ws = mm.alloc_workspace(mm.prefill_workspace_bytes(shape), "cuda")
        timer = mm.StageTimer()
        mm.prefill(xz, p, y=y, workspace=ws, eps=cfg.rms_eps)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            mm.prefill(xz, p, y=y, workspace=ws, eps=cfg.rms_eps, timer=timer)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        st = {k: v[0] / max(v[1], 1) for k, v in timer.read().items() if v[1]}
        T = cfg.batch * cfg.seqlen
        out[str(N)] = {"tokens_per_s": T / (ms * 1e-3), "ms_per_step": ms,
                       "scan_ms": st["selective_scan"],
                       "scan_state_updates_per_s": T * cfg.d_inner * N / (st["selective_scan"] * 1e-3),
                       "stages_ms_per_step": st}
        del p, xz, y, ws
        torch.cuda.empty_cache()
    return {"workload": PREFILL_WORKLOAD, "steps": steps, "by_d_state": out}


def backward_scan_alu_peak_updates_per_s() -> float:
    """ALU roofline of the backward's scan in state updates per second, counted in fp32 VALU
    issue slots at the published vector rate: per (token, channel, state) the forward state
    (dt*A, one v_exp_f32 taken as 2 slots, (dt*u)*B, the h FMA: 5 slots) and the reverse step
    (dh = C*dys + carry, dh*h_prev, dh*u, d dt = (dh*h_prev*a)*A + (dh*u)*B: 3,
    dA += (dh*h_prev*a)*dt, dB term dh*u*dt, dC term dys*h, du term dh*dt*B: 2,
    carry = a*dh: 12 slots): 17 issue slots."""
    return VALU_LANE_OPS_PER_S / 17.0


def backward_leg(args, mm, steps=None):
    """mamba_mixer_prefill_backward over the 128K workload (dy ~ N(0, 1), seeded)."""
    cfg = synth.CONFIGS[PREFILL_WORKLOAD]
    seed = synth.seed_for(PREFILL_WORKLOAD)
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev)
    xz = synth.make_xz(cfg, seed, dev)
    dy = synth.make_xz(cfg, seed + 1, dev)[:, :, :cfg.d_inner].contiguous()
    shape = mm.shape_of(xz, p, eps=cfg.rms_eps)
    ws = mm.alloc_workspace(mm.backward_workspace_bytes(shape), dev)
    timer = mm.StageTimer()
    steps = max(1, min(args.steps, 5)) if steps is None else steps
    grads = mm.prefill_backward(xz, p, dy, workspace=ws, eps=cfg.rms_eps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        mm.prefill_backward(xz, p, dy, grads=grads, workspace=ws, eps=cfg.rms_eps, timer=timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = {k: v[0] / max(v[1], 1) for k, v in timer.read().items() if v[1]}
    T, D, N, R = cfg.batch * cfg.seqlen, cfg.d_inner, cfg.d_state, cfg.dt_rank
    ms = wall * 1e3 / steps
    W = R + 2 * N
    # six products: x_proj, its input and weight gradients (inner size W), and the same three
    # for dt_proj (R)
    gemm_flops = 2 * T * D * (3 * W + 3 * R)
    return {"metric": "mixer prefill backward tokens/sec at L=128K", "value": T / (ms * 1e-3),
            "unit": "tokens/s", "ms_per_step": ms, "steps": steps,
            "config": {"workload": PREFILL_WORKLOAD, "d_inner": D, "dt_rank": R, "d_state": N,
                       "io_dtype": "bf16", "arithmetic": "f32"},
            "stages_ms_per_step": st,
            # the reverse scan stage: state updates per second (each (token, channel, state)
            # is recomputed twice forward and walked once backward)
            "scan_state_updates_per_s": T * D * N / (st["bwd_scan"] * 1e-3),
            "roofline": {"bound": "alu", "kernel": "bwd_scan stage (transfers, carries, reverse scan "
                                                   "with the softplus and gate derivatives)",
                         "achieved": T * D * N / (st["bwd_scan"] * 1e-3),
                         "peak": backward_scan_alu_peak_updates_per_s(), "unit": "state-updates/s",
                         "frac": T * D * N / (st["bwd_scan"] * 1e-3) / backward_scan_alu_peak_updates_per_s()},
            "gemm_algorithmic_flops": gemm_flops,
            "gemm_TFLOPs_in_recompute_and_proj": gemm_flops / ((st["bwd_recompute"] + st["bwd_proj"]) * 1e-3) / 1e12}


def cpu_baseline(tokens: int):
    """The fp64 oracle, as it stands, on a bounded sample of the workloads, on this host's
    cores: the first `tokens` tokens of the 128K input on every core (the oracle's own thread
    pool over token blocks for conv + x_proj + RMSNorm, the BLAS threads for dt_proj; its scan
    is one thread of numpy over all channels), plus one-thread times of the tiny fp32 workload
    and of the first 512 tokens of the 4K prefill."""
    import threadpoolctl
    import oracle
    nproc = os.cpu_count() or 1

    def inputs(name, ntok):
        cfg = synth.CONFIGS[name]
        seed = synth.seed_for(name)
        p = synth.make_params(cfg, seed, "cuda")
        xz = synth.make_xz(cfg, seed, "cuda", seqlen=ntok)
        return oracle.as_f64_params(p), xz.float().cpu().double().numpy(), cfg

    p64, x, cfg = inputs(PREFILL_WORKLOAD, tokens)
    blas = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    t0 = time.perf_counter()
    oracle.mixer_prefill(x, p64, eps=cfg.rms_eps, token_block=max(64, tokens // nproc),
                         workers=nproc)
    dt = time.perf_counter() - t0
    out = {"value": tokens * cfg.batch / dt, "unit": "tokens/s", "cores": max(nproc, blas),
           "nproc": nproc, "blas_threads": blas, "kind": "oracle",
           "sample": (f"first {tokens} tokens of the {PREFILL_WORKLOAD} input, all "
                      f"{cfg.d_inner} channels, fp64 numpy ({dt:.1f} s): conv + x_proj + RMSNorm "
                      f"on a pool of {nproc} threads over token blocks, dt_proj on {blas} BLAS "
                      f"threads, the sequential scan on one thread")}
    one = {}
    with threadpoolctl.threadpool_limits(1):
        for name, ntok in (("tiny_f32", synth.CONFIGS["tiny_f32"].seqlen), ("mini_prefill_4k", 512)):
            p64, x, cfg = inputs(name, ntok)
            t0 = time.perf_counter()
            oracle.mixer_prefill(x, p64, eps=cfg.rms_eps)
            dt = time.perf_counter() - t0
            one[name] = {"tokens": ntok, "s": dt, "tokens_per_s": ntok * cfg.batch / dt}
    out["one_thread"] = one
    return out


def profile_run(args, mm):
    """A short, fixed sequence of launches for rocprofv3 (kernel trace or counters)."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)                       # plain copy: 1 GiB read + 1 GiB written
    torch.cuda.synchronize()
    del a, b
    args.steps, args.warmup = max(1, min(args.steps, 3)), 1
    prefill_leg(args, mm)
    torch.cuda.synchronize()
    print("[profile] prefill done", file=sys.stderr, flush=True)
    prefill_leg(args, mm, general_a=False)
    torch.cuda.synchronize()
    print("[profile] paired-decay prefill done", file=sys.stderr, flush=True)
    prefill_leg(args, mm, fused_dt=True)
    torch.cuda.synchronize()
    print("[profile] fused dt_proj prefill done", file=sys.stderr, flush=True)
    decode_leg(args, mm, steps=32)
    torch.cuda.synchronize()
    print("[profile] decode done", file=sys.stderr, flush=True)
    if not args.no_layer:
        layer_leg(args, mm, steps=2)
        torch.cuda.synchronize()
        print("[profile] layer done", file=sys.stderr, flush=True)
    if not args.no_backward:
        backward_leg(args, mm, steps=1)
        torch.cuda.synchronize()
        print("[profile] backward done", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-layer", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-prefill-legs", action="store_true",
                    help="skip the paired-decay, fused dt_proj, ZOH, 4K and 2 x 256K prefill legs")
    ap.add_argument("--profile", action="store_true",
                    help="short run for rocprofv3: a few prefill and decode steps plus one plain "
                         "1 GiB device copy (the reference kernel for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import mamba_selective_scan_02_amd as mm
    mm.lib()  # fails loudly when the HIP library is missing
    if args.profile:
        args.copy_gbs = None
        profile_run(args, mm)
        return
    args.copy_gbs = copy_ceiling_gbs()
    pre, _ = prefill_leg(args, mm)
    line = {"metric": "mixer prefill tokens/sec at L=128K (+ decode steps/sec; % HBM peak)",
            "value": pre["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": pre["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic (seeded; Jamba-Mini-shaped widths, random weights)",
            "config": pre["config"], "roofline": headline_roofline(pre),
            "stages_ms_per_step": pre["stages_ms_per_step"], "stages": pre["stages"],
            "scan": pre["scan"], "mixer": pre["mixer"]}
    if not args.no_prefill_legs:
        legs = {}
        few = max(2, min(args.steps, 5))
        for name, kw in (("paired_decay", dict(general_a=False)),
                         ("fused_dt_proj", dict(fused_dt=True)),
                         ("zoh", dict(zoh=True)),
                         ("mini_prefill_4k", dict(workload="mini_prefill_4k", steps=args.steps)),
                         ("prefill_256k_b2", dict(workload="prefill_256k_b2", steps=few,
                                                  warmup=1))):
            kw.setdefault("steps", few)
            print(f"[bench] prefill leg {name}", file=sys.stderr, flush=True)
            leg, _ = prefill_leg(args, mm, **kw)
            legs[name] = {k: leg[k] for k in ("value", "ms_per_step", "steps", "config", "scan",
                                              "stages_ms_per_step")}
            legs[name]["unit"] = "tokens/s"
            torch.cuda.empty_cache()
        line["prefill_legs"] = legs
    if not args.no_decode:
        print("[bench] decode leg", file=sys.stderr, flush=True)
        line["decode"] = decode_leg(args, mm)
        torch.cuda.empty_cache()
        print("[bench] decode leg (wide)", file=sys.stderr, flush=True)
        line["decode_wide"] = decode_leg(args, mm, workload="decode_b256_wide")
        torch.cuda.empty_cache()
    if not args.no_layer:
        print("[bench] layer leg", file=sys.stderr, flush=True)
        line["layer"] = layer_leg(args, mm)
        torch.cuda.empty_cache()
    if not args.no_backward:
        print("[bench] backward leg", file=sys.stderr, flush=True)
        line["backward"] = backward_leg(args, mm)
        torch.cuda.empty_cache()
    if not args.no_sweep:
        print("[bench] d_state sweep", file=sys.stderr, flush=True)
        line["d_state_sweep"] = state_sweep_leg(args, mm)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.cpu_tokens)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
