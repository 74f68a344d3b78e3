"""Seeded synthetic inputs for the Mamba-1 mixer core.

This module is shared by the tests, the benchmark and the smoke check. It only
draws random numbers and lays them out; it holds none of the mixer's arithmetic
(no convolution, projection, normalisation, softplus, scan or gate), so that the
fp64 oracle and the HIP library never share a line of the method.

Workloads (shapes follow the Jamba-Mini-shaped mixer; the pages give d_state = 16
in "Why Mamba matters for Jamba" on the Jamba analysis page and no other width):

  tiny_f32            B=1,   L=256,    D=64,    N=16, K=4, R=8,   fp32 I/O
  mini_prefill_4k     B=1,   L=4096,   D=8192,  N=16, K=4, R=256, bf16 I/O
  long_prefill_128k   B=1,   L=131072, D=8192,  N=16, K=4, R=256, bf16 I/O
  prefill_256k_b2     B=2,   L=262144, D=8192,  N=16, K=4, R=256, bf16 I/O
  decode_b256         B=256, 512 steps, D=8192,  R=256 (states from a 1024-token prefill)
  decode_b256_wide    B=256, 512 steps, D=16384, R=512

Value recipe (same for every workload, widths scaled):
  xz              ~ N(0, 1), rounded to the I/O dtype (bf16 by round-to-nearest-even)
  conv_w          ~ U(-0.5, 0.5)             [D, K]; conv_b absent unless asked for
  x_proj_w        ~ N(0, 1/D)                [R + 2N, D]   rows = [dt_low | B | C]
  dt_proj_w       ~ N(0, 1/R)                [D, R]
  dt_proj_b       = inverse-softplus(dt0), dt0 = exp(U(ln 1e-3, ln 1e-1))   (fp32)
  A[i, n]         = -(n + 1)                 (S4D-real; fp32, all negative)
  Dskip           = 1                        (fp32)
  norm weights    = 1 (or U(0.5, 1.5) when gamma_random)
Edge-case options of make_params (parity tests only; the workloads use the recipe above):
  a_random        A[i, n] = -exp(U(-2, 3)) per (channel, state): decay rates from 0.14 to 20
  dt_range        (lo, hi): dt0 log-uniform in [lo, hi] instead of [1e-3, 1e-1] (large values
                  push dt_proj's pre-activation past softplus's linear-branch thresholds and
                  exp(dt A) to underflow; tiny ones give steps near 1e-7)
  d_random        Dskip ~ U(-1, 2)
Random numbers come from torch.Generator seeded per tensor, on the device the
tensor is made on; a test that compares two implementations feeds both the very
same tensors (copied, never regenerated).
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class MixerConfig:
    name: str
    batch: int
    seqlen: int
    d_inner: int
    d_state: int = 16
    d_conv: int = 4
    dt_rank: int = 256
    io_dtype: str = "bf16"          # "bf16" or "f32"
    rms_eps: float = 1e-6
    decode_steps: int = 0           # > 0 marks a decode workload
    decode_prefix: int = 0          # length of the prefill that seeds decode states
    d_model: int = 4096             # hidden size around the mixer (layer entry point only)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.io_dtype == "bf16" else torch.float32

    @property
    def xdbl_width(self) -> int:
        return self.dt_rank + 2 * self.d_state

    def with_(self, **kw) -> "MixerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny_f32": MixerConfig("tiny_f32", 1, 256, 64, 16, 4, 8, "f32"),
    "mini_prefill_4k": MixerConfig("mini_prefill_4k", 1, 4096, 8192, 16, 4, 256, "bf16"),
    "long_prefill_128k": MixerConfig("long_prefill_128k", 1, 131072, 8192, 16, 4, 256, "bf16"),
    "prefill_256k_b2": MixerConfig("prefill_256k_b2", 2, 262144, 8192, 16, 4, 256, "bf16"),
    "decode_b256": MixerConfig("decode_b256", 256, 1, 8192, 16, 4, 256, "bf16",
                               decode_steps=512, decode_prefix=1024),
    "decode_b256_wide": MixerConfig("decode_b256_wide", 256, 1, 16384, 16, 4, 512, "bf16",
                                    decode_steps=512, decode_prefix=1024),
}

# Tensor ids keep the streams of different tensors apart for one seed.
_TID = {"xz": 1, "conv_w": 2, "conv_b": 3, "x_proj_w": 4, "dt_proj_w": 5, "dt0": 6,
        "gamma": 7, "conv_state": 8, "ssm_state": 9, "decode_xz": 10, "misc": 11,
        "layer_x": 12, "in_proj_w": 13, "out_proj_w": 14, "norm_w": 15, "A": 16, "Dskip": 17}


def generator(seed: int, tensor: str, device, step: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + _TID[tensor] * 7919 + step * 104729) & ((1 << 62) - 1))
    return g


def _normal(shape, std, g, device, dtype):
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=g)
    return t.to(dtype)


def _uniform(shape, lo, hi, g, device, dtype=torch.float32):
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.uniform_(lo, hi, generator=g)
    return t.to(dtype)


def make_params(cfg: MixerConfig, seed: int, device="cpu", *, conv_bias: bool = False,
                gamma_random: bool = False, a_random: bool = False,
                dt_range: tuple = (1e-3, 1e-1), d_random: bool = False) -> dict:
    """Parameters of one mixer, laid out as the C ABI takes them."""
    D, N, K, R = cfg.d_inner, cfg.d_state, cfg.d_conv, cfg.dt_rank
    dt = cfg.torch_dtype
    p = {}
    p["conv_w"] = _uniform((D, K), -0.5, 0.5, generator(seed, "conv_w", device), device, dt)
    p["conv_b"] = (_uniform((D,), -0.5, 0.5, generator(seed, "conv_b", device), device, dt)
                   if conv_bias else None)
    p["x_proj_w"] = _normal((R + 2 * N, D), 1.0 / math.sqrt(D),
                            generator(seed, "x_proj_w", device), device, dt)
    p["dt_proj_w"] = _normal((D, R), 1.0 / math.sqrt(R),
                             generator(seed, "dt_proj_w", device), device, dt)
    # dt0 log-uniform in dt_range ([1e-3, 1e-1] in the workloads); the bias is its inverse
    # softplus, so that the projection's bias alone maps to dt0 (evaluated in float64).
    lo, hi = math.log(dt_range[0]), math.log(dt_range[1])
    u = _uniform((D,), 0.0, 1.0, generator(seed, "dt0", device), device, torch.float64)
    dt0 = torch.exp(lo + u * (hi - lo))
    p["dt_proj_b"] = (dt0 + torch.log(-torch.expm1(-dt0))).to(torch.float32)
    if a_random:
        la = _uniform((D, N), -2.0, 3.0, generator(seed, "A", device), device, torch.float64)
        p["A"] = (-torch.exp(la)).to(torch.float32).contiguous()
    else:
        p["A"] = (-torch.arange(1, N + 1, dtype=torch.float32, device=device)).repeat(D, 1).contiguous()
    p["Dskip"] = (_uniform((D,), -1.0, 2.0, generator(seed, "Dskip", device), device)
                  if d_random else torch.ones(D, dtype=torch.float32, device=device))
    if gamma_random:
        g = generator(seed, "gamma", device)
        p["dt_norm_w"] = _uniform((R,), 0.5, 1.5, g, device)
        p["B_norm_w"] = _uniform((N,), 0.5, 1.5, g, device)
        p["C_norm_w"] = _uniform((N,), 0.5, 1.5, g, device)
    else:
        p["dt_norm_w"] = torch.ones(R, dtype=torch.float32, device=device)
        p["B_norm_w"] = torch.ones(N, dtype=torch.float32, device=device)
        p["C_norm_w"] = torch.ones(N, dtype=torch.float32, device=device)
    return p


def make_xz(cfg: MixerConfig, seed: int, device="cpu", *, batch=None, seqlen=None,
            tensor: str = "xz", step: int = 0, chunk_tokens: int = 1 << 14) -> torch.Tensor:
    """xz ~ N(0, 1) of shape [B, L, 2D] in the I/O dtype, drawn in token chunks so that
    a 17 GB bf16 tensor never needs an fp32 copy of itself."""
    B = cfg.batch if batch is None else batch
    L = cfg.seqlen if seqlen is None else seqlen
    D2 = 2 * cfg.d_inner
    out = torch.empty((B, L, D2), dtype=cfg.torch_dtype, device=device)
    g = generator(seed, tensor, device, step)
    for b in range(B):
        for t0 in range(0, L, chunk_tokens):
            t1 = min(L, t0 + chunk_tokens)
            tmp = torch.empty((t1 - t0, D2), dtype=torch.float32, device=device)
            tmp.normal_(0.0, 1.0, generator=g)
            out[b, t0:t1] = tmp.to(cfg.torch_dtype)
    return out


def make_states(cfg: MixerConfig, seed: int, device="cpu", *, batch=None,
                scale: float = 1.0):
    """Random carried states: conv_state [B, D, K-1] (I/O dtype) and ssm_state
    [B, D, N] (fp32), both ~ N(0, scale^2)."""
    B = cfg.batch if batch is None else batch
    D, N, K = cfg.d_inner, cfg.d_state, cfg.d_conv
    cs = _normal((B, D, K - 1), scale, generator(seed, "conv_state", device), device,
                 cfg.torch_dtype)
    ss = _normal((B, D, N), scale, generator(seed, "ssm_state", device), device, torch.float32)
    return cs, ss


def seed_for(cfg_name: str) -> int:
    """Fixed seed per workload: 1000 + its position in CONFIGS."""
    return 1000 + list(CONFIGS).index(cfg_name)


def make_layer(cfg: MixerConfig, seed: int, device="cpu", *, gamma_random: bool = False) -> dict:
    """Weights of the layer around the mixer: in_proj [2 d_inner, d_model] ~ N(0, 1/d_model) and
    out_proj [d_model, d_inner] ~ N(0, 1/d_inner) in the I/O dtype; the input RMSNorm gain
    (fp32) is 1, or U(0.5, 1.5)."""
    D, Dm, dt = cfg.d_inner, cfg.d_model, cfg.torch_dtype
    lay = {"in_proj_w": _normal((2 * D, Dm), 1.0 / math.sqrt(Dm),
                                generator(seed, "in_proj_w", device), device, dt),
           "out_proj_w": _normal((Dm, D), 1.0 / math.sqrt(D),
                                 generator(seed, "out_proj_w", device), device, dt)}
    lay["norm_w"] = (_uniform((Dm,), 0.5, 1.5, generator(seed, "norm_w", device), device)
                     if gamma_random else torch.ones(Dm, dtype=torch.float32, device=device))
    return lay


def make_layer_x(cfg: MixerConfig, seed: int, device="cpu", *, batch=None, seqlen=None,
                 chunk_tokens: int = 1 << 14) -> torch.Tensor:
    """Layer input x ~ N(0, 1), [B, L, d_model] in the I/O dtype, drawn in token chunks."""
    B = cfg.batch if batch is None else batch
    L = cfg.seqlen if seqlen is None else seqlen
    out = torch.empty((B, L, cfg.d_model), dtype=cfg.torch_dtype, device=device)
    g = generator(seed, "layer_x", device)
    for b in range(B):
        for t0 in range(0, L, chunk_tokens):
            t1 = min(L, t0 + chunk_tokens)
            tmp = torch.empty((t1 - t0, cfg.d_model), dtype=torch.float32, device=device)
            tmp.normal_(0.0, 1.0, generator=g)
            out[b, t0:t1] = tmp.to(cfg.torch_dtype)
    return out
