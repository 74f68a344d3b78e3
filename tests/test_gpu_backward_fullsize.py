"""GPU backward at the full 128K-token workload (bf16 I/O, the launch configuration bench.py
times), checked by a property that holds at any size.

The fp64 backward oracle cannot run 131072 tokens x 8192 channels, so the gradients of
l(theta) = sum(dy * y(theta)) (the loss the backward differentiates) are checked against
directional derivatives of the same loss: for a seeded random direction V in one parameter
tensor (or in xz), (l(theta + eps V) - l(theta - eps V)) / (2 eps) must equal <grad, V>. The
loss values come from the GPU prefill in fp32 I/O on the same (exactly upcast) inputs, which
test_gpu_fullsize.py checks against the oracle at full size. l is linear in D (the difference
is exact there) and smooth elsewhere (central differences err by O(eps^2)).

V has i.i.d. N(0, s^2) entries (s = the tensor's rms), so <grad, V> has standard deviation
s |grad|; the error is measured in that unit, which does not depend on how large this one
draw of <grad, V> happens to be. The fp32 forward's rounding puts ~3e-5 .. 3e-3 of it into
the difference at eps = 1e-3 (measured, the largest for xz, whose bf16 gradient also carries
its own rounding). The bar, 1e-2, is far below the O(1) change that a wrong or missing term,
a wrong range carry, tile or split would make.
"""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

mm = pytest.importorskip("mamba_selective_scan_02_amd")

NAME = "long_prefill_128k"
EPS = 1e-3
REL_TOL = 1e-2
DIRECTIONS = ["Dskip", "A", "dt_proj_b", "x_proj_w", "dt_proj_w", "conv_w", "xz"]


def test_fullsize_backward_directional_derivatives():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = synth.CONFIGS[NAME]
    seed = synth.seed_for(NAME)
    dev = "cuda"
    print(f"[bwd-full] {NAME} B={cfg.batch} L={cfg.seqlen} D={cfg.d_inner} bf16 I/O", flush=True)
    p = synth.make_params(cfg, seed, dev)
    xz = synth.make_xz(cfg, seed, dev)
    dy = synth.make_xz(cfg, seed + 1, dev)[:, :, :cfg.d_inner].contiguous()
    g = mm.prefill_backward(xz, p, dy, eps=cfg.rms_eps)
    torch.cuda.synchronize()
    for k, v in g.items():
        if v is not None:
            assert torch.isfinite(v.float()).all(), k

    p32 = {k: (v.float() if v is not None else None) for k, v in p.items()}
    xz32 = xz.float()
    dy64 = dy.double()
    ws = mm.alloc_workspace(mm.prefill_workspace_bytes(mm.shape_of(xz32, p32, eps=cfg.rms_eps)), dev)

    def loss(params, x):
        y = mm.prefill(x, params, eps=cfg.rms_eps, workspace=ws)
        return (y.double() * dy64).sum().item()

    gen = torch.Generator(device="cpu").manual_seed(seed + 7)
    errs = {}
    for key in DIRECTIONS:
        base = xz32 if key == "xz" else p32[key]
        s = base.pow(2).mean().sqrt().item()
        V = torch.randn(base.shape, generator=gen).to(dev) * s
        grad = g["dxz" if key == "xz" else key].double()
        if key == "xz":
            lp, lm = loss(p32, xz32 + EPS * V), loss(p32, xz32 - EPS * V)
        else:
            q = dict(p32)
            q[key] = base + EPS * V
            lp = loss(q, xz32)
            q[key] = base - EPS * V
            lm = loss(q, xz32)
        gv = (grad * V.double()).sum().item()
        unit = s * grad.norm().item()          # standard deviation of <grad, V> over draws of V
        fd = (lp - lm) / (2 * EPS)
        errs[key] = abs(fd - gv) / unit
        print(f"[bwd-full] {key}: difference {fd:.6e}, <grad, V> {gv:.6e}, "
              f"error {errs[key]:.2e} of s |grad| = {unit:.4e}", flush=True)
        del V, grad
    for key, e in errs.items():
        assert e <= REL_TOL, f"{key}: directional derivative off by {e:.2e} (bar {REL_TOL})"
