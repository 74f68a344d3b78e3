"""fp64 CPU oracle of the Mamba-1 mixer core -- TEST INFRASTRUCTURE, not product code.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The HIP library never calls it, links it or falls back to it; the
two share no code (the seeded input generator in synth/ is the only module both
sides' callers use, and it holds none of the method's arithmetic).

Everything here is the plain definition, evaluated sequentially in float64 with
numpy; numpy's matmul is the only library primitive used as a step. Each function
cites the passage of the pages it follows. Sources:

  [Jamba]   "Jamba: A Hybrid Transformer-Mamba Language Model" (analysis page for
            arXiv 2403.19887), section "The Mamba Layer: State-Space Mechanism,
            Selectivity, and Parallel Scan" and section "RMSNorm definition and
            placement" / "Stabilization: RMSNorm in Mamba layers".
  [Mamba-1] The standard Mamba-1 mixer that page builds on (its reference [17]):
            causal depthwise conv1d + SiLU, x_proj / dt_proj with softplus, and the
            SiLU(z) output gate. The pages do not write these steps out; they are
            taken in their plainest form and every such reading is listed in the
            repository's design notes.

Pins (tests/test_oracle_*.py, all CPU): mpmath at 50 digits for SiLU, softplus and
RMSNorm; numpy.convolve for the convolution; scipy.signal.lfilter for a first-order
SSM; an unrolled O(L^2) cumulative-dt formula evaluated in mpmath for the scan;
scipy ODE integration of the continuous SSM for the ZOH input matrix; the closed
form h_L = exp(L*dt*A)*h_0 for zero input; chunked == sequential and
prefill == repeated decode invariants; a tiny whole-mixer fixture computed in
mpmath by a separate script (tests/golden/). The layer around the mixer (layer_f64):
residual identity with W_out = 0, linearity in W_out, and an mpmath evaluation of a tiny
layer whose mixer reduces to its D feed-through; its bf16 activation rounding (round_bf16)
against hand-worked ties and torch's float32 -> bfloat16 conversion. The gradients
(mixer_bwd_f64, the backward of the prefill): central finite differences of mixer_prefill for
every parameter, xz and both carried states (first-order and ZOH Bbar), chunk-length
independence of its state checkpoints, linearity in dy.
"""
from .mixer_f64 import (  # noqa: F401
    silu,
    softplus,
    rmsnorm,
    causal_conv1d_silu,
    x_proj,
    split_xdbl,
    dt_proj_softplus,
    selective_scan,
    mixer_prefill,
    mixer_decode_step,
    as_f64_params,
)
from .layer_f64 import layer_prefill, round_bf16  # noqa: F401,E402
from .mixer_bwd_f64 import mixer_prefill_backward  # noqa: F401,E402
