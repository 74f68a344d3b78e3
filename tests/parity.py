"""Tolerances and comparison metrics of the GPU-vs-oracle parity tests.

fp32 I/O: every output within 1e-4 absolute of the fp64 oracle (the required bar).
bf16 I/O (fp32 state): every output y_i within 2e-2 * max(|r_i|, rms(r)) of the oracle's
r_i -- a relative error of at most 2e-2 for outputs at or above the RMS of the output,
and an absolute error of at most 2e-2 * rms(r) below it. The floor is needed because the
bf16 path rounds u, dt_low and dt to bf16 (relative 2^-9 each) before they meet; the
resulting error scales with the magnitude of the terms C.h and D.u, not with their sum,
which may cancel to near zero. The conv state is a copy of inputs and must match bit for bit.
"""
import numpy as np

F32_ABS_TOL = 1e-4
BF16_REL_TOL = 2e-2


def to64(t):
    if hasattr(t, "detach"):
        return t.detach().float().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def abs_err(got, ref):
    got, ref = to64(got), to64(ref)
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def mixed_rel_err(got, ref):
    got, ref = to64(got), to64(ref)
    if not got.size:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    scale = np.maximum(np.abs(ref), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(got - ref) / scale))


def normwise_err(got, ref):
    got, ref = to64(got), to64(ref)
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (den if den > 0 else 1.0)


def check(got, ref, io_dtype: str, what: str):
    """Assert parity to the bar of the I/O dtype; returns the measured error."""
    assert np.all(np.isfinite(to64(got))), f"{what}: non-finite values"
    if io_dtype == "f32":
        e = abs_err(got, ref)
        assert e <= F32_ABS_TOL, f"{what}: max abs err {e:.3e} > {F32_ABS_TOL}"
    else:
        e = mixed_rel_err(got, ref)
        assert e <= BF16_REL_TOL, (f"{what}: mixed rel err {e:.3e} > {BF16_REL_TOL} "
                                   f"(normwise {normwise_err(got, ref):.3e})")
    return e
