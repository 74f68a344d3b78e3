"""Tolerances and comparison metrics of the GPU-vs-oracle parity tests.

fp32 I/O: every output within 1e-4 absolute of the fp64 oracle (the required bar).
bf16 I/O (fp32 state): every output y_i satisfies
    |y_i - r_i| <= 2e-2 * max(|r_i|, 0.01 * rms(r)),
i.e. a relative error of at most 2e-2 down to one hundredth of the output's RMS, and an
absolute error of at most 2e-4 * rms(r) below that (the floor only keeps the ratio finite
where r_i is zero). Every check also records the same ratio with the floor at rms(r) itself
(a looser figure, kept for comparison) and the normwise error max|y - r| / max|r|; the
session prints all three per check at the end (tests/conftest.py).
The conv state is a copy of inputs and must match bit for bit.
"""
import numpy as np

F32_ABS_TOL = 1e-4
BF16_REL_TOL = 2e-2
BF16_FLOOR = 0.01        # floor of the denominator, as a fraction of rms(r)

# (what, io dtype, error at the 0.01 rms floor (fp32: max abs), rms-floor error, normwise error,
# the asserted error) of every check this session
RECORDS = []


def to64(t):
    if hasattr(t, "detach"):
        return t.detach().float().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def abs_err(got, ref):
    got, ref = to64(got), to64(ref)
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def mixed_rel_err(got, ref, floor=BF16_FLOOR):
    """max_i |got_i - ref_i| / max(|ref_i|, floor * rms(ref)); 0 for empty inputs, and the
    plain absolute error when ref is identically zero."""
    got, ref = to64(got), to64(ref)
    if not got.size:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.max(np.abs(got - ref)))
    scale = np.maximum(np.abs(ref), floor * rms)
    return float(np.max(np.abs(got - ref) / scale))


def normwise_err(got, ref):
    got, ref = to64(got), to64(ref)
    if not got.size:
        return 0.0
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (den if den > 0 else 1.0)


def check(got, ref, io_dtype: str, what: str, f32_large_outputs: bool = False,
          bf16_floor: float = BF16_FLOOR):
    """Assert parity to the bar of the I/O dtype; returns the measured (asserted) error.

    bf16_floor: the floor of the relative bar as a fraction of rms(ref); 0.01 everywhere except
    the Mamba layer's bf16 output (tests/test_gpu_layer.py states why it takes rms(ref)).

    f32_large_outputs (edge cases only): outputs far above order one (steps dt of 12 to 40 give
    |y| in the thousands) hold the fp32 bar relative to the largest output,
    max|got - ref| <= 1e-4 * max(1, max|ref|), since fp32 itself rounds at 6e-8 |ref|; at
    max|ref| <= 1 this is the absolute bar."""
    g = to64(got)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    r = to64(ref)
    if io_dtype == "f32":
        e = abs_err(g, r)
        if f32_large_outputs and r.size:
            e /= max(1.0, float(np.max(np.abs(r))))
        RECORDS.append((what, io_dtype, e, None, normwise_err(g, r), e))
        assert e <= F32_ABS_TOL, f"{what}: max abs err {e:.3e} > {F32_ABS_TOL}"
    else:
        e01 = mixed_rel_err(g, r)
        e_rms = mixed_rel_err(g, r, floor=1.0)
        e = mixed_rel_err(g, r, floor=bf16_floor)
        nw = normwise_err(g, r)
        RECORDS.append((what if bf16_floor == BF16_FLOOR else f"{what} [asserted at floor "
                        f"{bf16_floor:g} rms: {e:.3e}]", io_dtype, e01, e_rms, nw, e))
        assert e <= BF16_REL_TOL, (f"{what}: rel err {e:.3e} (floor {bf16_floor:g} rms) > "
                                   f"{BF16_REL_TOL} (floor 0.01 rms {e01:.3e}, floor rms "
                                   f"{e_rms:.3e}, normwise {nw:.3e})")
    return e
