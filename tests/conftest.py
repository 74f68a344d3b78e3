import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Every parity check of the session with its measured errors: the asserted one (fp32:
    max abs; bf16: relative with the floor at 0.01 rms), the bf16 ratio with the floor at rms,
    and the normwise error."""
    try:
        from tests.parity import RECORDS
    except ImportError:
        return
    if not RECORDS:
        return
    tr = terminalreporter
    tr.write_sep("-", f"parity checks ({len(RECORDS)})")
    worst = {}
    for what, io, e, e_rms, nw, asserted in RECORDS:
        rms_s = "-" if e_rms is None else f"{e_rms:.3e}"
        tr.write_line(f"{io:5s} err {e:.3e}  rms-floor {rms_s:>9s}  normwise {nw:.3e}  {what}")
        worst[io] = max(worst.get(io, 0.0), asserted)
    tr.write_line("worst asserted error (bars: bf16 2e-2 relative, f32 1e-4): " +
                  ", ".join(f"{k} {v:.3e}" for k, v in sorted(worst.items())))
