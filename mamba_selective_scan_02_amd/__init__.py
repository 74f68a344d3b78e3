"""Python binding of the gfx950 Mamba-1 mixer-core library (libmamba_mixer.so).

Argument marshalling only: every step of the mixer runs in the library's HIP kernels.
torch supplies device memory (outputs and workspace are allocated with torch when the
caller does not pass them) and the current HIP stream. There is no CPU fallback: when
the library is missing, importing the entry points raises.

    from mamba_selective_scan_02_amd import prefill, decode_step
    y, conv_state, ssm_state = prefill(xz, params, return_states=True)
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmamba_mixer.so")

MM_OK, MM_ERR_INVALID_ARG, MM_ERR_UNSUPPORTED, MM_ERR_WORKSPACE, MM_ERR_HIP = 0, -1, -2, -3, -4
MM_F32, MM_BF16 = 0, 1
MM_FLAG_ZOH_B = 1
MM_FLAG_SCAN_SEQUENTIAL = 2
MM_FLAG_SCAN_CHUNKED = 4
MM_FLAG_SCAN_GENERAL_A = 8
MM_FLAG_FUSED_DTPROJ = 16
STAGES = ("conv_silu", "x_proj", "rmsnorm", "dt_proj_softplus", "selective_scan", "conv_state",
          "layer_rmsnorm", "in_proj", "out_proj", "bwd_recompute", "bwd_scan", "bwd_proj",
          "bwd_conv")
GRAD_NAMES = ("dxz", "conv_w", "conv_b", "x_proj_w", "dt_proj_w", "dt_proj_b", "A", "Dskip",
              "dt_norm_w", "B_norm_w", "C_norm_w", "conv_state", "ssm_state")


class MixerError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_status_string(status)} ({status})")


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("d_inner", ctypes.c_int32), ("d_state", ctypes.c_int32),
                ("d_conv", ctypes.c_int32), ("dt_rank", ctypes.c_int32),
                ("io_dtype", ctypes.c_int), ("rms_eps", ctypes.c_float),
                ("flags", ctypes.c_uint32)]


class Params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("conv_w", "conv_b", "x_proj_w", "dt_proj_w", "dt_proj_b", "A", "Dskip",
                 "dt_norm_w", "B_norm_w", "C_norm_w")]


class LayerParams(ctypes.Structure):
    _fields_ = [("norm_w", ctypes.c_void_p), ("in_proj_w", ctypes.c_void_p),
                ("out_proj_w", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
                ("mixer", Params)]


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_NAMES]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (python -m ...build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m mamba_selective_scan_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, S, I, V, Z = ctypes.POINTER, Shape, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        for name, args, res in [
            ("mm_prefill_workspace_bytes", [P(S)], Z),
            ("mm_decode_workspace_bytes", [P(S)], Z),
            ("mamba_mixer_prefill", [P(S), P(Params), V, V, V, V, I, V, Z, V], I),
            ("mamba_mixer_prefill_timed", [P(S), P(Params), V, V, V, V, I, V, Z, V, V], I),
            ("mamba_mixer_decode_step", [P(S), P(Params), V, V, V, V, V, Z, V], I),
            ("mamba_mixer_decode_step_timed", [P(S), P(Params), V, V, V, V, V, Z, V, V], I),
            ("mm_noalloc_scratch_bytes", [], Z),
            ("mamba_mixer_decode_step_noalloc", [P(S), P(Params), V, V, V, V, V], I),
            ("mm_stage_timer_create", [], V),
            ("mm_stage_timer_destroy", [V], None),
            ("mm_stage_timer_reset", [V], None),
            ("mm_stage_timer_read", [V, P(ctypes.c_double), P(ctypes.c_int64)], I),
            ("mm_stage_name", [I], ctypes.c_char_p),
            ("mm_status_string", [I], ctypes.c_char_p),
            ("mm_abi_version", [], I),
            ("mm_layer_workspace_bytes", [P(S), I], Z),
            ("mamba_layer_prefill", [P(S), I, P(LayerParams), V, V, V, V, I, V, Z, V], I),
            ("mamba_layer_prefill_timed", [P(S), I, P(LayerParams), V, V, V, V, I, V, Z, V, V], I),
            ("mm_backward_workspace_bytes", [P(S)], Z),
            ("mamba_mixer_prefill_backward", [P(S), P(Params), V, V, V, V, I, P(Grads), V, Z, V], I),
            ("mamba_mixer_prefill_backward_timed",
             [P(S), P(Params), V, V, V, V, I, P(Grads), V, Z, V, V], I),
        ]:
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _status_string(st: int) -> str:
    try:
        return lib().mm_status_string(st).decode()
    except ImportError:
        return "unknown"


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _io_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return MM_BF16
    if dtype == torch.float32:
        return MM_F32
    raise TypeError(f"unsupported I/O dtype {dtype} (bfloat16 or float32)")


def make_shape(batch, seqlen, d_inner, d_state, d_conv, dt_rank, dtype, eps=1e-6, flags=0) -> Shape:
    return Shape(batch, seqlen, d_inner, d_state, d_conv, dt_rank, _io_code(dtype), eps, flags)


def shape_of(xz: torch.Tensor, params: dict, *, decode=False, eps=1e-6, zoh=False,
             scan: str | None = None, general_a: bool = False, fused_dt: bool = False) -> Shape:
    if decode:
        B, D2 = xz.shape
        L = 1
    else:
        B, L, D2 = xz.shape
    D = D2 // 2
    N = params["A"].shape[1]
    K = params["conv_w"].shape[1]
    R = params["dt_proj_w"].shape[1]
    flags = MM_FLAG_ZOH_B if zoh else 0
    if scan is not None:
        flags |= {"sequential": MM_FLAG_SCAN_SEQUENTIAL, "chunked": MM_FLAG_SCAN_CHUNKED}[scan]
    if general_a:
        flags |= MM_FLAG_SCAN_GENERAL_A
    if fused_dt:
        flags |= MM_FLAG_FUSED_DTPROJ
    return make_shape(B, L, D, N, K, R, xz.dtype, eps, flags)


def params_struct(params: dict) -> Params:
    return Params(*[_ptr(params.get(n)) for n in
                    ("conv_w", "conv_b", "x_proj_w", "dt_proj_w", "dt_proj_b", "A", "Dskip",
                     "dt_norm_w", "B_norm_w", "C_norm_w")])


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def prefill_workspace_bytes(shape: Shape) -> int:
    return int(lib().mm_prefill_workspace_bytes(ctypes.byref(shape)))


def decode_workspace_bytes(shape: Shape) -> int:
    return int(lib().mm_decode_workspace_bytes(ctypes.byref(shape)))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


class StageTimer:
    """Per-stage HIP-event timer of the *_timed entry points (see mm_stage_timer_*)."""

    def __init__(self):
        self.h = lib().mm_stage_timer_create()

    def reset(self):
        lib().mm_stage_timer_reset(self.h)

    def read(self) -> dict:
        ms = (ctypes.c_double * len(STAGES))()
        n = (ctypes.c_int64 * len(STAGES))()
        st = lib().mm_stage_timer_read(self.h, ms, n)
        if st != MM_OK:
            raise MixerError(st, "mm_stage_timer_read")
        return {STAGES[i]: (ms[i], n[i]) for i in range(len(STAGES))}

    def __del__(self):
        try:
            if getattr(self, "h", None):
                lib().mm_stage_timer_destroy(self.h)
                self.h = None
        except Exception:
            pass


def prefill(xz, params, *, conv_state=None, ssm_state=None, states_valid=False, y=None,
            workspace=None, eps=1e-6, zoh=False, stream=None, timer: StageTimer | None = None,
            scan: str | None = None, general_a: bool = False, fused_dt: bool = False):
    """Run mamba_mixer_prefill. xz [B, L, 2D] (bf16 or fp32, on the GPU); conv_state
    [B, D, K-1] and ssm_state [B, D, N] are updated in place when given. scan = None picks
    the scan kernel by size; "sequential" / "chunked" force one. general_a sets
    MM_FLAG_SCAN_GENERAL_A (every exp(dt A) evaluated directly); fused_dt sets
    MM_FLAG_FUSED_DTPROJ (dt_proj inside the scan where it applies). Returns y."""
    shape = shape_of(xz, params, eps=eps, zoh=zoh, scan=scan, general_a=general_a,
                     fused_dt=fused_dt)
    if y is None:
        y = torch.empty(xz.shape[:-1] + (shape.d_inner,), dtype=xz.dtype, device=xz.device)
    need = prefill_workspace_bytes(shape)
    if workspace is None:
        workspace = alloc_workspace(need, xz.device)
    p = params_struct(params)
    args = (ctypes.byref(shape), ctypes.byref(p), _ptr(xz), _ptr(y), _ptr(conv_state),
            _ptr(ssm_state), 1 if states_valid else 0, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if timer is None:
        st = lib().mamba_mixer_prefill(*args)
    else:
        st = lib().mamba_mixer_prefill_timed(*args, timer.h)
    if st != MM_OK:
        raise MixerError(st, "mamba_mixer_prefill")
    return y


def decode_step(xz, params, conv_state, ssm_state, *, y=None, workspace=None, eps=1e-6,
                zoh=False, stream=None, timer: StageTimer | None = None):
    """Run mamba_mixer_decode_step on xz [B, 2D]; states are updated in place. Returns y [B, D]."""
    shape = shape_of(xz, params, decode=True, eps=eps, zoh=zoh)
    if y is None:
        y = torch.empty((xz.shape[0], shape.d_inner), dtype=xz.dtype, device=xz.device)
    need = decode_workspace_bytes(shape)
    if workspace is None:
        workspace = alloc_workspace(need, xz.device)
    p = params_struct(params)
    args = (ctypes.byref(shape), ctypes.byref(p), _ptr(xz), _ptr(y), _ptr(conv_state),
            _ptr(ssm_state), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream))
    if timer is None:
        st = lib().mamba_mixer_decode_step(*args)
    else:
        st = lib().mamba_mixer_decode_step_timed(*args, timer.h)
    if st != MM_OK:
        raise MixerError(st, "mamba_mixer_decode_step")
    return y


def decode_step_noalloc(xz, params, conv_state, ssm_state, *, y, eps=1e-6, zoh=False,
                        stream=None):
    """Run mamba_mixer_decode_step_noalloc (no workspace: the library's per-GPU scratch) on
    xz [B, 2D] into the caller's y [B, D]; states are updated in place. Returns y."""
    shape = shape_of(xz, params, decode=True, eps=eps, zoh=zoh)
    p = params_struct(params)
    st = lib().mamba_mixer_decode_step_noalloc(ctypes.byref(shape), ctypes.byref(p), _ptr(xz),
                                               _ptr(y), _ptr(conv_state), _ptr(ssm_state),
                                               _stream(stream))
    if st != MM_OK:
        raise MixerError(st, "mamba_mixer_decode_step_noalloc")
    return y


def layer_workspace_bytes(shape: Shape, d_model: int) -> int:
    return int(lib().mm_layer_workspace_bytes(ctypes.byref(shape), d_model))


def layer_prefill(x, params, layer, *, conv_state=None, ssm_state=None, states_valid=False,
                  out=None, workspace=None, eps=1e-6, norm_eps=1e-6, zoh=False, stream=None,
                  timer: StageTimer | None = None):
    """Run mamba_layer_prefill: out = x + W_out . mixer(W_in . RMSNorm(x)). x [B, L, d_model]
    bf16; params: the mixer's parameters; layer: {"norm_w", "in_proj_w", "out_proj_w"}."""
    B, L, Dm = x.shape
    D = params["Dskip"].shape[0]
    N = params["A"].shape[1]
    K = params["conv_w"].shape[1]
    R = params["dt_proj_w"].shape[1]
    shape = make_shape(B, L, D, N, K, R, x.dtype, eps, MM_FLAG_ZOH_B if zoh else 0)
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(layer_workspace_bytes(shape, Dm), x.device)
    lp = LayerParams(_ptr(layer["norm_w"]), _ptr(layer["in_proj_w"]), _ptr(layer["out_proj_w"]),
                     norm_eps, params_struct(params))
    args = (ctypes.byref(shape), Dm, ctypes.byref(lp), _ptr(x), _ptr(out), _ptr(conv_state),
            _ptr(ssm_state), 1 if states_valid else 0, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if timer is None:
        st = lib().mamba_layer_prefill(*args)
    else:
        st = lib().mamba_layer_prefill_timed(*args, timer.h)
    if st != MM_OK:
        raise MixerError(st, "mamba_layer_prefill")
    return out


def backward_workspace_bytes(shape: Shape) -> int:
    n = lib().mm_backward_workspace_bytes(ctypes.byref(shape))
    if n == 0:
        raise MixerError(MM_ERR_UNSUPPORTED, "mm_backward_workspace_bytes")
    return n


def prefill_backward(xz, params, dy, *, conv_state=None, ssm_state=None, states_valid=False,
                     grads: dict | None = None, state_grads=True, workspace=None, eps=1e-6,
                     zoh=False, stream=None, timer: StageTimer | None = None) -> dict:
    """Run mamba_mixer_prefill_backward: gradients of sum(dy * y) for y = prefill(xz, params,
    conv_state, ssm_state) (states as they were before the forward). Returns a dict with the
    keys of GRAD_NAMES (dxz in the I/O dtype, the rest float32; conv_b None without a conv
    bias; the state gradients None when state_grads is False)."""
    shape = shape_of(xz, params, eps=eps, zoh=zoh)
    B, L, D2 = xz.shape
    D, K, R = D2 // 2, params["conv_w"].shape[1], params["dt_proj_w"].shape[1]
    N = params["A"].shape[1]
    f32 = dict(dtype=torch.float32, device=xz.device)
    if grads is None:
        grads = {"dxz": torch.empty_like(xz), "conv_w": torch.empty(D, K, **f32),
                 "conv_b": (torch.empty(D, **f32) if params.get("conv_b") is not None else None),
                 "x_proj_w": torch.empty(R + 2 * N, D, **f32), "dt_proj_w": torch.empty(D, R, **f32),
                 "dt_proj_b": torch.empty(D, **f32), "A": torch.empty(D, N, **f32),
                 "Dskip": torch.empty(D, **f32), "dt_norm_w": torch.empty(R, **f32),
                 "B_norm_w": torch.empty(N, **f32), "C_norm_w": torch.empty(N, **f32),
                 "conv_state": torch.empty(B, D, K - 1, **f32) if state_grads else None,
                 "ssm_state": torch.empty(B, D, N, **f32) if state_grads else None}
    if workspace is None:
        workspace = alloc_workspace(backward_workspace_bytes(shape), xz.device)
    g = Grads(*[_ptr(grads.get(n)) for n in GRAD_NAMES])
    args = (ctypes.byref(shape), ctypes.byref(params_struct(params)), _ptr(xz), _ptr(dy),
            _ptr(conv_state), _ptr(ssm_state), 1 if states_valid else 0, ctypes.byref(g),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if timer is None:
        st = lib().mamba_mixer_prefill_backward(*args)
    else:
        st = lib().mamba_mixer_prefill_backward_timed(*args, timer.h)
    if st != MM_OK:
        raise MixerError(st, "mamba_mixer_prefill_backward")
    return grads
