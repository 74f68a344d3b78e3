"""The allocation-free decode step (mamba_mixer_decode_step_noalloc: the library's per-GPU
scratch array instead of a workspace argument) against mamba_mixer_decode_step, through the C
ABI: outputs and both updated states bit for bit (the same kernels), on two calls in a row, the
second with a smaller batch; a shape whose decode workspace exceeds the scratch is rejected
before anything is launched."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

mm = pytest.importorskip("mamba_selective_scan_02_amd")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _one(cfg, seed):
    dev = "cuda"
    p = synth.make_params(cfg, seed, dev, conv_bias=True, gamma_random=True)
    cs, ss = synth.make_states(cfg, seed, dev)
    xt = synth.make_xz(cfg, seed, dev, seqlen=1, tensor="decode_xz")[:, 0].contiguous()
    cs2, ss2 = cs.clone(), ss.clone()
    y_ref = mm.decode_step(xt, p, cs, ss)
    y = torch.empty_like(y_ref)
    mm.decode_step_noalloc(xt, p, cs2, ss2, y=y)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), "y differs from mamba_mixer_decode_step"
    assert torch.equal(cs2, cs), "conv_state differs"
    assert torch.equal(ss2, ss), "ssm_state differs"


@pytest.mark.parametrize("K", [4, 3])
def test_noalloc_decode_matches_decode_step(K):
    _need_gpu()
    print(f"[noalloc] d_conv={K}", flush=True)
    # the fused decode kernels (d_conv 4) and the general path (d_conv 3); the second call has
    # fewer sequences, so it reuses the scratch left by a larger one
    _one(synth.MixerConfig("noalloc_big", 256, 1, 8192, 16, K, 256, "bf16"), 900 + K)
    _one(synth.MixerConfig("noalloc_small", 37, 1, 1024, 16, K, 64, "bf16"), 910 + K)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    _need_gpu()
    limit = mm.lib().mm_noalloc_scratch_bytes()
    shape = mm.make_shape(4096, 1, 16384, 16, 4, 512, torch.bfloat16)
    assert mm.decode_workspace_bytes(shape) > limit
    fake = 0x100000
    p = mm.Params(*([fake] * 10))
    st = mm.lib().mamba_mixer_decode_step_noalloc(mm.ctypes.byref(shape), mm.ctypes.byref(p),
                                                  fake, 2 * fake, 3 * fake, 4 * fake, None)
    assert st == mm.MM_ERR_WORKSPACE
