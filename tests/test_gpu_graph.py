"""The decode step under HIP graph capture: a loop of decode steps captured once and replayed
several times (the states restored by eager copies between replays) gives bit-identical outputs
and states to the same steps run eagerly. The library's forward paths launch kernels only on
the caller's stream (no memset / copy nodes), so the captured graph is the kernels alone."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

mm = pytest.importorskip("mamba_selective_scan_02_amd")


@pytest.mark.parametrize("K", [4, 3])
def test_decode_loop_graph_replays_match_eager(K):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = synth.MixerConfig(f"graph_dec_K{K}", 64, 1, 1024, 16, K, 128, "bf16")
    seed, steps, dev = 500 + K, 12, "cuda"
    print(f"[graph] decode B={cfg.batch} D={cfg.d_inner} K={K} steps={steps}", flush=True)
    p = synth.make_params(cfg, seed, dev, conv_bias=True)
    cs0, ss0 = synth.make_states(cfg, seed, dev)
    xs = synth.make_xz(cfg, seed, dev, seqlen=steps, tensor="decode_xz").transpose(0, 1).contiguous()
    shape = mm.shape_of(xs[0], p, decode=True)
    ws = mm.alloc_workspace(mm.decode_workspace_bytes(shape), xs.device)
    # eager reference
    cs, ss = cs0.clone(), ss0.clone()
    ys_e = torch.empty(steps, cfg.batch, cfg.d_inner, dtype=cfg.torch_dtype, device=dev)
    for i in range(steps):
        mm.decode_step(xs[i], p, cs, ss, y=ys_e[i], workspace=ws)
    torch.cuda.synchronize()
    cs_e, ss_e = cs.clone(), ss.clone()
    # capture
    cs_g, ss_g = cs0.clone(), ss0.clone()
    ys_g = torch.zeros_like(ys_e)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                mm.decode_step(xs[i], p, cs_g, ss_g, y=ys_g[i], workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        cs_g.copy_(cs0)
        ss_g.copy_(ss0)
        ys_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys_g, ys_e), f"replay {rep}: y"
        assert torch.equal(cs_g, cs_e), f"replay {rep}: conv_state"
        assert torch.equal(ss_g, ss_e), f"replay {rep}: ssm_state"
        # eager work of the program between replays
        mm.decode_step(xs[0], p, cs.clone(), ss.clone(), workspace=ws)
