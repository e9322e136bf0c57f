"""The forward pass under HIP graph capture: the C ABI allocates nothing,
never synchronises and records no memset, so a captured pass can be
replayed.  Each replay (with eager work and new inputs between replays) must
give the bytes of the eager pass on the same inputs."""
import numpy as np
import pytest
import torch

import expert_dispatch_router_amd as moe
from expert_dispatch_router_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,opts", [("tiny", {}), ("mixtral_128", {}),
                                       ("qwen2_128", {"routing_kernels": 2}),
                                       ("tiny", {"gather_mode": 2, "split_k": 2}),
                                       ("tiny", {"fold_combine": 2, "split_k": 2, "fuse_down": 1}),
                                       ("mixtral_128", {"fold_combine": 2}),
                                       ("tiny", {"fuse_down": 2}),
                                       # two-launch routing, the 64-column-per-wave down tile
                                       ("qwen2_128", {}), ("skewed_256", {}),
                                       ("qwen2_128", {"routing_kernels": 3, "xcd_order": 2}),
                                       # the stream-K gate/up schedule: unit counters cleared
                                       # by the routing kernels on every replay
                                       ("skewed_128", {"schedule": 2}),
                                       ("qwen2_128", {"schedule": 2, "routing_kernels": 2}),
                                       # the variable-size gate/up table: merged by the rule
                                       # (skewed T=512), always (schedule 3, one-workgroup
                                       # routing), and not merged (skewed T=128)
                                       ("skewed_512", {}), ("skewed_128", {}),
                                       ("skewed_128", {"schedule": 3, "routing_kernels": 1})])
def test_forward_graph_replays_match_eager(name, opts):
    cfg = synth.CONFIGS[name]
    x, lg, wgu, wd = synth.make_inputs(cfg, 0, DEV)
    score = "sigmoid" if cfg.score else "softmax"
    out = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(moe.moe_workspace_size(cfg.T, cfg.d, cfg.ffn, cfg.E, cfg.top_k, **opts),
                     dtype=torch.uint8, device=DEV)
    fwd = lambda o, w: moe.moe_forward(x, lg, wgu, wd, cfg.top_k, cfg.renormalize, out=o,
                                       score=score, workspace=w, **opts)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd(out, ws)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(out, ws)
    gen = torch.Generator(device="cpu").manual_seed(7)
    for rep in range(4):
        if rep >= 2:  # new routing inputs in the captured buffer
            lg.copy_(torch.randn(lg.shape, generator=gen).to(DEV))
        eager = fwd(torch.empty_like(out), torch.empty_like(ws))
        torch.cuda.synchronize()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
    toks = np.unique(np.linspace(0, cfg.T - 1, 8).astype(np.int32))
    ref = parity.oracle_out(x, lg, wgu, wd, cfg.top_k, cfg.score, cfg.renormalize, tokens=toks)
    # the last replays ran on N(0, 1) logits: under unrenormalised softmax
    # rows differ in scale, and elements are held to their format floor
    # where that exceeds the required bound (tests/format_model.py)
    fl = parity.format_floor(x, lg, wgu, wd, cfg.top_k, cfg.score, cfg.renormalize, ref,
                             tokens=toks)
    parity.check_out(out[torch.from_numpy(toks).long().to(DEV)], ref, f"{name} graph", floor=fl)
    del g
