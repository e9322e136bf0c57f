"""GPU parity of the down projection fused into the gate/up GEMM
(fuse_down = 2): each gate/up workgroup multiplies its SwiGLU tile by the
matching W_down columns and writes one fp32 partial per column tile, which
the combination adds in tile order.  Against the oracle at the usual
tolerance (the summation order differs from the separate down GEMM, so the
bytes may differ from it), and deterministic."""
import numpy as np
import pytest
import torch

import expert_dispatch_router_amd as moe
from expert_dispatch_router_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (block_rows, tile_variant option) of the compiled fused tiles
FUSED = [(64, 2), (128, 0), (192, 1)]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


_MID = {}


def _mid():
    if not _MID:
        cfg, x, lg, wgu, wd = parity.make_case(200, 512, 384, 12, 3, seed=5)
        _MID["v"] = (x, lg, wgu, wd, parity.oracle_out(x, lg, wgu, wd, 3, 0, True))
    return _MID["v"]


@pytest.mark.parametrize("bm,tv", FUSED)
def test_fused_down_every_tile(bm, tv):
    x, lg, wgu, wd, ref = _mid()
    out = moe.moe_forward(x, lg, wgu, wd, 3, True, score=0, block_rows=bm, tile_variant=tv,
                          fuse_down=2)
    parity.check_out(out, ref, f"fused bm={bm}")
    again = moe.moe_forward(x, lg, wgu, wd, 3, True, score=0, block_rows=bm, tile_variant=tv,
                            fuse_down=2)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "deterministic"


@pytest.mark.parametrize("bm,tv", FUSED)
def test_fused_down_partial_column_tiles(bm, tv):
    """d=320, F=192: the last gate/up column tile (and so the last partial)
    covers fewer columns than the tile."""
    cfg, x, lg, wgu, wd = parity.make_case(70, 320, 192, 6, 2, seed=13)
    out = moe.moe_forward(x, lg, wgu, wd, 2, True, block_rows=bm, tile_variant=tv, fuse_down=2)
    parity.check_out(out, parity.oracle_out(x, lg, wgu, wd, 2, 0, True), f"fused partial bm={bm}")


@pytest.mark.parametrize("gather", [1, 2, 3])
@pytest.mark.parametrize("routing", [1, 2])
def test_fused_down_routing_and_gather_paths(routing, gather):
    x, lg, wgu, wd, ref = _mid()
    out = moe.moe_forward(x, lg, wgu, wd, 3, True, score=0, block_rows=128, fuse_down=2,
                          routing_kernels=routing, gather_mode=gather)
    parity.check_out(out, ref, f"fused routing={routing} gather={gather}")


@pytest.mark.parametrize("T,E,k,score,renorm", [(1, 8, 2, 0, True), (17, 1, 1, 1, False),
                                                (40, 6, 6, 0, False), (130, 64, 8, 1, True)])
def test_fused_down_shapes(T, E, k, score, renorm):
    cfg, x, lg, wgu, wd = parity.make_case(T, 256, 128, E, k, score=score, renorm=renorm,
                                           seed=T + E)
    out = moe.moe_forward(x, lg, wgu, wd, k, renorm, score=score, block_rows=128, fuse_down=2)
    parity.check_out(out, parity.oracle_out(x, lg, wgu, wd, k, score, renorm),
                     f"fused T={T} E={E}")


def test_fused_down_tiny_all_tokens():
    cfg = synth.CONFIGS["tiny"]
    x, lg, wgu, wd = synth.make_inputs(cfg, 0, DEV)
    out = moe.moe_forward(x, lg, wgu, wd, cfg.top_k, cfg.renormalize, score=cfg.score,
                          fuse_down=2)
    ref = parity.oracle_out(x, lg, wgu, wd, cfg.top_k, cfg.score, cfg.renormalize)
    parity.check_out(out, ref, "tiny fused")


def test_fused_down_hot_expert():
    gen = torch.Generator().manual_seed(3)
    lg = torch.randn(300, 8, generator=gen)
    lg[:, 1] += 30.0
    cfg, x, lg, wgu, wd = parity.make_case(300, 256, 128, 8, 2, seed=3, logits=lg)
    out = moe.moe_forward(x, lg, wgu, wd, 2, True, block_rows=64, tile_variant=2, fuse_down=2)
    parity.check_out(out, parity.oracle_out(x, lg, wgu, wd, 2, 0, True), "fused hot expert")
