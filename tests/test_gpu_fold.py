"""GPU parity of the weighted combination folded into the down GEMM
(fold_combine = 2).  The folded path must give the bytes of the separate
combination kernel (same sums, same fixed order), meet the oracle tolerance,
and clear its arrival counters itself: the workspace is filled with 0xFF
before the first call and reused, un-cleared, for a second call."""
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


def _fold_matches_separate(x, lg, wgu, wd, k, renorm, score, what, **opts):
    opts.setdefault("fuse_down", 1)  # the fold lives in the separate down GEMM
    T, d = x.shape
    E, F = lg.shape[1], wd.shape[2]
    # the folded combination counts the parts as planned; the separate one is
    # compared at that same split (left automatic, it may take fewer parts
    # on the device, another summation order)
    opts.setdefault("split_k", moe.moe_plan_ex(T, d, F, E, k, fold_combine=2, **opts)["split_k"])
    sep = moe.moe_forward(x, lg, wgu, wd, k, renorm, score=score, fold_combine=1, **opts)
    ws = torch.empty(moe.moe_workspace_size(T, d, F, E, k, fold_combine=2, **opts),
                     dtype=torch.uint8, device=DEV)
    ws.fill_(0xFF)  # counters start as garbage: the routing kernels must clear them
    for call in range(2):
        out = torch.full_like(sep, float("nan"))
        moe.moe_forward(x, lg, wgu, wd, k, renorm, score=score, out=out, workspace=ws,
                        fold_combine=2, **opts)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), sep.view(torch.int16)), f"{what} call {call}"
    return out


_MID = {}


def _mid():
    if not _MID:
        cfg, x, lg, wgu, wd = parity.make_case(200, 512, 384, 12, 3, seed=5)
        _MID["v"] = (x, lg, wgu, wd, parity.oracle_out(x, lg, wgu, wd, 3, 0, True))
    return _MID["v"]


@pytest.mark.parametrize("split", [1, 3])
@pytest.mark.parametrize("bm", [16, 32, 64, 128, 192])
def test_fold_every_block_size_and_split(bm, split):
    x, lg, wgu, wd, ref = _mid()
    out = _fold_matches_separate(x, lg, wgu, wd, 3, True, 0, f"bm={bm} split={split}",
                                 block_rows=bm, split_k=split)
    parity.check_out(out, ref, f"fold bm={bm} split={split}")


@pytest.mark.parametrize("bm,dvar", [(128, 1), (128, 2), (192, 1), (192, 2)])
def test_fold_down_variants(bm, dvar):
    x, lg, wgu, wd, ref = _mid()
    out = _fold_matches_separate(x, lg, wgu, wd, 3, True, 0, f"bm={bm} dvar={dvar}",
                                 block_rows=bm, down_variant=dvar, split_k=2)
    parity.check_out(out, ref, f"fold bm={bm} dvar={dvar}")


@pytest.mark.parametrize("bm", [32, 192])
def test_fold_partial_column_tiles(bm):
    """d=320: the last down-GEMM column tile is partly empty."""
    cfg, x, lg, wgu, wd = parity.make_case(70, 320, 192, 6, 2, seed=13)
    out = _fold_matches_separate(x, lg, wgu, wd, 2, True, 0, f"partial bm={bm}",
                                 block_rows=bm, split_k=2)
    parity.check_out(out, parity.oracle_out(x, lg, wgu, wd, 2, 0, True), f"fold partial bm={bm}")


@pytest.mark.parametrize("routing", [1, 2])
@pytest.mark.parametrize("score,renorm", [(0, False), (1, True)])
def test_fold_routing_paths_and_scores(routing, score, renorm):
    """Both routing paths clear the counters (one workgroup / three launches)."""
    cfg, x, lg, wgu, wd = parity.make_case(96, 256, 256, 16, 4, score=score, renorm=renorm, seed=9)
    out = _fold_matches_separate(x, lg, wgu, wd, 4, renorm, score, f"routing={routing}",
                                 routing_kernels=routing)
    parity.check_out(out, parity.oracle_out(x, lg, wgu, wd, 4, score, renorm), "fold scores")


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (17, 1, 1), (40, 6, 6), (130, 64, 8), (130, 256, 8)])
def test_fold_shapes(T, E, k):
    cfg, x, lg, wgu, wd = parity.make_case(T, 256, 128, E, k, seed=T + E)
    out = _fold_matches_separate(x, lg, wgu, wd, k, True, 0, f"T={T} E={E} k={k}")
    parity.check_out(out, parity.oracle_out(x, lg, wgu, wd, k, 0, True), f"fold T={T} E={E}")


def test_fold_hot_expert_many_blocks():
    gen = torch.Generator().manual_seed(3)
    lg = torch.randn(300, 8, generator=gen)
    lg[:, 1] += 30.0
    cfg, x, lg, wgu, wd = parity.make_case(300, 256, 128, 8, 2, seed=3, logits=lg)
    out = _fold_matches_separate(x, lg, wgu, wd, 2, True, 0, "hot expert", block_rows=32,
                                 split_k=2)
    parity.check_out(out, parity.oracle_out(x, lg, wgu, wd, 2, 0, True), "fold hot expert")


@pytest.mark.parametrize("name", ["tiny", "mixtral_512", "dsv3_512", "skewed_512"])
def test_fold_full_size(name):
    """Workload sizes with automatic options: every token equal to the
    separate combination, and every token against the oracle."""
    cfg = synth.CONFIGS[name]
    x, lg, wgu, wd = synth.make_inputs(cfg, 0, DEV)
    out = _fold_matches_separate(x, lg, wgu, wd, cfg.top_k, cfg.renormalize, cfg.score, name)
    ref = parity.workload_reference(name, x, lg, wgu, wd, cfg)
    parity.check_workload(out, ref, name, x, lg, wgu, wd, cfg, what=name + " fold")
    del x, lg, wgu, wd, out
    torch.cuda.empty_cache()
