"""GPU parity of the stream-K gate/up schedule (moe_options.schedule = 2):
256 persistent workgroups share the K steps of every (block, column tile)
unit of the device-built schedule; a unit split between workgroups is
finished by the one that completes it, adding the fp32 partial sums in K
order.

Every case meets the output tolerance against the oracle.  Where no unit
is split (the workgroups' shares are whole units) the bytes equal those of
the same 128-column tile on the one-workgroup-per-unit schedule; otherwise
they may differ by the association of the K sums, so the two are held to
the tolerance and the schedule to bitwise determinism (same inputs, same
bytes, also with the workspace of an earlier call of other sizes: the
routing kernels clear the unit counters on every call).  Shapes cover fewer
units than workgroups (one unit split over 64 workgroups), a ragged last
share, several units per workgroup, every K rotation, both row-gather paths,
and the skewed workloads at full size on every token."""
import numpy as np
import pytest
import torch

import expert_dispatch_router_amd as moe
from expert_dispatch_router_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
NARROW = 4  # tile_variant option value of the 128-column LDS-staged tile (variant 3)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


_CACHE = {}


def _case(name, T, d, F, E, k, seed, score=0, renorm=True):
    if name not in _CACHE:
        cfg, x, lg, wgu, wd = parity.make_case(T, d, F, E, k, score=score, renorm=renorm, seed=seed)
        _CACHE[name] = (x, lg, wgu, wd, k, score, renorm,
                        parity.oracle_out(x, lg, wgu, wd, k, score, renorm))
    return _CACHE[name]


CASES = {
    # one expert, one block, one 128-column tile: a single unit of 64 K steps
    # split over 64 workgroups (the other 192 get no work)
    "one_unit": (40, 4096, 128, 1, 1, 41),
    # 3 units of 5 K steps: 15 iterations, most workgroups idle
    "few_iters": (30, 320, 384, 2, 1, 42),
    # ~90 units of 8 K steps: shares of 2-3 steps, every unit split
    "split_units": (300, 512, 640, 12, 3, 43),
    # 8 experts x 2 blocks x 28 tiles x 16 steps: shares of 7 steps
    "many_units": (512, 1024, 3584, 8, 4, 44),
    # ragged rows (blocks end mid-subtile), 6 K steps, ffn not a multiple of 128
    "ragged": (150, 384, 448, 6, 2, 45),
}


def _forward(x, lg, wgu, wd, k, score, renorm, **opts):
    return moe.moe_forward(x, lg, wgu, wd, k, renorm, score=score, **opts)


@pytest.mark.parametrize("name", sorted(CASES))
def test_stream_k_matches_oracle(name):
    x, lg, wgu, wd, k, score, renorm, ref = _case(name, *CASES[name])
    out = _forward(x, lg, wgu, wd, k, score, renorm, schedule=2)
    parity.check_out(out, ref, f"stream-K {name}",
                     floor=parity.format_floor(x, lg, wgu, wd, k, score, renorm, ref))
    base = _forward(x, lg, wgu, wd, k, score, renorm, block_rows=128, tile_variant=NARROW,
                    schedule=1)
    parity.check_out(base, ref, f"one workgroup per unit {name}",
                     floor=parity.format_floor(x, lg, wgu, wd, k, score, renorm, ref))
    again = _forward(x, lg, wgu, wd, k, score, renorm, schedule=2)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "not deterministic"


def test_stream_k_whole_units_give_the_same_bytes():
    """When every workgroup's share is whole units (units x steps a multiple
    of 256 x steps: 8 blocks x 32 tiles, 4 per workgroup), nothing is split
    and the result equals the one-workgroup-per-unit schedule's bytes."""
    # E = 8 experts of exactly 128 rows each (a logit that picks one expert per token)
    T, d, F, E, k = 1024, 256, 4096, 8, 1
    cfg, x, lg, wgu, wd = parity.make_case(T, d, F, E, k, seed=46)
    lg = torch.full((T, E), -4.0, device=DEV)
    lg[torch.arange(T, device=DEV), torch.arange(T, device=DEV) % E] = 4.0
    info = moe.moe_plan_ex(T, d, F, E, k, schedule=2)
    assert info["stream_k"] == 1
    out = moe.moe_forward(x, lg, wgu, wd, k, True, schedule=2)
    base = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=128, tile_variant=NARROW, schedule=1)
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))
    toks = np.array([0, 1, 7, 500, 1023], dtype=np.int32)
    ref = parity.oracle_out(x, lg, wgu, wd, k, 0, True, tokens=toks)
    parity.check_out(out[torch.from_numpy(toks).long().to(DEV)], ref, "whole units")


@pytest.mark.parametrize("gather", [1, 2])
@pytest.mark.parametrize("rotate", [1, 2, 3, 4])
def test_stream_k_gather_and_rotation(gather, rotate):
    x, lg, wgu, wd, k, score, renorm, ref = _case("split_units", *CASES["split_units"])
    out = _forward(x, lg, wgu, wd, k, score, renorm, schedule=2, gather_mode=gather, rotate=rotate)
    parity.check_out(out, ref, f"stream-K gather={gather} rotate={rotate}",
                     floor=parity.format_floor(x, lg, wgu, wd, k, score, renorm, ref))


def test_stream_k_workspace_reuse():
    """One workspace for calls of other sizes in a row: the unit counters
    are cleared by every call's routing, so results repeat bit for bit."""
    big = _case("split_units", *CASES["split_units"])
    small = _case("few_iters", *CASES["few_iters"])
    need = max(moe.moe_workspace_size(c[0].shape[0], c[0].shape[1], c[3].shape[2], c[1].shape[1],
                                      c[4], schedule=2) for c in (big, small))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    first = {}
    for rep in range(3):
        for name, c in (("big", big), ("small", small)):
            x, lg, wgu, wd, k, score, renorm, ref = c
            out = _forward(x, lg, wgu, wd, k, score, renorm, schedule=2, workspace=ws)
            if rep == 0:
                first[name] = out.clone()
                parity.check_out(out, ref, f"reuse {name}",
                                 floor=parity.format_floor(x, lg, wgu, wd, k, score, renorm, ref))
            else:
                assert torch.equal(out.view(torch.int16), first[name].view(torch.int16)), name


@pytest.mark.parametrize("name", ["skewed_128", "skewed_256", "skewed_512", "qwen2_128"])
def test_stream_k_workloads_every_token(name):
    """Skew-prone workloads at full size with the stream-K schedule: every
    token against the oracle."""
    cfg = synth.CONFIGS[name]
    x, lg, wgu, wd = synth.make_inputs(cfg, 0, DEV)
    out = moe.moe_forward(x, lg, wgu, wd, cfg.top_k, cfg.renormalize, score=cfg.score, schedule=2)
    ref = parity.workload_reference(name, x, lg, wgu, wd, cfg)
    parity.check_workload(out, ref, name, x, lg, wgu, wd, cfg, what=name + " stream-K")
    del x, lg, wgu, wd, out
    torch.cuda.empty_cache()
