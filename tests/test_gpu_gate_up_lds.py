"""GPU parity of the LDS-staged GEMM tiles: the gate/up tile of BM = 192
(7 waves x 32 columns) and of BM = 128 (8 waves x 32), and the down tile of
BM = 128 and 192 (8 waves x 32), all with weights and activations fetched
into LDS by direct-to-LDS loads.

Each case meets the output tolerance against the oracle and, because the
tile sums every output's K chunks in the same order as the register-ring
tiles (64-wide steps, the same per-block K rotation), gives the same bytes
as the 112-column tile (variant 2) on the same inputs -- except under the
per-workgroup rotation, whose start depends on the tiling.  Cases cover ragged
blocks (rows ending mid-subtile), experts spanning several blocks, one and
two K steps, an odd number of K steps, both row-gather paths, every K
rotation, the XCD-grouped order and a partial last column tile; forcing
the tile with K-step-tiled activations is an error."""
import numpy as np
import pytest
import torch

import expert_dispatch_router_amd as moe
from tests import parity

pytestmark = pytest.mark.gpu
LDS = 3        # tile_variant option value of the LDS-staged tile (variant 2 of BM = 192)
REGRING = 2    # the 112-column register-ring tile


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


_CACHE = {}


def _case(name, T, d, F, E, k, seed):
    if name not in _CACHE:
        cfg, x, lg, wgu, wd = parity.make_case(T, d, F, E, k, seed=seed)
        _CACHE[name] = (x, lg, wgu, wd, k, parity.oracle_out(x, lg, wgu, wd, k, 0, True))
    return _CACHE[name]


CASES = {
    # ~50 rows per expert: one partial block each, rows end mid-subtile; 5 K steps
    "ragged": (150, 320, 448, 6, 2, 31),
    # ~267 rows per expert: a full block and a partial one per expert
    "multi_block": (400, 256, 448, 3, 2, 32),
    # one K step
    "one_step": (90, 64, 448, 4, 2, 33),
    # two K steps, 6 column tiles
    "two_steps": (120, 128, 1344, 5, 3, 34),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_lds_tile_matches_oracle_and_register_tile(name):
    x, lg, wgu, wd, k, ref = _case(name, *CASES[name])
    out = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=192, tile_variant=LDS)
    parity.check_out(out, ref, f"lds {name}")
    base = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=192, tile_variant=REGRING)
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


@pytest.mark.parametrize("gather", [1, 2])
@pytest.mark.parametrize("rotate", [1, 2, 3, 4])
def test_lds_tile_gather_and_rotation(gather, rotate):
    x, lg, wgu, wd, k, ref = _case("ragged", *CASES["ragged"])
    out = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=192, tile_variant=LDS,
                          gather_mode=gather, rotate=rotate)
    parity.check_out(out, ref, f"lds gather={gather} rotate={rotate}")
    if rotate != 3:  # a per-workgroup start depends on the tiling: the order differs there
        base = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=192, tile_variant=REGRING,
                               gather_mode=gather, rotate=rotate)
        assert torch.equal(out.view(torch.int16), base.view(torch.int16))


@pytest.mark.parametrize("xcd", [1, 2, 3])
def test_lds_tile_workgroup_orders(xcd):
    x, lg, wgu, wd, k, ref = _case("multi_block", *CASES["multi_block"])
    out = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=192, tile_variant=LDS, xcd_order=xcd)
    parity.check_out(out, ref, f"lds xcd={xcd}")


def test_lds_tile_is_automatic_at_192_rows():
    """~150 rows per expert picks BM = 192; ffn = 448 is two whole tiles, so
    the automatic options run the LDS-staged tile: the same bytes as forcing
    it, and within the tolerance.  (d = 2048 keeps the launch out of the
    small-launch path that fuses the down projection into the gate/up GEMM.)"""
    cfg, x, lg, wgu, wd = parity.make_case(600, 2048, 448, 4, 1, seed=35)
    bm, _, fused = moe.moe_plan(600, 2048, 448, 4, 1, with_fusion=True)
    assert bm == 192 and not fused
    out = moe.moe_forward(x, lg, wgu, wd, 1, True)
    forced = moe.moe_forward(x, lg, wgu, wd, 1, True, block_rows=192, tile_variant=LDS)
    assert torch.equal(out.view(torch.int16), forced.view(torch.int16))
    parity.check_out(out, parity.oracle_out(x, lg, wgu, wd, 1, 0, True), "lds automatic")


def test_lds_tile_rejected_where_it_cannot_run():
    x, lg, wgu, wd, k, _ = _case("ragged", *CASES["ragged"])
    with pytest.raises(moe.MoeError):  # K-step-tiled activations
        moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=192, tile_variant=LDS, gather_mode=3)


@pytest.mark.parametrize("bm", [128, 192])
def test_lds_tile_partial_last_tile(bm):
    """ffn = 576 is 2.57 tiles of 224 columns and 2.25 of 256: the last tile
    holds 128 (BM = 192) or 64 (BM = 128) real columns.  Its weight rows
    past ffn read as zeros and its outputs there are not stored: within the
    tolerance and the same bytes as the register-ring tile (both with the
    separate down GEMM: at this size the 64-column tile of BM = 128 would
    otherwise take the fused small-launch path)."""
    x, lg, wgu, wd, k, ref = _case("partial", 180, 256, 576, 6, 2, 41)
    out = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=bm, tile_variant=LDS, fuse_down=1)
    parity.check_out(out, ref, f"lds partial tile bm={bm}")
    base = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=bm, tile_variant=REGRING,
                           fuse_down=1)
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


# ------------------------------------------------- the LDS-staged down tile

DOWN_LDS = 3   # down_variant option value of the LDS-staged down tile (variant 2)


def _down_case():
    # d = 512 (two 256-column tiles), F = 384 (6 K steps), ~50 rows per expert
    return _case("down", 200, 512, 384, 12, 3, 37)


@pytest.mark.parametrize("split", [1, 2, 3])
@pytest.mark.parametrize("bm", [128, 192])
def test_lds_down_matches_oracle_and_register_tile(bm, split):
    """The down GEMM with its weights staged in LDS (8 waves x 32 columns):
    within the tolerance, and the same bytes as the register-ring down tile
    (variant 0), which sums every output's K chunks in the same order."""
    x, lg, wgu, wd, k, ref = _down_case()
    out = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=bm, split_k=split,
                          down_variant=DOWN_LDS)
    parity.check_out(out, ref, f"lds down bm={bm} split={split}")
    base = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=bm, split_k=split, down_variant=1)
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


def test_lds_down_several_blocks_per_expert():
    x, lg, wgu, wd, k, ref = _case("multi_block_down", 400, 256, 448, 3, 2, 38)
    for bm in (128, 192):
        out = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=bm, split_k=2,
                              down_variant=DOWN_LDS)
        parity.check_out(out, ref, f"lds down multi-block bm={bm}")


def test_lds_down_is_automatic():
    """At BM = 128 and 192 with d a multiple of 256 the automatic options
    run the LDS-staged down tile (the same bytes as forcing it); with the
    combination folded into the down GEMM they keep the register tile, and
    forcing the LDS tile there is an error."""
    x, lg, wgu, wd, k, ref = _down_case()
    for bm in (128, 192):
        auto = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=bm)
        forced = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=bm, down_variant=DOWN_LDS)
        assert torch.equal(auto.view(torch.int16), forced.view(torch.int16))
        folded = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=bm, fold_combine=2)
        parity.check_out(folded, ref, f"folded bm={bm}")
        with pytest.raises(moe.MoeError):
            moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=bm, fold_combine=2,
                            down_variant=DOWN_LDS)


def test_lds_gate_up_at_128_rows():
    """The 256-column LDS-staged gate/up tile of BM = 128; ffn = 512 is two
    whole tiles.  Within the tolerance, the same bytes as the register-ring
    tile, and chosen automatically when the launch fills a round (here 12
    blocks x 2 tiles do not: the automatic choice keeps a register tile)."""
    x, lg, wgu, wd, k, ref = _case("gate_up_128", 200, 512, 512, 12, 3, 39)
    out = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=128, tile_variant=3)
    parity.check_out(out, ref, "lds gate/up bm=128")
    base = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=128, tile_variant=1)
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


NARROW = 4  # tile_variant option value of the narrow LDS-staged tile (variant 3 of BM = 128)


def test_lds_gate_up_at_128_rows_is_automatic():
    """At BM = 128 the automatic options run the narrow LDS-staged tile (8
    waves x 16 columns, three stages): the same bytes as forcing it, as the
    256-column LDS tile and as the 128-column register-ring tile."""
    x, lg, wgu, wd, k, ref = _case("gate_up_128_auto", 256, 256, 1024, 64, 8, 40)
    assert moe.moe_plan(256, 256, 1024, 64, 8)[0] == 128
    assert moe.moe_plan_ex(256, 256, 1024, 64, 8)["gate_up_variant"] == NARROW - 1
    auto = moe.moe_forward(x, lg, wgu, wd, k, True)
    parity.check_out(auto, ref, "lds gate/up bm=128 automatic")
    for tv in (NARROW, 3, 1):
        forced = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=128, tile_variant=tv)
        assert torch.equal(auto.view(torch.int16), forced.view(torch.int16)), tv


@pytest.mark.parametrize("name", ["ragged", "multi_block", "one_step", "two_steps"])
def test_narrow_lds_gate_up_tile(name):
    """The narrow LDS-staged tile at BM = 128 on ragged blocks, experts
    with several blocks, one and two K steps and a partial last column
    tile (ffn = 448, 1344): the oracle's tolerance, and the bytes of the
    128-column register-ring tile."""
    x, lg, wgu, wd, k, ref = _case(name, *CASES[name])
    out = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=128, tile_variant=NARROW)
    parity.check_out(out, ref, f"narrow {name}")
    base = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=128, tile_variant=1)
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


# ------------------------ 192-row LDS tiles: blocks of at most 128 rows

def _exact_counts_case(counts, d, F, seed):
    """top-1 logits giving expert e exactly counts[e] tokens."""
    E = len(counts)
    owner = np.repeat(np.arange(E), counts)
    np.random.default_rng(seed).shuffle(owner)
    T = len(owner)
    lg = torch.full((T, E), -3.0)
    lg[torch.arange(T), torch.from_numpy(owner)] = 3.0
    _, x, lg, wgu, wd = parity.make_case(T, d, F, E, 1, seed=seed, logits=lg)
    return x, lg, wgu, wd, parity.oracle_out(x, lg, wgu, wd, 1, 0, True)


@pytest.mark.parametrize("split", [1, 2])
def test_192_row_tiles_switch_at_64_and_128_rows(split):
    """The LDS-staged gate/up (224 columns) and down (256 columns) tiles of
    BM = 192 run a block of at most 64 rows at 64 rows and one of at most
    128 at 128 (the same columns, fewer activation groups): blocks of 1 and
    64 rows (64-row path), 65 and 128 (128-row path), 129 and 192 rows
    (192-row path) give the same bytes as the register-ring tiles, and meet
    the tolerance."""
    x, lg, wgu, wd, ref = _exact_counts_case([128, 129, 1, 192, 64, 0, 65], 512, 448, 43)
    out = moe.moe_forward(x, lg, wgu, wd, 1, True, block_rows=192, tile_variant=LDS,
                          down_variant=3, split_k=split)
    parity.check_out(out, ref, f"192-row tiles split={split}")
    base = moe.moe_forward(x, lg, wgu, wd, 1, True, block_rows=192, tile_variant=REGRING,
                           down_variant=1, split_k=split)
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


# ------------------------------------------- the wide LDS-staged down tile

DOWN_WIDE = 4  # down_variant option value of the wide LDS-staged down tile (variant 3)

WIDE_CASES = {
    # d = 512: one whole 512-column tile at BM = 128; 448 + a partial 64 at BM = 192
    "d512": (200, 512, 384, 12, 3, 37),
    # d = 256: half a tile at BM = 128 (waves past the last column store nothing)
    "d256_multi_block": (400, 256, 448, 3, 2, 38),
    # d = 1024: two whole tiles at BM = 128; 448 + 448 + 128 at BM = 192; one K step
    "d1024_one_step": (96, 1024, 64, 5, 2, 39),
}


@pytest.mark.parametrize("split", [1, 2, 3])
@pytest.mark.parametrize("bm,variant", [(128, DOWN_WIDE), (192, DOWN_WIDE), (128, DOWN_WIDE + 1)])
@pytest.mark.parametrize("name", sorted(WIDE_CASES))
def test_lds_wide_down_matches_oracle_and_register_tile(name, bm, variant, split):
    """The down GEMM with 64 columns per wave staged in LDS (512 columns at
    BM = 128, 448 at BM = 192 and in the 7-wave tile of BM = 128, the last
    tile possibly partial): within the tolerance, and the same bytes as the
    register-ring down tile (variant 0), which sums every output's K chunks
    in the same order."""
    x, lg, wgu, wd, k, ref = _case(name, *WIDE_CASES[name])
    out = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=bm, split_k=split,
                          down_variant=variant)
    parity.check_out(out, ref, f"wide down {name} bm={bm} variant={variant} split={split}")
    base = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=bm, split_k=split, down_variant=1)
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


@pytest.mark.parametrize("xcd", [1, 2])
@pytest.mark.parametrize("rotate", [1, 2, 3, 4])
def test_lds_wide_down_orders_and_rotation(rotate, xcd):
    """Every K rotation and both workgroup orders: within the tolerance;
    without the per-workgroup rotation (whose start depends on the tiling)
    the same bytes as the 256-column LDS-staged down tile."""
    x, lg, wgu, wd, k, ref = _case("d512", *WIDE_CASES["d512"])
    for bm in (128, 192):
        out = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=bm, split_k=2,
                              down_variant=DOWN_WIDE, rotate=rotate, xcd_order=xcd)
        parity.check_out(out, ref, f"wide down bm={bm} rotate={rotate} xcd={xcd}")
        if rotate != 3:
            base = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=bm, split_k=2,
                                   down_variant=DOWN_LDS, rotate=rotate, xcd_order=xcd)
            assert torch.equal(out.view(torch.int16), base.view(torch.int16))


def test_lds_wide_down_rejected_where_it_cannot_run():
    """Forcing the wide tile with the combination folded into the down GEMM,
    or at a block size that has no wide tile, is an error."""
    x, lg, wgu, wd, k, ref = _case("d512", *WIDE_CASES["d512"])
    with pytest.raises(moe.MoeError):
        moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=128, fold_combine=2,
                        down_variant=DOWN_WIDE)
    with pytest.raises(moe.MoeError):
        moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=64, down_variant=DOWN_WIDE)


def test_xcd_order_when_real_workgroups_round_past_the_grid():
    """XCD grouping renumbers the real workgroups (blocks x tiles) rounded
    up to a multiple of eight; the launch must hold every id below that.
    Here A = 192 rows at BM = 192 (nb_max = 6, five blocks): the down GEMM's
    2 x 5 real workgroups round to 16 while 2 x 6 would be launched.  Every
    GEMM tile with the grouped order meets the tolerance and gives the same
    bytes as the plain order."""
    x, lg, wgu, wd, k, ref = _case("xcd_round", 64, 704, 448, 5, 3, 44)
    for tv, dv in ((0, 1), (LDS, 1), (0, 2), (LDS, DOWN_WIDE)):
        grouped = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=192, tile_variant=tv,
                                  down_variant=dv, xcd_order=2, fuse_down=1)
        parity.check_out(grouped, ref, f"xcd grouped tv={tv} dv={dv}")
        plain = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=192, tile_variant=tv,
                                down_variant=dv, xcd_order=1, fuse_down=1)
        assert torch.equal(grouped.view(torch.int16), plain.view(torch.int16))


# ------------------------------------------------------- 256-row blocks

NARROW = 4     # tile_variant option value of the 128-column LDS-staged tile of BM = 128
DOWN_LDS = 3   # down_variant option value of the 256-column LDS-staged down tile

CASES_256 = {
    # ~50 rows per expert: one partial block each, rows end mid-subtile
    "ragged": (150, 512, 448, 6, 2, 51),
    # ~400 rows per expert: a full 256-row block and a partial one per expert
    "multi_block": (600, 256, 448, 3, 2, 52),
    # ffn = 64: one down K step, a gate/up column tile of 64 real columns
    "short_ffn": (90, 256, 64, 4, 2, 53),
    # ffn = 576: 4.5 gate/up tiles of 128 columns, 9 down K steps
    "partial_tile": (180, 256, 576, 6, 2, 54),
    # d = 1280: 20 gate/up K steps, 5 down column tiles
    "deep_k": (300, 1280, 448, 4, 2, 55),
}


@pytest.mark.parametrize("name", sorted(CASES_256))
def test_256_row_blocks(name):
    """block_rows = 256 (only when asked for) runs the narrow gate/up tile
    and the 256-column down tile on blocks of up to 256 rows: within the
    tolerance, and -- with the K start rotated per expert and one down part
    on both sides -- the same bytes as the same two tiles on 128-row blocks,
    since every output sums the same 64-wide K steps in the same order."""
    x, lg, wgu, wd, k, ref = _case("bm256_" + name, *CASES_256[name])
    out = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=256, split_k=1)
    parity.check_out(out, ref, f"bm=256 {name}")
    base = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=128, tile_variant=NARROW,
                           down_variant=DOWN_LDS, split_k=1, fuse_down=1)
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))
    auto = moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=256)
    parity.check_out(auto, ref, f"bm=256 {name} automatic split")


def test_256_row_blocks_rejected_where_they_cannot_run():
    x, lg, wgu, wd, k, _ = _case("bm256_multi_block", *CASES_256["multi_block"])
    for opts in ({"tile_variant": 1}, {"unfused_swiglu": 1}, {"gather_mode": 3},
                 {"fold_combine": 2}, {"down_variant": 1}, {"fuse_down": 2}):
        with pytest.raises(moe.MoeError):
            moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=256, **opts)
    x, lg, wgu, wd, k, _ = _case("two_steps", *CASES["two_steps"])  # d = 128
    with pytest.raises(moe.MoeError):
        moe.moe_forward(x, lg, wgu, wd, k, True, block_rows=256)


@pytest.mark.parametrize("name", ["skewed_512", "skewed_128"])
def test_256_row_blocks_skewed_every_token(name):
    from expert_dispatch_router_amd import synth
    cfg = synth.CONFIGS[name]
    x, lg, wgu, wd = synth.make_inputs(cfg, 0, torch.device("cuda:0"))
    out = moe.moe_forward(x, lg, wgu, wd, cfg.top_k, cfg.renormalize, score=cfg.score,
                          block_rows=256)
    ref = parity.workload_reference(name, x, lg, wgu, wd, cfg)
    parity.check_workload(out, ref, name, x, lg, wgu, wd, cfg, what=name + " bm=256")
    del x, lg, wgu, wd, out
    torch.cuda.empty_cache()
