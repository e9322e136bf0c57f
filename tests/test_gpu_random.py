"""GPU parity over randomized small problems: shapes, scores, options and
routing paths drawn from a fixed seed, each checked against the oracle
(routing bit for bit, output within the tolerance).

The draws leave the workloads' regimes on purpose: ffn down to 64,
unrenormalised softmax over up to 256 experts (rows of very different
scale), top-k up to 16, the unfused ablation.  There the bf16 formats of h
(g and u in the ablation) and of the output alone can miss the required
max-abs bound (tests/test_format_floor.py), so each element is held to the
larger of that bound and its own format floor (tests/format_model.py: exact
arithmetic with just those roundings) plus a small slack; the relative
Frobenius bound applies as it is.  Every token is compared, except in the
draws with many blocks, which compare the tokens holding the first and last
row of every schedule block."""
import numpy as np
import pytest
import torch

import expert_dispatch_router_amd as moe
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cases(n=24, seed=1234):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 5, 8, 13, 32, 60, 64, 100]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 3, 17, 64, 130, 257]))
        d = int(64 * rng.integers(2, 13))
        F = int(64 * rng.integers(1, 17))
        score = int(rng.integers(0, 2))
        renorm = bool(rng.integers(0, 2))
        opts = {}
        if rng.random() < 0.5:
            opts["block_rows"] = int(rng.choice([16, 32, 64, 128, 192]))
        if rng.random() < 0.4:
            opts["split_k"] = int(rng.integers(1, 4))
        opts["routing_kernels"] = int(rng.integers(0, 3))
        if opts["routing_kernels"] == 1 and not (T <= 1024 and E <= 64):
            opts["routing_kernels"] = 2
        opts["gather_mode"] = int(rng.integers(0, 4))
        opts["rotate"] = int(rng.integers(0, 4))
        opts["xcd_order"] = int(rng.integers(0, 3))
        out.append((i, T, d, F, E, k, score, renorm, opts))
    return out


def _check(out, x, lg, wgu, wd, k, score, renorm, what, unfused=False, tokens=None):
    ref = parity.oracle_out(x, lg, wgu, wd, k, score, renorm, tokens=tokens)
    fl = parity.format_floor(x, lg, wgu, wd, k, score, renorm, ref, tokens=tokens,
                             rounding="unfused" if unfused else "fused")
    got = out if tokens is None else out[torch.from_numpy(tokens).long().to(out.device)]
    parity.check_out(got, ref, what, floor=fl)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_problem(case):
    i, T, d, F, E, k, score, renorm, opts = case
    cfg, x, lg, wgu, wd = parity.make_case(T, d, F, E, k, score=score, renorm=renorm, seed=100 + i)
    out = moe.moe_forward(x, lg, wgu, wd, k, renorm, score="sigmoid" if score else "softmax",
                          **opts)
    _check(out, x, lg, wgu, wd, k, score, renorm, f"case{i} T={T} d={d} F={F} E={E} k={k} {opts}")
    r = moe.moe_route(lg, k, renorm, "sigmoid" if score else "softmax",
                      block_rows=opts.get("block_rows", 0),
                      routing_kernels=opts["routing_kernels"])
    parity.check_routing(r, parity.oracle_routing(lg, k, score, renorm, r["bm"]))


def _cases_new_options(n=16, seed=4321):
    """Draws over the later options: the combination folded into the down
    GEMM, the down projection fused into the gate/up GEMM, the longest-first
    block order (each with the other options drawn as above)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 5, 8, 13, 32, 60, 64, 100]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 3, 17, 64, 130, 257]))
        d = int(64 * rng.integers(2, 13))
        F = int(64 * rng.integers(1, 17))
        score = int(rng.integers(0, 2))
        renorm = bool(rng.integers(0, 2))
        opts = {"routing_kernels": 2 if E > 32 else int(rng.integers(0, 3)),
                "gather_mode": int(rng.integers(0, 4)),
                "xcd_order": int(rng.choice([0, 1, 3]))}
        kind = i % 3
        if kind == 0:
            opts["fold_combine"] = 2
            opts["fuse_down"] = 1
            if rng.random() < 0.5:
                opts["split_k"] = int(rng.integers(1, 4))
            if rng.random() < 0.5:
                opts["block_rows"] = int(rng.choice([16, 32, 64, 128, 192]))
        elif kind == 1:
            opts["fuse_down"] = 2
            opts["block_rows"], tv = [(64, 2), (128, 0), (192, 1)][int(rng.integers(0, 3))]
            if tv:
                opts["tile_variant"] = tv
        else:
            opts["block_rows"] = int(rng.choice([16, 32, 64, 128, 192]))
        out.append((i, T, d, F, E, k, score, renorm, opts))
    return out


@pytest.mark.parametrize("case", _cases_new_options(), ids=lambda c: f"opt{c[0]}")
def test_random_problem_new_options(case):
    i, T, d, F, E, k, score, renorm, opts = case
    cfg, x, lg, wgu, wd = parity.make_case(T, d, F, E, k, score=score, renorm=renorm, seed=500 + i)
    out = moe.moe_forward(x, lg, wgu, wd, k, renorm, score="sigmoid" if score else "softmax",
                          **opts)
    _check(out, x, lg, wgu, wd, k, score, renorm, f"opt{i} T={T} d={d} F={F} E={E} k={k} {opts}")


def _cases_lds_tiles(n=16, seed=2468):
    """Draws over the LDS-staged tiles (the gate/up tile of BM = 128 and 192,
    the 32- and 64-column-per-wave down tiles, partial last column tiles
    included) and the two-launch routing, with the other options drawn."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 5, 8, 13, 32, 60, 64, 100]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 3, 17, 64, 130, 257, 600]))
        d = int(64 * rng.integers(2, 17))
        F = int(64 * rng.integers(3, 17))
        score = int(rng.integers(0, 2))
        renorm = bool(rng.integers(0, 2))
        bm = int(rng.choice([128, 192]))
        opts = {"block_rows": bm, "gather_mode": int(rng.integers(0, 3)),
                "rotate": int(rng.integers(0, 4)), "xcd_order": int(rng.integers(0, 3)),
                "fuse_down": 1}
        if rng.random() < 0.7:
            # the LDS-staged gate/up tiles: 2 subtiles per wave, or (BM = 128) one
            opts["tile_variant"] = int(rng.choice([3, 4])) if bm == 128 else 3
        dv = [0, 4] + ([3] if d % 256 == 0 else [])
        opts["down_variant"] = int(rng.choice(dv))
        if rng.random() < 0.6:
            opts["split_k"] = int(rng.integers(1, 5))
        fits = (T * k + 63) // 64 * E <= 16384
        opts["routing_kernels"] = int(rng.choice([0, 2, 3] if fits else [0, 2]))
        out.append((i, T, d, F, E, k, score, renorm, opts))
    return out


@pytest.mark.parametrize("case", _cases_lds_tiles(), ids=lambda c: f"lds{c[0]}")
def test_random_problem_lds_tiles(case):
    i, T, d, F, E, k, score, renorm, opts = case
    cfg, x, lg, wgu, wd = parity.make_case(T, d, F, E, k, score=score, renorm=renorm, seed=900 + i)
    out = moe.moe_forward(x, lg, wgu, wd, k, renorm, score="sigmoid" if score else "softmax",
                          **opts)
    _check(out, x, lg, wgu, wd, k, score, renorm, f"lds{i} T={T} d={d} F={F} E={E} k={k} {opts}")
    r = moe.moe_route(lg, k, renorm, "sigmoid" if score else "softmax", block_rows=opts["block_rows"],
                      routing_kernels=opts["routing_kernels"])
    parity.check_routing(r, parity.oracle_routing(lg, k, score, renorm, r["bm"]))


def _cases_many_blocks(n=12, seed=97531):
    """Larger draws (many schedule blocks: the automatic XCD order, the
    two-launch routing at larger A, several blocks per expert), every
    option drawn; the oracle checks the tokens of every block's first and
    last row."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([16, 64, 128, 256]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([700, 1300, 2000]))
        d = int(64 * rng.integers(2, 7))
        F = int(64 * rng.integers(2, 7))
        score = int(rng.integers(0, 2))
        renorm = bool(rng.integers(0, 2))
        opts = {"gather_mode": int(rng.integers(0, 3)), "rotate": int(rng.integers(0, 4)),
                "xcd_order": int(rng.integers(0, 4))}
        if rng.random() < 0.6:
            bm = int(rng.choice([16, 32, 64, 128, 192]))
            opts["block_rows"] = bm
            if bm in (128, 192):
                opts["tile_variant"] = int(rng.choice([0, 3]))
                opts["down_variant"] = int(rng.choice([0, 4]))
        if rng.random() < 0.4:
            opts["split_k"] = int(rng.integers(1, 4))
        fits = (T * k + 63) // 64 * E <= 16384
        opts["routing_kernels"] = int(rng.choice([0, 2, 3] if fits else [0, 2]))
        out.append((i, T, d, F, E, k, score, renorm, opts))
    return out


def _cases_stream_k(n=12, seed=4242):
    """Draws over the stream-K gate/up schedule (schedule = 2): units from
    one to thousands, K steps from 2 to 16, ragged blocks and partial last
    column tiles, with the routing, gather, rotation, split and down tile
    drawn."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 5, 8, 13, 32, 64, 100]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 3, 17, 64, 130, 257, 600]))
        d = int(64 * rng.integers(2, 17))
        F = int(64 * rng.integers(1, 16))  # odd multiples of 64: a partial last column tile
        score = int(rng.integers(0, 2))
        renorm = bool(rng.integers(0, 2))
        opts = {"schedule": 2, "gather_mode": int(rng.integers(0, 3)),
                "rotate": int(rng.integers(0, 5)), "xcd_order": int(rng.integers(0, 3))}
        if rng.random() < 0.4:
            opts["split_k"] = int(rng.integers(1, 4))
        fits = (T * k + 63) // 64 * E <= 16384
        opts["routing_kernels"] = int(rng.choice([0, 2, 3] if fits else [0, 2]))
        out.append((i, T, d, F, E, k, score, renorm, opts))
    return out


@pytest.mark.parametrize("case", _cases_stream_k(), ids=lambda c: f"sk{c[0]}")
def test_random_problem_stream_k(case):
    i, T, d, F, E, k, score, renorm, opts = case
    cfg, x, lg, wgu, wd = parity.make_case(T, d, F, E, k, score=score, renorm=renorm, seed=1300 + i)
    out = moe.moe_forward(x, lg, wgu, wd, k, renorm, score="sigmoid" if score else "softmax",
                          **opts)
    _check(out, x, lg, wgu, wd, k, score, renorm, f"sk{i} T={T} d={d} F={F} E={E} k={k} {opts}")


def _cases_var_rows(n=12, seed=5151):
    """Draws over the variable-size gate/up table, merged always (schedule
    = 3): skewed routing (hot experts past 128 and 256 rows) and uniform,
    ragged K and partial last column tiles, with the routing, gather,
    rotation, split and workgroup order drawn."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 5, 8, 16, 33, 64]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 17, 130, 257, 600, 1000]))
        d = int(64 * rng.integers(1, 17))
        F = int(64 * rng.integers(1, 16))
        score = int(rng.integers(0, 2))
        renorm = bool(rng.integers(0, 2))
        skew = float(rng.choice([0.0, 1.0, 2.0]))
        opts = {"schedule": 3, "gather_mode": int(rng.integers(0, 3)),
                "rotate": int(rng.integers(0, 5)), "xcd_order": int(rng.integers(0, 2))}
        if rng.random() < 0.4:
            opts["split_k"] = int(rng.integers(1, 4))
        fits = (T * k + 63) // 64 * E <= 16384
        opts["routing_kernels"] = int(rng.choice([0, 1, 2, 3] if fits and E <= 64 and T <= 1024
                                                 else [0, 2]))
        out.append((i, T, d, F, E, k, score, renorm, skew, opts))
    return out


@pytest.mark.parametrize("case", _cases_var_rows(), ids=lambda c: f"var{c[0]}")
def test_random_problem_variable_rows(case):
    i, T, d, F, E, k, score, renorm, skew, opts = case
    cfg, x, lg, wgu, wd = parity.make_case(T, d, F, E, k, score=score, renorm=renorm,
                                           seed=1700 + i, skew=skew)
    out = moe.moe_forward(x, lg, wgu, wd, k, renorm, score="sigmoid" if score else "softmax",
                          **opts)
    _check(out, x, lg, wgu, wd, k, score, renorm,
           f"var{i} T={T} d={d} F={F} E={E} k={k} skew={skew} {opts}")


@pytest.mark.parametrize("case", _cases_many_blocks(), ids=lambda c: f"big{c[0]}")
def test_random_problem_many_blocks(case):
    i, T, d, F, E, k, score, renorm, opts = case
    cfg, x, lg, wgu, wd = parity.make_case(T, d, F, E, k, score=score, renorm=renorm,
                                           seed=1300 + i)
    out = moe.moe_forward(x, lg, wgu, wd, k, renorm, score="sigmoid" if score else "softmax",
                          **opts)
    r = moe.moe_route(lg, k, renorm, "sigmoid" if score else "softmax",
                      block_rows=opts.get("block_rows", 0),
                      routing_kernels=opts["routing_kernels"])
    parity.check_routing(r, parity.oracle_routing(lg, k, score, renorm, r["bm"]))
    toks = parity.tokens_per_block(lg, k, score, renorm, r["bm"])
    _check(out, x, lg, wgu, wd, k, score, renorm, f"big{i} T={T} d={d} F={F} E={E} k={k} {opts}",
           tokens=toks)


def _cases_all_options(n=60, seed=31337):
    """Every option drawn at once (block size, both tile variants, split,
    rotation, routing kernels, gather mode, workgroup order, folded
    combination, fused down projection, unfused ablation), over shapes from
    one token to 1500 and from 1 to 256 experts with top-k up to 16.  Option
    sets the library refuses up front are left out; the rest must meet the
    tolerance (held to the ablation's own format floor where it runs)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.choice([1, 2, 3, 8, 16, 33, 64, 100, 128, 256]))
        k = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.choice([1, 2, 5, 31, 64, 100, 257, 513, 1000, 1500]))
        d = int(64 * rng.integers(1, 14))
        F = int(64 * rng.integers(1, 14))
        score = int(rng.integers(0, 2))
        renorm = bool(rng.integers(0, 2))
        opts = {}
        if rng.random() < 0.7:
            opts["block_rows"] = int(rng.choice([16, 32, 64, 128, 192]))
            if rng.random() < 0.5:
                opts["tile_variant"] = int(rng.integers(0, 4))
            if rng.random() < 0.5:
                opts["down_variant"] = int(rng.integers(0, 6))
        for key, hi in (("split_k", 5), ("rotate", 4), ("routing_kernels", 4), ("gather_mode", 4),
                        ("xcd_order", 4), ("fold_combine", 3), ("fuse_down", 3),
                        ("unfused_swiglu", 2)):
            if rng.random() < 0.4:
                opts[key] = int(rng.integers(0, hi))
        try:
            moe.moe_workspace_size(T, d, F, E, k, **opts)
        except moe.MoeError:
            continue
        out.append((len(out), T, d, F, E, k, score, renorm, opts))
    return out


@pytest.mark.parametrize("case", _cases_all_options(), ids=lambda c: f"all{c[0]}")
def test_random_problem_all_options(case):
    i, T, d, F, E, k, score, renorm, opts = case
    cfg, x, lg, wgu, wd = parity.make_case(T, d, F, E, k, score=score, renorm=renorm,
                                           seed=2000 + i)
    out = moe.moe_forward(x, lg, wgu, wd, k, renorm, score="sigmoid" if score else "softmax",
                          **opts)
    _check(out, x, lg, wgu, wd, k, score, renorm, f"all{i} T={T} d={d} F={F} E={E} k={k} {opts}",
           unfused=bool(opts.get("unfused_swiglu")))
