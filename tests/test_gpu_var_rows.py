"""GPU parity of the gate/up GEMM over the variable-size block table
(moe_options.schedule = 3, and the automatic schedule 0 that merges on the
device only when one round of workgroups needs it): experts with more than
128 rows take 256-row blocks (the last holding the rest) and the narrow
LDS-staged tile at 256 rows, the others the same tile at 128 rows; the down
GEMM keeps the 128-row blocks.

Every output sums the same 64-wide K steps in the same order whichever tile
computes it, so with the K start rotated per expert (the automatic rotation)
or not rotated the bytes equal those of the fixed 128-row table (schedule 1)
-- which also shows that the table covers every routed row exactly once
(an uncovered row would leave h unwritten).  Under the per-block and
per-workgroup rotations the start depends on the table, and the check is
the tolerance against the oracle.  Row counts are set exactly where the
cutting has edges: 1, 128, 129, 130, 256, 257 and 384 rows, an expert with
none; ragged K and a partial last column tile; both row-gather paths; the
automatic rule on the skewed workloads at full size (T = 512 merges, T = 128
does not) on every token; one workspace for merging and non-merging calls
in a row.  The table the routing kernels build, and their decision to
merge, equal the oracle's (O5c) bit for bit, read back from the
workspace."""
import numpy as np
import pytest
import torch

import expert_dispatch_router_amd as moe
import oracle
from expert_dispatch_router_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _exact_logits(counts, seed):
    """top-1 logits giving expert e exactly counts[e] tokens (tokens in a
    seeded order)."""
    E = len(counts)
    owner = np.repeat(np.arange(E), counts)
    np.random.default_rng(seed).shuffle(owner)
    T = len(owner)
    lg = torch.full((T, E), -3.0)
    lg[torch.arange(T), torch.from_numpy(owner)] = 3.0
    return lg


_CACHE = {}


def _case(name):
    if name not in _CACHE:
        spec = CASES[name]
        if "counts" in spec:
            counts, d, F, seed = spec["counts"], spec["d"], spec["F"], spec["seed"]
            lg = _exact_logits(counts, seed)
            T, E, k = lg.shape[0], lg.shape[1], 1
            _, x, lg, wgu, wd = parity.make_case(T, d, F, E, k, seed=seed, logits=lg)
        else:
            T, d, F, E, k, seed, skew = spec["shape"]
            _, x, lg, wgu, wd = parity.make_case(T, d, F, E, k, seed=seed, skew=skew)
        _CACHE[name] = (x, lg, wgu, wd, k, parity.oracle_out(x, lg, wgu, wd, k, 0, True))
    return _CACHE[name]


CASES = {
    # the cutting's edges: 0, 1, 128, 129, 130, 256, 257 and 384 rows
    "edges": dict(counts=[129, 256, 257, 384, 1, 0, 128, 130], d=256, F=448, seed=61),
    # ragged K (5 steps), ffn = 576: 4.5 column tiles of 128
    "ragged": dict(counts=[300, 40, 200, 3], d=320, F=576, seed=62),
    # one K step, one column tile of 64 real columns
    "short": dict(counts=[260, 17], d=64, F=64, seed=63),
    # top-4 of 16 experts under Zipf-like skew: hot experts of 200-400 rows
    "skewed": dict(shape=(400, 512, 704, 16, 4, 64, 2.0)),
}


def _fwd(c, **opts):
    x, lg, wgu, wd, k, _ = c
    return moe.moe_forward(x, lg, wgu, wd, k, True, **opts)


@pytest.mark.parametrize("name", sorted(CASES))
def test_variable_rows_match_oracle_and_fixed_table(name):
    c = _case(name)
    x, lg, wgu, wd, k, ref = c
    out = _fwd(c, schedule=3)
    parity.check_out(out, ref, f"variable rows {name}",
                     floor=parity.format_floor(x, lg, wgu, wd, k, 0, True, ref))
    fixed = _fwd(c, schedule=1, block_rows=128, fuse_down=1)  # the same down GEMM as schedule 3
    assert torch.equal(out.view(torch.int16), fixed.view(torch.int16)), name
    again = _fwd(c, schedule=3)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "not deterministic"


@pytest.mark.parametrize("gather", [1, 2])
@pytest.mark.parametrize("rotate", [1, 2, 3, 4])
def test_variable_rows_gather_and_rotation(gather, rotate):
    c = _case("skewed")
    x, lg, wgu, wd, k, ref = c
    out = _fwd(c, schedule=3, gather_mode=gather, rotate=rotate)
    parity.check_out(out, ref, f"variable rows gather={gather} rotate={rotate}",
                     floor=parity.format_floor(x, lg, wgu, wd, k, 0, True, ref))
    if rotate in (1, 4):  # no rotation, or per expert: the start does not depend on the table
        fixed = _fwd(c, schedule=1, block_rows=128, fuse_down=1, gather_mode=gather,
                     rotate=rotate)
        assert torch.equal(out.view(torch.int16), fixed.view(torch.int16))


@pytest.mark.parametrize("routing", [1, 2, 3])
def test_variable_rows_every_routing_path(routing):
    """The table is built by each routing path: the one-workgroup kernel,
    and the histogram kernel with and without the fused reorder."""
    c = _case("ragged")
    out = _fwd(c, schedule=3, routing_kernels=routing)
    fixed = _fwd(c, schedule=1, block_rows=128, fuse_down=1, routing_kernels=routing)
    assert torch.equal(out.view(torch.int16), fixed.view(torch.int16))
    parity.check_out(out, c[5], f"variable rows routing={routing}",
                     floor=parity.format_floor(*c[:5], 0, True, c[5]))


def test_variable_rows_workspace_reuse():
    """One workspace for a merging call (schedule 3) and calls of other
    sizes and tables in a row: the routing kernels rewrite the table and its
    count on every call, so results repeat bit for bit."""
    a, b = _case("edges"), _case("skewed")
    args = lambda c: (c[0].shape[0], c[0].shape[1], c[3].shape[2], c[1].shape[1], c[4])
    need = max(moe.moe_workspace_size(*args(c), block_rows=128, fuse_down=1, schedule=s)
               for c in (a, b) for s in (0, 3))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    first = {}
    for rep in range(3):
        for name, c, s in (("a3", a, 3), ("b0", b, 0), ("b3", b, 3), ("a0", a, 0)):
            out = _fwd(c, block_rows=128, fuse_down=1, schedule=s, workspace=ws)
            if rep == 0:
                first[name] = out.clone()
            else:
                assert torch.equal(out.view(torch.int16), first[name].view(torch.int16)), name
    assert torch.equal(first["a3"].view(torch.int16), first["a0"].view(torch.int16))
    assert torch.equal(first["b3"].view(torch.int16), first["b0"].view(torch.int16))


@pytest.mark.parametrize("name", ["skewed_512", "skewed_256", "skewed_128", "qwen2_128"])
def test_variable_rows_workloads_every_token(name):
    """The automatic schedule at full size: the device merges at skewed
    T=512 (30 fixed blocks x 11 column tiles > 256 workgroups, 23 merged)
    and keeps the fixed table at the others; every token against the
    oracle, and the bytes of the fixed table either way."""
    cfg = synth.CONFIGS[name]
    x, lg, wgu, wd = synth.make_inputs(cfg, 0, DEV)
    assert moe.moe_plan_ex(cfg.T, cfg.d, cfg.ffn, cfg.E, cfg.top_k)["variable_rows"] == 1
    out = moe.moe_forward(x, lg, wgu, wd, cfg.top_k, cfg.renormalize, score=cfg.score)
    fixed = moe.moe_forward(x, lg, wgu, wd, cfg.top_k, cfg.renormalize, score=cfg.score, schedule=1)
    assert torch.equal(out.view(torch.int16), fixed.view(torch.int16))
    forced = moe.moe_forward(x, lg, wgu, wd, cfg.top_k, cfg.renormalize, score=cfg.score,
                             schedule=3)
    assert torch.equal(forced.view(torch.int16), fixed.view(torch.int16))
    ref = parity.workload_reference(name, x, lg, wgu, wd, cfg)
    parity.check_workload(out, ref, name, x, lg, wgu, wd, cfg, what=name + " variable rows")
    del x, lg, wgu, wd, out, fixed, forced
    torch.cuda.empty_cache()


def _device_table(T, d, F, E, k, x, lg, wgu, wd, renorm, score, **opts):
    """Runs the forward pass in a workspace of its own and reads back the
    variable-size table and its count the routing kernels left there."""
    info = moe.moe_plan_ex(T, d, F, E, k, **opts)
    assert info["variable_rows"] in (1, 2)
    ws = torch.empty(moe.moe_workspace_size(T, d, F, E, k, **opts), dtype=torch.uint8, device=DEV)
    moe.moe_forward(x, lg, wgu, wd, k, renorm, score=score, workspace=ws, **opts)
    torch.cuda.synchronize()
    c0 = info["var_count_offset"]
    n = int(ws[c0:c0 + 4].view(torch.int32).item())
    if n < 0:
        return None, n, info
    t0 = info["var_table_offset"]
    return ws[t0:t0 + 12 * n].view(torch.int32).reshape(n, 3).cpu().numpy(), n, info


def _oracle_table(lg, k, score, renorm, F, mode):
    r = parity.oracle_routing(lg, k, score, renorm, 128)
    return oracle.var_block_table(r["counts"], r["offsets"], 128, -(-F // 128), mode)


@pytest.mark.parametrize("name,opts,merged", [
    ("edges", {"schedule": 3}, True),
    ("ragged", {"schedule": 3, "routing_kernels": 1}, True),
    ("ragged", {"schedule": 3, "routing_kernels": 2}, True),
    ("ragged", {"schedule": 3, "routing_kernels": 3}, True),
    ("skewed", {"schedule": 3}, True),
])
def test_device_table_matches_oracle(name, opts, merged):
    """The table the routing kernels build equals the oracle's (O5c) bit for
    bit, and so does the decision to merge."""
    x, lg, wgu, wd, k, _ = _case(name)
    T, d = x.shape
    E, F = lg.shape[1], wd.shape[2]
    vb, n, info = _device_table(T, d, F, E, k, x, lg, wgu, wd, True, 0, **opts)
    want, wn = _oracle_table(lg, k, 0, True, F, info["variable_rows"])
    assert n == wn and (n >= 0) == merged
    if merged:
        assert np.array_equal(vb, want)


@pytest.mark.parametrize("name,merged", [("skewed_512", True), ("skewed_256", False),
                                         ("skewed_128", False), ("qwen2_128", False)])
def test_device_table_rule_on_workloads(name, merged):
    """The automatic rule at full size: skewed T=512 merges (30 x 11
    workgroups to 23 x 11), the others keep the fixed table; the device's
    table and decision equal the oracle's."""
    cfg = synth.CONFIGS[name]
    x, lg, wgu, wd = synth.make_inputs(cfg, 0, DEV)
    vb, n, info = _device_table(cfg.T, cfg.d, cfg.ffn, cfg.E, cfg.top_k, x, lg, wgu, wd,
                                cfg.renormalize, cfg.score)
    assert info["variable_rows"] == 1
    want, wn = _oracle_table(lg, cfg.top_k, cfg.score, cfg.renormalize, cfg.ffn, 1)
    assert n == wn and (n >= 0) == merged
    if merged:
        assert np.array_equal(vb, want)
    del x, lg, wgu, wd
    torch.cuda.empty_cache()
