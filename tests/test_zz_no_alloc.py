"""moe_forward_static, the entry point that allocates nothing (its workspace
is a fixed device array inside the library), against moe_forward: the same
kernels on the same inputs must give the same bytes, call after call --
the second call smaller than the first, so it runs over what the first left
in the array -- and meet the tolerance against the oracle."""
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


def _both(x, lg, wgu, wd, k, renorm, score):
    want = moe.moe_forward(x, lg, wgu, wd, k, renorm, score=score)
    got = torch.full_like(want, float("nan"))
    moe.moe_forward_static(x, lg, wgu, wd, k, renorm, got, score=score)
    torch.cuda.synchronize()
    return got, want


def test_static_workspace_matches_forward_call_after_call():
    """Two calls in a row, the second with a smaller problem; then the first
    again.  Each is byte-equal to moe_forward and within the tolerance."""
    cases = [(300, 512, 384, 12, 3, 0, True, 41), (70, 256, 192, 8, 2, 1, True, 42),
             (300, 512, 384, 12, 3, 0, True, 41)]
    for T, d, F, E, k, score, renorm, seed in cases:
        print(f"static workspace: T={T} d={d} F={F} E={E} k={k}", flush=True)
        cfg, x, lg, wgu, wd = parity.make_case(T, d, F, E, k, score=score, renorm=renorm, seed=seed)
        got, want = _both(x, lg, wgu, wd, k, renorm, score)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (T, d, F, E, k)
        ref = parity.oracle_out(x, lg, wgu, wd, k, score, renorm)
        parity.check_out(got, ref, f"static T={T}",
                         floor=parity.format_floor(x, lg, wgu, wd, k, score, renorm, ref))


def test_static_workspace_at_workload_sizes():
    """The Mixtral-shaped T=512 workload (its workspace near a quarter of
    the array), the skewed T=512 one (whose gate/up GEMM runs over the
    variable-size block table the routing kernels merge, in the array),
    skewed T=128 (the table not merged: its count alone is written over the
    previous call's), then the tiny one: byte-equal to moe_forward; then a
    problem too large for the array is refused with MOE_ERR_STATIC_LIMIT."""
    for name in ("mixtral_512", "skewed_512", "skewed_128", "tiny"):
        print(f"static workspace: {name}", flush=True)
        cfg = synth.CONFIGS[name]
        x, lg, wgu, wd = synth.make_inputs(cfg, 0, DEV)
        got, want = _both(x, lg, wgu, wd, cfg.top_k, cfg.renormalize, cfg.score)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), name
        del x, lg, wgu, wd, got, want
        torch.cuda.empty_cache()
    # 4096 tokens of 4096 hidden, 8 experts of ffn 14336: ~500 MB of workspace
    T, d, F, E = 4096, 4096, 14336, 8
    x = torch.zeros(T, d, dtype=torch.bfloat16, device=DEV)
    lg = torch.zeros(T, E, device=DEV)
    wgu = torch.zeros(E, 2 * F, d, dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros(E, d, F, dtype=torch.bfloat16, device=DEV)
    out = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
    assert moe.moe_workspace_size(T, d, F, E, 2) > moe.MOE_STATIC_WORKSPACE_BYTES
    with pytest.raises(moe.MoeError) as e:
        moe.moe_forward_static(x, lg, wgu, wd, 2, True, out)
    assert e.value.status == -8
