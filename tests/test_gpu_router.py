"""GPU parity of the router scores (logits = x . W_r^T) and of the forward
pass from hidden states, through the C ABI, against the CPU oracle.

Scores: the oracle's fp64 sum rounded once to fp32 is the exact dot product
to well within one fp32 ulp; the GPU sums bf16 products (exact in fp32) in
fp32 in some order, so |gpu - exact| <= gamma_d * sum_c |x_c w_c| with
gamma_d = d*u/(1 - d*u), u = 2^-24, whatever the order.  The tests allow
that bound plus one ulp of the result.

Forward from hidden states: the expert choice is an integer decided by the
fp32 scores, so the oracle routes the GPU's own scores (both sides decide in
the same precision) and the output meets the forward tolerance.
"""
import numpy as np
import pytest
import torch

import expert_dispatch_router_amd as moe
import oracle
from expert_dispatch_router_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"
U = 2.0 ** -24


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _router_case(T, d, E, seed):
    cfg = synth.MoEConfig("router", T, d, 64, E, 1, 0, True)
    x = synth.make_x(cfg, seed, DEV)
    wr = synth.make_router_weight(cfg, seed, DEV)
    return x, wr


def _check_scores(got, x, wr):
    xb = parity.to_np_u16(x)
    wb = parity.to_np_u16(wr)
    ref = oracle.router_logits(xb, wb).astype(np.float64)
    mag = np.abs(oracle.bf16_to_f32(xb).astype(np.float64)) @ \
        np.abs(oracle.bf16_to_f32(wb).astype(np.float64)).T
    d = xb.shape[1]
    bound = (d * U / (1 - d * U)) * mag + U * np.abs(ref) + 1e-30
    g = got.detach().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape
    err = np.abs(g - ref)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3f}"
    return ref


@pytest.mark.parametrize("T,d,E", [(1, 64, 1), (17, 128, 6), (100, 512, 60), (33, 1024, 256),
                                   (40, 7168, 256), (5, 64, 512), (300, 256, 16), (64, 4096, 8),
                                   (130, 2048, 33), (513, 1024, 17), (97, 3584, 64),
                                   (1030, 192, 130), (1024, 64, 16), (2000, 320, 40),
                                   (1100, 7168, 256), (1024, 64, 128), (1300, 1024, 144),
                                   (2049, 512, 512), (1500, 4096, 160)])
def test_router_scores_within_the_summation_bound(T, d, E):
    """Shapes with one part and with the reduction split in several (the
    partial sums added in order), ragged in tokens and experts, for every
    wave tile (16..64 tokens x 16..64 experts) and for the LDS-staged tile
    of large problems (T >= 1024, E >= 128 a multiple of 16: one K step,
    a partial column tile, two column tiles, a last block of one row)."""
    x, wr = _router_case(T, d, E, seed=T + d + E)
    got = moe.moe_router_logits(x, wr)
    _check_scores(got, x, wr)


@pytest.mark.parametrize("name", ["mixtral_512", "dsv3_512", "dsv3_4096"])
def test_router_scores_full_size(name):
    cfg = synth.CONFIGS[name]
    x = synth.make_x(cfg, 0, DEV)
    wr = synth.make_router_weight(cfg, 0, DEV)
    got = moe.moe_router_logits(x, wr)
    _check_scores(got, x, wr)


def test_router_scores_deterministic_and_stream():
    x, wr = _router_case(200, 2048, 64, seed=9)
    a = moe.moe_router_logits(x, wr)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = moe.moe_router_logits(x, wr, stream=s)
    s.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("name,per_block", [("tiny", False), ("mixtral_512", False),
                                            ("qwen2_128", False), ("dsv3_512", False),
                                            ("dsv3_4096", True)])
def test_forward_from_hidden_states(name, per_block):
    """The forward pass from hidden states at workload sizes: every token
    against the oracle on the same scores (DeepSeek-V3 T=4096: the tokens
    holding the first and last row of every schedule block, so every block
    of both GEMMs is compared)."""
    cfg = synth.CONFIGS[name]
    x = synth.make_x(cfg, 0, DEV)
    wr = synth.make_router_weight(cfg, 0, DEV)
    wgu, wd = synth.make_weights(cfg, 0, DEV)
    logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=DEV)
    out = moe.moe_forward_router(x, wr, wgu, wd, cfg.top_k, cfg.renormalize, logits_out=logits,
                                 score=cfg.score)
    # the scores written out are the router kernel's, bit for bit
    alone = moe.moe_router_logits(x, wr)
    assert torch.equal(logits.view(torch.int32), alone.view(torch.int32))
    _check_scores(logits, x, wr)
    # the rest is the forward pass on those scores, bit for bit
    ref_path = moe.moe_forward(x, logits, wgu, wd, cfg.top_k, cfg.renormalize, score=cfg.score)
    assert torch.equal(out.view(torch.int16), ref_path.view(torch.int16))
    # and meets the forward tolerance against the oracle on the same scores
    toks = None
    if per_block:
        bm, _ = moe.moe_plan(cfg.T, cfg.d, cfg.ffn, cfg.E, cfg.top_k)
        toks = parity.tokens_per_block(logits, cfg.top_k, cfg.score, cfg.renormalize, bm)
    ref = parity.oracle_out(x, logits, wgu, wd, cfg.top_k, cfg.score, cfg.renormalize, tokens=toks)
    got = out if toks is None else out[torch.from_numpy(toks).long().to(DEV)]
    parity.check_workload(got, ref, name, x, logits, wgu, wd, cfg, tokens=toks,
                          what=name + " from hidden states")
    del x, wr, wgu, wd, out
    torch.cuda.empty_cache()


def test_forward_router_without_logits_out_matches():
    cfg = synth.CONFIGS["tiny"]
    x = synth.make_x(cfg, 1, DEV)
    wr = synth.make_router_weight(cfg, 1, DEV)
    wgu, wd = synth.make_weights(cfg, 1, DEV)
    a = moe.moe_forward_router(x, wr, wgu, wd, cfg.top_k, cfg.renormalize)
    lg = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=DEV)
    b = moe.moe_forward_router(x, wr, wgu, wd, cfg.top_k, cfg.renormalize, logits_out=lg)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _random_router_shapes(n=10, seed=8642):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        T = int(rng.integers(1, 3000))
        E = int(rng.choice([1, 7, 16, 100, 128, 144, 256, 400, 512]))
        d = int(64 * rng.integers(1, 40))
        out.append((T, d, E))
    return out


@pytest.mark.parametrize("T,d,E", _random_router_shapes())
def test_router_scores_random_shapes(T, d, E):
    """Random sizes across both router tilings (the wave tiles, and the
    LDS-staged tile where T >= 1024 and E >= 128 is a multiple of 16)."""
    x, wr = _router_case(T, d, E, seed=3 * T + d + E)
    got = moe.moe_router_logits(x, wr)
    _check_scores(got, x, wr)
