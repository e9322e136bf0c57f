"""Pins P4 and P7: special cases that reduce the oracle to a textbook SwiGLU
MLP or to exact zeros, its bf16 rounding against torch's conversion, and the
hand-worked examples stored under tests/golden/.

Definitions ([R] = the Pith review of "Cross-Platform Fused MoE Dispatch in
Triton"): SwiGLU expert FFN with gate and up projections and SiLU ("What
carries the argument"); weighted combination of the selected experts
(abstract).
"""
import glob
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(a):
    return oracle.round_bf16(np.asarray(a, dtype=np.float32))


def _f64(b):
    return oracle.bf16_to_f32(b).astype(np.float64)


def _mlp_torch(x_bits, wg_bits, wu_bits, wd_bits):
    """Textbook SwiGLU MLP with torch float64 ops: (silu(x Wg^T) * x Wu^T) Wd^T."""
    x = torch.from_numpy(_f64(x_bits))
    g = x @ torch.from_numpy(_f64(wg_bits)).T
    u = x @ torch.from_numpy(_f64(wu_bits)).T
    return ((torch.nn.functional.silu(g) * u) @ torch.from_numpy(_f64(wd_bits)).T).numpy()


def _rand(rng, *shape, scale=1.0):
    return _bits(rng.standard_normal(shape) * scale)


def _relerr(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


def test_single_expert_is_swiglu_mlp():
    rng = np.random.default_rng(0)
    T, d, F = 12, 32, 20
    x = _rand(rng, T, d)
    wgu = _rand(rng, 1, 2 * F, d, scale=d ** -0.5)
    wd = _rand(rng, 1, d, F, scale=F ** -0.5)
    logits = rng.standard_normal((T, 1)).astype(np.float32)
    for score in (0, 1):
        res = oracle.forward(x, logits, wgu, wd, 1, True, score, F)
        assert np.all(res["w"] == 1.0)
        ref = _mlp_torch(x, wgu[0, :F], wgu[0, F:], wd[0])
        assert _relerr(res["ref32"], ref) <= 1e-5


def test_identical_experts_renormalised_is_mlp():
    rng = np.random.default_rng(1)
    T, d, F, E, k = 10, 24, 16, 6, 3
    x = _rand(rng, T, d)
    one_gu = _rand(rng, 2 * F, d, scale=d ** -0.5)
    one_d = _rand(rng, d, F, scale=F ** -0.5)
    wgu = np.stack([one_gu] * E)
    wd = np.stack([one_d] * E)
    logits = (2 * rng.standard_normal((T, E))).astype(np.float32)
    ref = _mlp_torch(x, one_gu[:F], one_gu[F:], one_d)
    for score in (0, 1):
        res = oracle.forward(x, logits, wgu, wd, k, True, score, F)
        assert _relerr(res["ref32"], ref) <= 1e-5


def test_k_equals_E_full_softmax_is_dense_soft_moe():
    rng = np.random.default_rng(2)
    T, d, F, E = 9, 16, 24, 5
    x = _rand(rng, T, d)
    wgu = _rand(rng, E, 2 * F, d, scale=d ** -0.5)
    wd = _rand(rng, E, d, F, scale=F ** -0.5)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    res = oracle.forward(x, logits, wgu, wd, E, False, 0, F)
    p = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=1).numpy()
    ref = sum(p[:, e:e + 1] * _mlp_torch(x, wgu[e, :F], wgu[e, F:], wd[e]) for e in range(E))
    assert _relerr(res["ref32"], ref) <= 1e-5


def test_top1_picks_argmax_expert_mlp():
    rng = np.random.default_rng(3)
    T, d, F, E = 8, 16, 8, 4
    x = _rand(rng, T, d)
    wgu = _rand(rng, E, 2 * F, d, scale=d ** -0.5)
    wd = _rand(rng, E, d, F, scale=F ** -0.5)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    res = oracle.forward(x, logits, wgu, wd, 1, True, 0, F)
    am = np.argmax(logits, axis=1)
    ref = np.stack([_mlp_torch(x[t:t + 1], wgu[am[t], :F], wgu[am[t], F:], wd[am[t]])[0] for t in range(T)])
    assert np.all(res["w"] == 1.0)
    assert _relerr(res["ref32"], ref) <= 1e-5


def test_zero_down_or_zero_input_gives_exact_zero():
    rng = np.random.default_rng(4)
    T, d, F, E, k = 6, 16, 8, 4, 2
    x = _rand(rng, T, d)
    wgu = _rand(rng, E, 2 * F, d, scale=d ** -0.5)
    wd = _rand(rng, E, d, F, scale=F ** -0.5)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r1 = oracle.forward(x, logits, wgu, np.zeros_like(wd), k, True, 0, F)
    assert np.all(r1["ref32"] == 0.0)
    r2 = oracle.forward(np.zeros_like(x), logits, wgu, wd, k, True, 1, F)
    assert np.all(r2["ref32"] == 0.0)


def test_round_bf16_matches_torch():
    """P7: the oracle's round-to-nearest-even against torch's fp32 -> bf16."""
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2**32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    edges = np.array([0x00000000, 0x80000000, 0x00008000, 0x00018000, 0x3F808000, 0x3F818000,
                      0x3F80FFFF, 0x00000001, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0xFF7FFFFF,
                      0x7F800000, 0xFF800000, 0x7F7F8000, 0x7F7F7FFF], dtype=np.uint32)
    u = np.concatenate([u, edges])
    f = u.view(np.float32)
    got = oracle.round_bf16(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(oracle.bf16_to_f32(got[nan])))


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "hand_*.json"))))
def test_hand_worked_golden(path):
    """Hand-derived examples whose every intermediate value is exact in fp32
    and bf16 (derivation and source stored in each file)."""
    with open(path) as fh:
        g = json.load(fh)
    x = _bits(g["x"])
    wgu = _bits(g["w_gate_up"])
    wd = _bits(g["w_down"])
    logits = np.array(g["logits"], dtype=np.float32)
    res = oracle.forward(x, logits, wgu, wd, g["top_k"], g["renormalize"], g["score"], g["ffn"],
                         BM=g["block_rows"])
    exp = g["expected"]
    assert res["ids"].tolist() == exp["ids"]
    assert res["w"].tolist() == exp["w"]
    assert res["counts"].tolist() == exp["counts"]
    assert res["offsets"].tolist() == exp["offsets"]
    assert res["perm"].tolist() == exp["perm"]
    assert res["inv"].tolist() == exp["inv"]
    assert res["blocks"].tolist() == exp["blocks"]
    assert res["ref32"].tolist() == exp["out"]
    assert oracle.bf16_to_f32(res["ref16"]).tolist() == exp["out"]
