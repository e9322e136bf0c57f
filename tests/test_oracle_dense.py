"""Pin P1: the oracle's FFN and combination against a float64 dense brute force.

The brute force (tests/dense_reference.py) evaluates every expert for every
token with matrix operations and masks by the routing; the oracle loops over
tokens and their k experts.  Shapes use d != F and E > k so a transposed
operand, a swapped gate/up half or a dropped expert all fail.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from tests.dense_reference import dense_moe_f64


def _rand_case(rng, T, E, k, d, F):
    x = rng.standard_normal((T, d)).astype(np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    wgu = (rng.standard_normal((E, 2 * F, d)) / np.sqrt(d)).astype(np.float32)
    wd = (rng.standard_normal((E, d, F)) / np.sqrt(F)).astype(np.float32)
    return oracle.round_bf16(x), logits, oracle.round_bf16(wgu), oracle.round_bf16(wd)


def _rel_fro(a, b):
    return np.linalg.norm((np.asarray(a, np.float64) - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300)


@pytest.mark.parametrize("score,renorm", [(0, True), (0, False), (1, True), (1, False)])
def test_oracle_matches_dense_fixed(score, renorm):
    rng = np.random.default_rng(1234 + 2 * score + renorm)
    T, E, k, d, F = 23, 7, 3, 40, 24
    x, logits, wgu, wd = _rand_case(rng, T, E, k, d, F)
    res = oracle.forward(x, logits, wgu, wd, k, renorm, score, F)
    ref = dense_moe_f64(x, logits, wgu, wd, k, score, renorm)
    assert _rel_fro(res["ref32"], ref) <= 1e-5


@settings(max_examples=40, deadline=None)
@given(T=st.integers(1, 20), E=st.integers(1, 10), kk=st.integers(1, 10),
       d=st.sampled_from([8, 16, 24, 40]), F=st.sampled_from([8, 12, 32]),
       score=st.sampled_from([0, 1]), renorm=st.booleans(), seed=st.integers(0, 2**31 - 1))
def test_oracle_matches_dense_random(T, E, kk, d, F, score, renorm, seed):
    k = min(kk, E)
    rng = np.random.default_rng(seed)
    x, logits, wgu, wd = _rand_case(rng, T, E, k, d, F)
    res = oracle.forward(x, logits, wgu, wd, k, renorm, score, F)
    ref = dense_moe_f64(x, logits, wgu, wd, k, score, renorm)
    assert _rel_fro(res["ref32"], ref) <= 1e-5


def test_oracle_token_subset_equals_full_rows():
    rng = np.random.default_rng(7)
    T, E, k, d, F = 16, 6, 2, 24, 16
    x, logits, wgu, wd = _rand_case(rng, T, E, k, d, F)
    ids, w = oracle.route(logits, k, 0, True)
    full = oracle.ffn(x, ids, w, wgu, wd, F)
    toks = np.array([13, 2, 2, 0], dtype=np.int32)
    part = oracle.ffn(x, ids, w, wgu, wd, F, tokens=toks)
    assert np.array_equal(part, full[toks])


def test_oracle_per_expert_weights_may_be_sparse():
    """Experts no listed token routes to may be passed as None."""
    rng = np.random.default_rng(8)
    T, E, k, d, F = 8, 6, 2, 16, 8
    x, logits, wgu, wd = _rand_case(rng, T, E, k, d, F)
    ids, w = oracle.route(logits, k, 0, True)
    toks = np.array([3], dtype=np.int32)
    used = set(int(e) for e in ids[3])
    wgu_l = [wgu[e] if e in used else None for e in range(E)]
    wd_l = [wd[e] if e in used else None for e in range(E)]
    a = oracle.ffn(x, ids, w, wgu_l, wd_l, F, tokens=toks)
    b = oracle.ffn(x, ids, w, wgu, wd, F, tokens=toks)
    assert np.array_equal(a, b)
    unused = [e for e in range(E) if e not in used]
    if unused:
        with pytest.raises(ValueError):
            bad = list(wgu_l)
            bad[int(ids[3][0])] = None
            oracle.ffn(x, ids, w, bad, wd_l, F, tokens=toks)
