"""Pins P2, P3, P5, P8: the oracle's routing against library closed forms,
invariants and adversarial ties.

Definitions ([R] = the Pith review of "Cross-Platform Fused MoE Dispatch in
Triton"): tokens are scored and reordered onto experts ("The reading"); fixed
blocks of rows are mapped to (expert, token-offset) pairs ("What carries the
argument"; Algorithm 1 in the "Referee Report").  Readings used: ties go to
the lower expert index; rows within one expert keep ascending flat index;
blocks never span experts.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.special import expit, softmax

import oracle
from tests.dense_reference import topk_lexsort


def _route_all(logits, k, score, renorm, BM):
    ids, w = oracle.route(logits, k, score, renorm)
    E = logits.shape[1]
    counts, offsets = oracle.counts_offsets(ids, E)
    perm, inv = oracle.permute(ids, E, offsets)
    blocks, nb = oracle.block_table(counts, offsets, BM)
    return ids, w, counts, offsets, perm, inv, blocks, nb


def _closed_forms(ids, E, BM):
    flat = ids.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.argsort(perm, kind="stable").astype(np.int32)
    nb = int(sum(-(-int(c) // BM) for c in counts))
    return counts, offsets, perm, inv, nb


def _check_invariants(ids, w, counts, offsets, perm, inv, blocks, nb, E, k, BM, renorm):
    T = ids.shape[0]
    A = T * k
    assert np.array_equal(np.sort(perm), np.arange(A))           # bijection
    assert np.array_equal(inv[perm], np.arange(A))                # inv o perm = id
    assert int(counts.sum()) == A == int(offsets[E])
    for t in range(T):
        assert len(set(ids[t].tolist())) == k                     # distinct per token
    flat = ids.reshape(-1)
    for p in range(A):                                            # sorted by expert
        e = flat[perm[p]]
        assert offsets[e] <= p < offsets[e + 1]
    covered = np.zeros(A, dtype=np.int32)                         # blocks tile once
    for b in range(nb):
        e, r0 = blocks[b]
        r1 = min(r0 + BM, offsets[e + 1])
        assert offsets[e] <= r0 < offsets[e + 1]
        covered[r0:r1] += 1
    assert np.all(covered == 1)
    assert np.all(np.diff(w, axis=1) <= 0)                        # non-increasing in j
    if renorm:
        assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1.0) <= 4 * k * 2.0 ** -24)


@settings(max_examples=60, deadline=None)
@given(T=st.integers(0, 40), E=st.integers(1, 40), kk=st.integers(1, 16),
       BM=st.sampled_from([1, 3, 16, 32, 64]), score=st.sampled_from([0, 1]),
       renorm=st.booleans(), ties=st.booleans(), seed=st.integers(0, 2**31 - 1))
def test_routing_closed_forms_and_invariants(T, E, kk, BM, score, renorm, ties, seed):
    k = min(kk, E)
    rng = np.random.default_rng(seed)
    if ties:
        logits = rng.choice(np.array([-1.0, -0.0, 0.0, 1.0], dtype=np.float32), size=(T, E))
    else:
        logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w, counts, offsets, perm, inv, blocks, nb = _route_all(logits, k, score, renorm, BM)
    assert np.array_equal(ids, topk_lexsort(logits, k))          # P2 top-k
    c2, o2, p2, i2, nb2 = _closed_forms(ids, E, BM)
    assert np.array_equal(counts, c2) and np.array_equal(offsets, o2)
    assert np.array_equal(perm, p2) and np.array_equal(inv, i2)
    assert nb == nb2
    _check_invariants(ids, w, counts, offsets, perm, inv, blocks, nb, E, k, BM, renorm)


@pytest.mark.parametrize("score,renorm", [(0, True), (0, False), (1, True), (1, False)])
def test_weights_closed_form(score, renorm):
    """P5: fp32 weights against scipy float64 softmax / expit."""
    rng = np.random.default_rng(99)
    T, E, k = 200, 64, 8
    logits = (3 * rng.standard_normal((T, E))).astype(np.float32)
    ids, w = oracle.route(logits, k, score, renorm)
    l64 = logits.astype(np.float64)
    sel = np.take_along_axis(l64, ids.astype(np.int64), axis=1)
    if score == 0:
        ref = softmax(sel, axis=1) if renorm else np.take_along_axis(softmax(l64, axis=1), ids.astype(np.int64), axis=1)
    else:
        ref = expit(sel)
        if renorm:
            ref = ref / ref.sum(axis=1, keepdims=True)
    assert np.max(np.abs(w - ref) / np.abs(ref)) <= 1e-6


def test_topk_hand_worked_ties():
    """P8 by hand: equal logits rank the lower expert first; -0.0 == +0.0."""
    logits = np.array([
        [0.0, 0.0, 0.0, 0.0],        # all tied -> 0,1,2
        [-0.0, 0.0, -1.0, -0.0],     # signed zeros tie -> 0,1,3
        [1.0, 2.0, 2.0, -5.0],       # 2.0 twice -> 1,2 then 0
        [-3.0, -2.0, -1.0, -1.0],    # -> 2,3,1
    ], dtype=np.float32)
    ids = oracle.select_topk(logits, 3)
    assert ids.tolist() == [[0, 1, 2], [0, 1, 3], [1, 2, 0], [2, 3, 1]]


def test_permutation_and_blocks_hand_worked():
    """Hand-worked reorder and block table for 3 tokens, k=2, E=3, BM=2.
    ids (flat) = [2,0 | 0,2 | 2,1]  -> counts [2,1,3], offsets [0,2,3,6];
    expert 0 rows take flat 1,2; expert 1 takes flat 5; expert 2 takes 0,3,4.
    perm = [1,2,5,0,3,4]; inv = [3,0,1,4,5,2];
    blocks (BM=2) = (0,0) (1,2) (2,3) (2,5)."""
    ids = np.array([[2, 0], [0, 2], [2, 1]], dtype=np.int32)
    counts, offsets = oracle.counts_offsets(ids, 3)
    perm, inv = oracle.permute(ids, 3, offsets)
    blocks, nb = oracle.block_table(counts, offsets, 2)
    assert counts.tolist() == [2, 1, 3]
    assert offsets.tolist() == [0, 2, 3, 6]
    assert perm.tolist() == [1, 2, 5, 0, 3, 4]
    assert inv.tolist() == [3, 0, 1, 4, 5, 2]
    assert nb == 4 and blocks.tolist() == [[0, 0], [1, 2], [2, 3], [2, 5]]


def test_empty_experts_have_no_blocks():
    ids = np.array([[3, 1]] * 5, dtype=np.int32)
    counts, offsets = oracle.counts_offsets(ids, 6)
    blocks, nb = oracle.block_table(counts, offsets, 4)
    assert counts.tolist() == [0, 5, 0, 5, 0, 0]
    assert blocks.tolist() == [[1, 0], [1, 4], [3, 5], [3, 9]] and nb == 4


def test_weights_hand_worked():
    """Closed forms by hand: two tied selected logits share 1/2 each;
    sigmoid(0) = 1/2; k = 1 with renormalisation gives exactly 1."""
    l = np.array([[0.0, 0.0, -5.0]], dtype=np.float32)
    _, w = oracle.route(l, 2, 0, True)
    assert w.tolist() == [[0.5, 0.5]]
    _, w = oracle.route(np.zeros((1, 4), np.float32), 2, 1, False)
    assert w.tolist() == [[0.5, 0.5]]
    _, w = oracle.route(np.zeros((1, 4), np.float32), 2, 0, False)
    assert w.tolist() == [[0.25, 0.25]]
    rng = np.random.default_rng(3)
    for score in (0, 1):
        _, w = oracle.route(rng.standard_normal((50, 9)).astype(np.float32), 1, score, True)
        assert np.all(w == 1.0)


def test_sigmoid_saturation_keeps_logit_order():
    """Large logits saturate sigmoid to 1.0f; selection still follows the
    logits (reading: the key is the raw logit), so the order is unique."""
    l = np.array([[20.0, 30.0, 25.0, -1.0]], dtype=np.float32)
    ids, w = oracle.route(l, 3, 1, False)
    assert ids.tolist() == [[1, 2, 0]]
    assert np.all(w == 1.0)


def test_block_order_hand_worked():
    """Blocks (BM=2) of the hand-worked case above hold 2, 1, 2, 1 rows:
    longest first, equal counts in block order -> 0, 2, 1, 3."""
    ids = np.array([[2, 0], [0, 2], [2, 1]], dtype=np.int32)
    counts, offsets = oracle.counts_offsets(ids, 3)
    blocks, nb = oracle.block_table(counts, offsets, 2)
    assert oracle.block_order(blocks, offsets, 2).tolist() == [0, 2, 1, 3]


def test_block_order_is_the_stable_sort_by_rows():
    """Against numpy's stable argsort of the negated row counts, and the
    pairwise definition (a permutation; rows non-increasing; equal rows in
    ascending block index), on skewed random routings."""
    rng = np.random.default_rng(21)
    for trial in range(40):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, min(E, 6) + 1))
        T = int(rng.integers(0, 300))
        BM = int(rng.choice([1, 2, 3, 16, 32, 64, 128, 192]))
        bias = -2.0 * np.log(rng.permutation(E) + 1.0)
        lg = (rng.standard_normal((T, E)) + bias).astype(np.float32)
        ids, _ = oracle.route(lg, k, 0, True)
        counts, offsets = oracle.counts_offsets(ids, E)
        blocks, nb = oracle.block_table(counts, offsets, BM)
        order = oracle.block_order(blocks, offsets, BM)
        rows = np.array([min(BM, offsets[e + 1] - r0) for e, r0 in blocks], dtype=np.int64)
        assert order.tolist() == np.argsort(-rows, kind="stable").tolist(), trial
        assert sorted(order.tolist()) == list(range(nb))
        for a, b in zip(order[:-1], order[1:]):
            assert rows[a] > rows[b] or (rows[a] == rows[b] and a < b)


# ---------------------------------------------- variable block size per expert

_EDGES = np.array([129, 0, 256, 257, 1, 384, 128, 130], dtype=np.int32)


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def test_var_block_table_hand_worked():
    """Experts of 129, 0, 256, 257, 1, 384, 128 and 130 rows at BM = 128:
    merged, every expert past 128 rows takes 256-row blocks (the last holding
    the rest), the others 128-row blocks -- worked by hand.  The fixed
    cutting has 2+0+2+3+1+3+1+2 = 14 blocks, the merged one 9."""
    off = _offsets(_EDGES)
    want = [[0, 0, 129],
            [2, 129, 256],
            [3, 385, 256], [3, 641, 1],
            [4, 642, 1],
            [5, 643, 256], [5, 899, 128],
            [6, 1027, 128],
            [7, 1155, 130]]
    vb, n = oracle.var_block_table(_EDGES, off, 128, 4, 2)      # mode 2: always merged
    assert n == 9 and vb.tolist() == want
    # mode 1: merged only when 14 * tiles > round >= 9 * tiles
    assert oracle.var_block_table(_EDGES, off, 128, 4, 1) == (None, -1)     # 56: one round
    assert oracle.var_block_table(_EDGES, off, 128, 18, 1) == (None, -1)    # 252: one round
    assert oracle.var_block_table(_EDGES, off, 128, 19, 1)[1] == 9          # 266 -> 171
    assert oracle.var_block_table(_EDGES, off, 128, 28, 1)[1] == 9          # 392 -> 252
    assert oracle.var_block_table(_EDGES, off, 128, 29, 1) == (None, -1)    # 406 -> 261
    assert oracle.var_block_table(_EDGES, off, 128, 28, 1, round_wgs=252)[1] == 9
    assert oracle.var_block_table(_EDGES, off, 128, 28, 1, round_wgs=251) == (None, -1)


def test_var_block_table_covers_every_row_once():
    """On skewed random routings, merged always: the blocks tile each
    expert's rows [offsets[e], offsets[e+1]) in order without gap or
    overlap, hold at most 2 BM rows (at most BM for an expert of at most BM
    rows, where they equal the fixed table's blocks), and are no more than
    the fixed table's."""
    rng = np.random.default_rng(23)
    for trial in range(40):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, min(E, 6) + 1))
        T = int(rng.integers(0, 600))
        BM = int(rng.choice([16, 64, 128]))
        bias = -2.0 * np.log(rng.permutation(E) + 1.0)
        lg = (rng.standard_normal((T, E)) + bias).astype(np.float32)
        ids, _ = oracle.route(lg, k, 0, True)
        counts, offsets = oracle.counts_offsets(ids, E)
        fixed, nf = oracle.block_table(counts, offsets, BM)
        vb, n = oracle.var_block_table(counts, offsets, BM, 1, 2)
        assert n <= nf, trial
        vb = vb.reshape(-1, 3)
        for e in range(E):
            mine = vb[vb[:, 0] == e]
            at = int(offsets[e])
            for _, r0, rows in mine:
                assert r0 == at and 0 < rows <= (2 * BM if counts[e] > BM else BM), trial
                at += int(rows)
            assert at == offsets[e + 1], trial
            if counts[e] <= BM:
                assert [(int(a), int(b)) for a, b, _ in mine] == \
                    [(int(a), int(b)) for a, b in fixed[fixed[:, 0] == e]], trial
        assert vb[:, 0].tolist() == sorted(vb[:, 0].tolist()), trial
