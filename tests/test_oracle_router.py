"""Pins of the oracle's router scores (O0: logits = x . W_r^T) against what
the mathematics fixes, without calling the function twice for one answer:

* a basis of one-hot tokens returns W_r transposed, entry by entry (any
  transposed operand or wrong index fails it);
* bilinearity on small integers, where every sum is exact;
* a closed form for constant inputs;
* the fp64 accumulation: a term far below fp32's resolution survives a
  cancellation, and the result is the one rounding of the exact sum.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def _bf16(a):
    """fp32 values that are exact in bf16 -> bf16 bits (checked)."""
    a = np.asarray(a, dtype=np.float32)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f32(bits), a), "value not exact in bf16"
    return bits


def test_one_hot_basis_returns_the_transposed_router_matrix():
    rng = np.random.default_rng(1)
    d, E = 64, 6
    w = rng.integers(-100, 101, size=(E, d)).astype(np.float32) / 8.0   # exact in bf16
    x = np.eye(d, dtype=np.float32) * 2.0
    out = oracle.router_logits(_bf16(x), _bf16(w))
    assert out.shape == (d, E)
    assert np.array_equal(out, 2.0 * w.T)


def test_bilinear_on_small_integers():
    rng = np.random.default_rng(2)
    T, d, E = 5, 128, 9
    x1 = rng.integers(-4, 5, size=(T, d)).astype(np.float32)
    x2 = rng.integers(-4, 5, size=(T, d)).astype(np.float32)
    w1 = rng.integers(-4, 5, size=(E, d)).astype(np.float32)
    w2 = rng.integers(-4, 5, size=(E, d)).astype(np.float32)
    L = lambda x, w: oracle.router_logits(_bf16(x), _bf16(w)).astype(np.float64)
    # every partial sum is an integer below 2^24: all results are exact
    assert np.array_equal(L(x1 + x2, w1), L(x1, w1) + L(x2, w1))
    assert np.array_equal(L(x1, w1 - w2), L(x1, w1) - L(x1, w2))
    assert np.array_equal(L(3 * x1, w1), 3 * L(x1, w1))
    # symmetry of the Gram matrix: scoring W against itself
    g = L(w1, w1)
    assert np.array_equal(g, g.T)
    assert np.array_equal(np.diag(g), (w1.astype(np.float64) ** 2).sum(1))


def test_constant_inputs_closed_form():
    T, d, E = 3, 4096, 2
    x = np.full((T, d), 0.375, np.float32)
    w = np.full((E, d), -1.25, np.float32)
    out = oracle.router_logits(_bf16(x), _bf16(w))
    assert np.all(out == np.float32(d * 0.375 * -1.25))


def test_sums_in_fp64_then_rounds_once():
    d = 64
    x = np.zeros((1, d), np.float32)
    w = np.zeros((2, d), np.float32)
    x[0, :3] = [1.0, 2.0 ** -30, -1.0]
    w[0, :3] = 1.0
    # an fp32 running sum would lose 2^-30 against 1.0; fp64 keeps it
    w[1, :2] = [1.0, 1.0]
    out = oracle.router_logits(_bf16(x), _bf16(w))
    assert out[0, 0] == np.float32(2.0 ** -30)
    # 1 + 2^-30 rounds to 1.0 in fp32 (round to nearest, one rounding)
    assert out[0, 1] == np.float32(1.0)


def test_empty_and_argument_errors():
    x = np.zeros((0, 64), np.uint16)
    w = np.zeros((4, 64), np.uint16)
    assert oracle.router_logits(x, w).shape == (0, 4)
    with pytest.raises(ValueError):
        oracle.router_logits(np.zeros((2, 64), np.uint16), np.zeros((4, 32), np.uint16))
