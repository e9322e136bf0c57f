"""Host checks of the parity helpers' own arithmetic."""
import numpy as np
import torch

from tests import parity


def test_bf16_half_ulp_bounds_rounding():
    """The half-ulp allowance covers bf16's round-to-nearest error of any
    value, and is tight (some values use almost all of it)."""
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    r = torch.from_numpy(v).bfloat16().float().numpy().astype(np.float64)
    hu = parity.bf16_half_ulp(v)
    assert np.all(np.abs(r - v) <= hu)
    assert np.max(np.abs(r - v) / hu) > 0.99
    assert parity.bf16_half_ulp(np.array([0.0, 1.0, -1.5, 2.0]))[1:].tolist() == [2**-8, 2**-8, 2**-7]


def test_floor_bound_forgives_only_the_floor():
    """With per-element floors the max-abs check allows each element its
    floor plus FLOOR_EPS of max(RMS, row RMS) where that exceeds the
    required bound, and nothing more: a correctly rounded heavy-tailed
    output passes, a few row-scale slacks more fails."""
    rng = np.random.default_rng(4)
    ref = rng.standard_normal((16, 64)).astype(np.float32)
    ref[3, 5] = 9.968  # far above the RMS, near a rounding midpoint: its bf16 error exceeds 2e-2 * RMS
    out = torch.from_numpy(ref).bfloat16()
    _, plain = parity.errors(out, ref)
    assert plain > parity.MAX_ABS_TOL
    floor = parity.bf16_half_ulp(ref.astype(np.float64))
    _, scaled = parity.errors(out, ref, floor)
    assert scaled <= parity.MAX_ABS_TOL
    rms = np.sqrt(np.mean(ref.astype(np.float64) ** 2))
    row = np.sqrt(np.mean(ref[3].astype(np.float64) ** 2))
    bad = out.clone().float()
    bad[3, 5] = float(ref[3, 5]) + floor[3, 5] + 3 * parity.FLOOR_EPS * max(rms, row)
    _, scaled_bad = parity.errors(bad, ref, floor)
    assert scaled_bad > parity.MAX_ABS_TOL
    # an ordinary element is held to the required bound whatever its floor
    bad2 = out.clone().float()
    bad2[0, 0] = float(ref[0, 0]) + 0.03 * rms
    _, e2 = parity.errors(bad2, ref, floor)
    assert e2 > parity.MAX_ABS_TOL
