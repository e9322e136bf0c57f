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


def test_beyond_format_keeps_real_errors():
    """Measuring beyond the format's rounding forgives exactly that rounding:
    a correctly rounded heavy-tailed output passes, one ulp more fails."""
    rng = np.random.default_rng(4)
    ref = rng.standard_normal((16, 64)).astype(np.float32)
    ref[3, 5] = 9.7  # far above the RMS
    out = torch.from_numpy(ref).bfloat16()
    _, plain = parity.errors(out, ref)
    _, beyond = parity.errors(out, ref, beyond_format=True)
    assert beyond == 0.0 and plain > 0
    bad = out.clone()
    bad[3, 5] = torch.tensor(9.7 + 0.25).bfloat16()
    _, beyond_bad = parity.errors(bad, ref, beyond_format=True)
    assert beyond_bad > 2e-2
