"""What the data formats of the GPU path alone cost in accuracy (test-only).

The HIP path stores the SwiGLU intermediate h in bf16 (it is the next
matrix product's operand) and writes the output in bf16; the unfused SwiGLU
ablation also stores the gate and up products in bf16.  This module computes
the MoE output in float64 with exactly those roundings and no other error
(every product and sum exact to float64), using the oracle's routing (ids
and fp32 weights).  The difference between that and the oracle's fp32 result
is the error that the formats force on any implementation, element by
element: the "format floor" the parity checks allow where the required
max-abs bound cannot be met by the format itself (small ffn, rows whose
routing weights sum far from one, the ablation's extra roundings).

With ``rounding=None`` the model is the plain MoE output in float64; the
CPU tests pin it against the oracle there, and pin the roundings against
torch's float32 -> bfloat16 conversion (round to nearest even).

Definitions: [R] = the Pith review of "Cross-Platform Fused MoE Dispatch in
Triton"; SwiGLU expert FFN and weighted combination ("The reading", "What
carries the argument"); the unfused sequence of global reads and writes the
fusion removes ("Referee Report", minor comment 1 on section 3.3).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

FORMATS = (None, "fused", "unfused")


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 (round to nearest) -> bfloat16 (round to nearest
    even, torch's conversion), returned as float64: the path a GPU value
    takes from an fp32 accumulator to a bf16 store."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def _silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def moe_output(x, logits, wgu, wd, k, score, renorm, tokens=None, rounding="fused"):
    """float64 MoE output [n, d] (before the output rounding) for the listed
    tokens (all when None), with the bf16 roundings of ``rounding``:
    None (none), "fused" (h), "unfused" (g, u and h).  x, logits, wgu, wd as
    for the parity checks (torch tensors on any device)."""
    assert rounding in FORMATS
    lg = logits.detach().cpu().numpy()
    T = lg.shape[0]
    F = wd.shape[2]
    ids, w = oracle.route(lg, k, score, renorm)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    xs = _f64(x)
    acc = np.zeros((len(toks), xs.shape[1]))
    sub_ids = ids[toks]
    for e in np.unique(sub_ids):
        rows, js = np.nonzero(sub_ids == e)          # (token slot, j) pairs routed to e
        X = xs[toks[rows]]
        Wgu = _f64(wgu[int(e)])
        G = X @ Wgu[:F].T
        U = X @ Wgu[F:].T
        if rounding == "unfused":
            G, U = bf16_round(G), bf16_round(U)
        H = _silu(G) * U
        if rounding is not None:
            H = bf16_round(H)
        Y = H @ _f64(wd[int(e)]).T
        wt = w[toks[rows], js].astype(np.float64)[:, None]
        acc[rows] += wt * Y   # a token appears once per expert
    return acc


def floor(model_out: np.ndarray, ref32: np.ndarray) -> np.ndarray:
    """Per element, the error the formats allow: the distance from the
    oracle of the model's value before the output rounding, plus half a
    bf16 ulp of that value (the output rounding, whichever way it goes; the
    ulp of the binade above where the value lies within 2^-7 below a power
    of two, in case an implementation's value crosses it)."""
    from tests.parity import bf16_half_ulp

    m = np.asarray(model_out, dtype=np.float64)
    return np.abs(m - np.asarray(ref32, dtype=np.float64)) + bf16_half_ulp(np.abs(m) * (1 + 2.0 ** -7))
