"""Seeded synthetic inputs for the MoE forward path.

This module generates inputs only: it holds none of the method's arithmetic
(no routing, no GEMM, no combination).  The tests, the smoke check and the
benchmark feed the same bytes to the HIP library and to the CPU oracle.

Workload shapes follow the model-shaped configurations that the Pith review
of "Cross-Platform Fused MoE Dispatch in Triton" names in its "Core claim"
and "Referee Report" (Mixtral-, Qwen2-MoE- and DeepSeek-V3-shaped layers) and
the skewed regime of "What would settle it" (64 experts, top-4, Zipf-like
alpha = 2 expert popularity, 128-512 tokens).  The exact sizes are:

  tiny       T=64   d=256  F=512   E=8   k=2  softmax over selected (renorm)
  mixtral    T=128/256/512, d=4096 F=14336 E=8 k=2 softmax over selected
  qwen2      T=128/256/512, d=3584 F=2560  E=64 k=8 full softmax, no renorm
  skewed     T=128/256/512, d=2048 F=1408  E=64 k=4 softmax over selected,
             logits + per-expert bias -2*ln(rank_e), rank a seeded permutation
  dsv3       T=512/4096,    d=7168 F=2048  E=256 k=8 sigmoid, renormalised

Distributions: x ~ N(0,1) bf16 [T,d]; logits ~ N(0,1) fp32 [T,E];
W_gate_up[e] ~ N(0, 1/d) bf16 [2F,d] (gate rows first, then up rows);
W_down[e] ~ N(0, 1/F) bf16 [d,F].  Every draw is fp32 ``torch.randn`` scaled
and then rounded to bf16 by torch (round-to-nearest-even).

Seeds: base S; x <- S+1, logits <- S+2, skew ranks <- S+3,
W_gate_up[e] <- S+1000+e, W_down[e] <- S+2000+e.  Weights are drawn on the
device they are generated on (torch's CPU and GPU generators give different
streams for one seed), so a run records the device it drew on.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import torch

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    ffn: int
    E: int
    top_k: int
    score: int          # SCORE_SOFTMAX or SCORE_SIGMOID
    renormalize: bool
    skew_alpha: float = 0.0   # > 0: add -alpha*ln(rank_e) to expert e's logits

    @property
    def rows(self) -> int:
        return self.T * self.top_k

    def weight_bytes(self) -> int:
        return self.E * 6 * self.ffn * self.d


def _mk(name, T, d, ffn, E, k, score, renorm, skew=0.0):
    return MoEConfig(name, T, d, ffn, E, k, score, renorm, skew)


CONFIGS = {
    "tiny": _mk("tiny", 64, 256, 512, 8, 2, SCORE_SOFTMAX, True),
    **{f"mixtral_{T}": _mk(f"mixtral_{T}", T, 4096, 14336, 8, 2, SCORE_SOFTMAX, True)
       for T in (128, 256, 512)},
    **{f"qwen2_{T}": _mk(f"qwen2_{T}", T, 3584, 2560, 64, 8, SCORE_SOFTMAX, False)
       for T in (128, 256, 512)},
    **{f"skewed_{T}": _mk(f"skewed_{T}", T, 2048, 1408, 64, 4, SCORE_SOFTMAX, True, 2.0)
       for T in (128, 256, 512)},
    **{f"dsv3_{T}": _mk(f"dsv3_{T}", T, 7168, 2048, 256, 8, SCORE_SIGMOID, True)
       for T in (512, 4096)},
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_x(cfg: MoEConfig, seed: int = 0, device="cpu") -> torch.Tensor:
    g = _gen(seed + 1, "cpu")
    x = torch.randn(cfg.T, cfg.d, generator=g, dtype=torch.float32)
    return x.to(torch.bfloat16).to(device)


def make_logits(cfg: MoEConfig, seed: int = 0, device="cpu") -> torch.Tensor:
    g = _gen(seed + 2, "cpu")
    logits = torch.randn(cfg.T, cfg.E, generator=g, dtype=torch.float32)
    if cfg.skew_alpha > 0.0:
        gr = _gen(seed + 3, "cpu")
        rank = torch.randperm(cfg.E, generator=gr).to(torch.float64) + 1.0
        bias = (-cfg.skew_alpha * torch.log(rank)).to(torch.float32)
        logits = logits + bias[None, :]
    return logits.to(device)


def make_weights(cfg: MoEConfig, seed: int = 0, device="cpu"):
    """Returns (W_gate_up bf16 [E,2F,d], W_down bf16 [E,d,F]) on ``device``,
    drawn one expert at a time on that device."""
    E, d, F = cfg.E, cfg.d, cfg.ffn
    wgu = torch.empty(E, 2 * F, d, dtype=torch.bfloat16, device=device)
    wd = torch.empty(E, d, F, dtype=torch.bfloat16, device=device)
    sg = 1.0 / math.sqrt(d)
    sd = 1.0 / math.sqrt(F)
    for e in range(E):
        g1 = _gen(seed + 1000 + e, device)
        wgu[e].copy_((torch.randn(2 * F, d, generator=g1, device=device) * sg).to(torch.bfloat16))
        g2 = _gen(seed + 2000 + e, device)
        wd[e].copy_((torch.randn(d, F, generator=g2, device=device) * sd).to(torch.bfloat16))
    return wgu, wd


def make_router_weight(cfg: MoEConfig, seed: int = 0, device="cpu") -> torch.Tensor:
    """Router matrix W_r bf16 [E, d] ~ N(0, 1/d), drawn on the CPU, so that
    x . W_r^T has unit-variance scores for x ~ N(0, 1)."""
    g = _gen(seed + 5, "cpu")
    w = torch.randn(cfg.E, cfg.d, generator=g, dtype=torch.float32) / math.sqrt(cfg.d)
    return w.to(torch.bfloat16).to(device)


def make_inputs(cfg: MoEConfig, seed: int = 0, device="cpu", weight_device=None):
    """All four inputs.  x and logits are drawn on the CPU and moved;
    weights are drawn on ``weight_device`` (default: ``device``)."""
    wdev = device if weight_device is None else weight_device
    x = make_x(cfg, seed, device)
    logits = make_logits(cfg, seed, device)
    wgu, wd = make_weights(cfg, seed, wdev)
    if torch.device(wdev) != torch.device(device):
        wgu, wd = wgu.to(device), wd.to(device)
    return x, logits, wgu, wd


def bf16_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")


def sha256(t: torch.Tensor) -> str:
    a = t.detach().contiguous().cpu()
    if a.dtype == torch.bfloat16:
        a = a.view(torch.int16)
    return hashlib.sha256(a.numpy().tobytes()).hexdigest()
