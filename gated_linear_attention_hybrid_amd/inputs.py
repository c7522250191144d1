"""Seeded synthetic workloads for the hybrid layer.

This module only draws random tensors (torch generators, fp32 draws rounded to
bf16 with round-to-nearest-even where the workload is bf16).  It holds none of
the layer's arithmetic, so the GPU library and the CPU oracle can both be fed
from it without sharing any computation.

The shapes and distributions stand in for the pages' setting: a LLaMA-3-8B-shaped
attention layer (32 heads of 128), 32K-token contexts, batch 8 at 32K ("Lizard"
summary, Results; "LT2" summary, Results).  No dataset is used.

Draw order for a prefill workload: Wphi_q, Wphi_k, meta, q, k, v, gate.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    f: int
    dv: int
    chunk: int
    window: int
    n_meta: int
    dtype: str            # "bf16" or "f32"
    x_std: float          # std of q, k, v
    gate_mean: float      # gate logits ~ N(gate_mean, gate_std)
    gate_std: float
    w_std: float          # std of the Hedgehog projections (unit-variance logits)
    seed: int
    steps: int = 0        # decode steps (decode workloads)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


_S128 = 1.0 / math.sqrt(128.0)

WORKLOADS = {
    # tiny fp32 layer: 2 heads of 64, Hedgehog 2x32, window 16
    "tiny_fp32": Workload("tiny_fp32", B=1, H=2, L=256, d=64, f=64, dv=64, chunk=64, window=16,
                          n_meta=4, dtype="f32", x_std=1.0, gate_mean=2.0, gate_std=1.0,
                          w_std=1.0 / 8.0, seed=1000),
    # LLaMA-3-8B-shaped layer prefill, 2K tokens
    "prefill_2k": Workload("prefill_2k", B=1, H=32, L=2048, d=128, f=128, dv=128, chunk=64,
                           window=64, n_meta=4, dtype="bf16", x_std=_S128, gate_mean=3.0,
                           gate_std=1.0, w_std=1.0, seed=1001),
    # long-context prefill, 32K tokens
    "prefill_32k": Workload("prefill_32k", B=1, H=32, L=32768, d=128, f=128, dv=128, chunk=64,
                            window=64, n_meta=4, dtype="bf16", x_std=_S128, gate_mean=3.0,
                            gate_std=1.0, w_std=1.0, seed=1002),
    # recurrent decode: batch 8, 32 heads, state 128x128 from a 32K-token prefix
    "decode_b8": Workload("decode_b8", B=8, H=32, L=32768, d=128, f=128, dv=128, chunk=64,
                          window=64, n_meta=4, dtype="bf16", x_std=_S128, gate_mean=3.0,
                          gate_std=1.0, w_std=1.0, seed=1003, steps=256),
    # strong decay: sigmoid(N(-2,1.5)) ~ 0.12-0.19, the cumulative gate underflows
    "strong_decay_8k": Workload("strong_decay_8k", B=8, H=32, L=8192, d=128, f=128, dv=128,
                                chunk=128, window=64, n_meta=4, dtype="bf16", x_std=_S128,
                                gate_mean=-2.0, gate_std=1.5, w_std=1.0, seed=1004),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, std, mean, gen, device, dtype):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x.to(dtype)  # RNE rounding for bf16


def make_prefill(wl: Workload, device="cpu", gate_log_zero: bool = False) -> dict:
    """Inputs of one prefill call.  Returns q, k, v, gate [B,H,L,*], wq, wk
    [H,d,f/2], meta [H,M] (fp32) on ``device``.  ``gate_log_zero`` replaces the
    gate by log-gates equal to 0 (Gamma = 1, ungated linear attention)."""
    dev = torch.device(device)
    gen = _gen(wl.seed, dev)
    dt = wl.torch_dtype
    B, H, L = wl.B, wl.H, wl.L
    out = {}
    out["wq"] = _randn((H, wl.d, wl.f // 2), wl.w_std, 0.0, gen, dev, dt)
    out["wk"] = _randn((H, wl.d, wl.f // 2), wl.w_std, 0.0, gen, dev, dt)
    out["meta"] = _randn((H, wl.n_meta), 1.0, 0.0, gen, dev, torch.float32)
    out["q"] = _randn((B, H, L, wl.d), wl.x_std, 0.0, gen, dev, dt)
    out["k"] = _randn((B, H, L, wl.d), wl.x_std, 0.0, gen, dev, dt)
    out["v"] = _randn((B, H, L, wl.dv), wl.x_std, 0.0, gen, dev, dt)
    if gate_log_zero:
        out["gate"] = torch.zeros((B, H, L, wl.f), device=dev, dtype=dt)
    else:
        out["gate"] = _randn((B, H, L, wl.f), wl.gate_std, wl.gate_mean, gen, dev, dt)
    return out


def make_decode_token(wl: Workload, step: int, device="cpu") -> dict:
    """Per-step inputs of decode step ``step``: q, k [B,H,d], v [B,H,dv], gate
    [B,H,f], drawn from their own stream so any step can be regenerated alone."""
    dev = torch.device(device)
    gen = _gen(wl.seed * 1000003 + 7919 * (step + 1), dev)
    dt = wl.torch_dtype
    B, H = wl.B, wl.H
    return {
        "q": _randn((B, H, wl.d), wl.x_std, 0.0, gen, dev, dt),
        "k": _randn((B, H, wl.d), wl.x_std, 0.0, gen, dev, dt),
        "v": _randn((B, H, wl.dv), wl.x_std, 0.0, gen, dev, dt),
        "gate": _randn((B, H, wl.f), wl.gate_std, wl.gate_mean, gen, dev, dt),
    }


def _delta_draws(wl: Workload, shape_tok, gen, dev, decay_mean=None):
    dt = wl.torch_dtype
    out = {
        "q": _randn(shape_tok + (wl.d,), wl.x_std, 0.0, gen, dev, dt),
        "k": _randn(shape_tok + (wl.d,), wl.x_std, 0.0, gen, dev, dt),
        "v": _randn(shape_tok + (wl.dv,), wl.x_std, 0.0, gen, dev, dt),
    }
    mean = wl.gate_mean if decay_mean is None else decay_mean
    # log-decays and write strengths as a Gated DeltaNet layer forms them from
    # its projections: log sigmoid and sigmoid of normal logits
    la = torch.randn(shape_tok, generator=gen, device=dev) * wl.gate_std + mean
    out["log_alpha"] = torch.nn.functional.logsigmoid(la).to(dt)
    bl = torch.randn(shape_tok, generator=gen, device=dev)
    out["beta"] = torch.sigmoid(bl).to(dt)
    return out


def make_delta(wl: Workload, device="cpu", decay_mean=None) -> dict:
    """Inputs of one gated delta rule prefill: q, k [B,H,L,d], v [B,H,L,dv],
    log_alpha and beta [B,H,L].  Draw order q, k, v, decay logits, write-strength
    logits; decay logits ~ N(gate_mean or decay_mean, gate_std), write-strength
    logits ~ N(0, 1); its own seed stream (seed + 500)."""
    dev = torch.device(device)
    return _delta_draws(wl, (wl.B, wl.H, wl.L), _gen(wl.seed + 500, dev), dev, decay_mean)


def make_delta_token(wl: Workload, step: int, device="cpu") -> dict:
    """Per-step inputs of gated delta rule decode step ``step`` ([B,H,*])."""
    dev = torch.device(device)
    return _delta_draws(wl, (wl.B, wl.H), _gen((wl.seed + 500) * 1000003 + 7919 * (step + 1), dev), dev)


def to_f64(t: torch.Tensor):
    """Exact widening of a (bf16 or fp32) tensor to a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()
