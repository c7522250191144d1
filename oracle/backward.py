"""fp64 CPU oracle of the hybrid layer's backward pass.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module to compute expected gradients.  The GPU library
never imports it, and it never imports the GPU library.

What it computes: the exact gradient of the plain token-by-token definition of
the layer (Lizard technical summary, gist.science 2507.09025, Methodology A.1:
gated state S_t = diag(Gamma_t) S_{t-1} + phi(k_t) v_t^T read out with
phi(q_t); A.2: window softmax whose denominator also holds exp of the learned
meta-memory scalars; Methodology C: phi = [softmax(xW), softmax(-xW)]), for a
loss L = <o, dO> + <S_L, dS_L>.  The same summary's two-stage training
(Methodology B) fits exactly these parameters -- gate, feature maps, meta tokens
-- so the gradients with respect to q, k, v, the gate input, both feature-map
weights, the meta scalars and the initial state are all returned.

How: the forward is written as the plain recurrence and the plain masked window
softmax in float64 PyTorch CPU ops (no chunking, no log-space rewrite), and the
derivative is taken by reverse-mode automatic differentiation, a library
primitive applied to that definition.  The tests pin it to central finite
differences of the independent C oracle (``oracle.c``), so neither this forward
nor autograd is trusted on its own.
"""
from __future__ import annotations

import numpy as np
import torch

from .oracle import GATE_LOG, GATE_LOG_HEAD, GATE_LOG_TOKEN, GATE_LOGITS, PART_BOTH, PART_GLA, PART_SWA

NAMES = ("q", "k", "v", "gate", "wq", "wk", "meta", "state_in")


def _t(a):
    if a is None:
        return None
    return torch.as_tensor(np.asarray(a, dtype=np.float64)).clone().requires_grad_(True)


def _gamma_log(g, kind, B, H, L, f):
    """log Gamma [B,H,L,f] for gate layout ``kind`` (Methodology A.1: Gamma =
    sigmoid of the gate logits; the log layouts give log Gamma directly)."""
    if kind == GATE_LOGITS:
        return torch.nn.functional.logsigmoid(g)
    if kind == GATE_LOG:
        return g
    if kind == GATE_LOG_TOKEN:
        return g[..., None].expand(B, H, L, f)
    if kind == GATE_LOG_HEAD:
        return g.reshape(1, H, 1, 1).expand(B, H, L, f)
    raise ValueError("unknown gate kind %r" % (kind,))


def _phi(x, w):
    """Hedgehog map of every token: [softmax(x W_h), softmax(-x W_h)] per head."""
    u = torch.einsum("bhld,hdf->bhlf", x, w)
    return torch.cat([torch.softmax(u, -1), torch.softmax(-u, -1)], -1)


def forward(q, k, v, g, wq, wk, meta, *, window, scale=None, gate_kind=GATE_LOGITS,
            parts=PART_BOTH, state_in=None):
    """The layer's forward in float64 torch ops: returns (o, final state or None)."""
    B, H, L, d = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = torch.zeros((B, H, L, dv), dtype=torch.float64)
    S = None
    if parts & PART_GLA:
        f = 2 * wq.shape[-1]
        pq, pk = _phi(q, wq), _phi(k, wk)
        gam = torch.exp(_gamma_log(g, gate_kind, B, H, L, f))
        S = state_in if state_in is not None else torch.zeros((B, H, f, dv), dtype=torch.float64)
        outs = []
        for t in range(L):
            S = gam[:, :, t, :, None] * S + pk[:, :, t, :, None] * v[:, :, t, None, :]
            outs.append((pq[:, :, t, :, None] * S).sum(-2))
        if L:
            o = o + torch.stack(outs, 2)
    if parts & PART_SWA and L:
        s = scale * torch.einsum("bhtd,bhjd->bhtj", q, k)
        t_idx = torch.arange(L)[:, None]
        j_idx = torch.arange(L)[None, :]
        keep = (j_idx <= t_idx) & (j_idx > t_idx - window)
        s = s.masked_fill(~keep, float("-inf"))
        if meta is not None and meta.shape[-1]:
            sinks = meta.reshape(1, H, 1, -1).expand(B, H, L, meta.shape[-1])
            p = torch.softmax(torch.cat([s, sinks], -1), -1)[..., :L]
        else:
            p = torch.softmax(s, -1)
        o = o + p @ v
    return o, S


def layer_bwd(q, k, v, g, wq, wk, meta, do, *, window, scale=None, gate_kind=GATE_LOGITS,
              parts=PART_BOTH, state_in=None, dstate_out=None):
    """Gradients of <o, do> + <S_final, dstate_out> with respect to every input.

    Shapes as the forward (q, k [B,H,L,d]; v [B,H,L,dv]; gate in its layout;
    wq, wk [H,d,f/2]; meta [H,M] or None; state_in [B,H,f,dv] or None; do
    [B,H,L,dv]; dstate_out [B,H,f,dv] or None).  Returns a dict of float64
    numpy arrays named as the inputs (None for an input that was None or that
    ``parts`` leaves unused)."""
    T = {n: _t(a) for n, a in zip(NAMES, (q, k, v, g, wq, wk, meta, state_in))}
    gla = bool(parts & PART_GLA)
    if not gla:
        for n in ("gate", "wq", "wk", "state_in"):
            T[n] = None
    if not parts & PART_SWA:
        T["meta"] = None
    o, S = forward(T["q"], T["k"], T["v"], T["gate"], T["wq"], T["wk"], T["meta"], window=window,
                   scale=scale, gate_kind=gate_kind, parts=parts, state_in=T["state_in"])
    loss = (o * torch.as_tensor(np.asarray(do, dtype=np.float64))).sum()
    if gla and dstate_out is not None:
        loss = loss + (S * torch.as_tensor(np.asarray(dstate_out, dtype=np.float64))).sum()
    live = [n for n in NAMES if T[n] is not None]
    grads = torch.autograd.grad(loss, [T[n] for n in live], allow_unused=True)
    out = {n: None for n in NAMES}
    for n, gr in zip(live, grads):
        out[n] = np.zeros(T[n].shape) if gr is None else gr.detach().numpy()
    return out


__all__ = ["forward", "layer_bwd", "NAMES", "GATE_LOG", "GATE_LOGITS", "GATE_LOG_TOKEN",
           "GATE_LOG_HEAD", "PART_BOTH", "PART_GLA", "PART_SWA"]
