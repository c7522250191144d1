"""fp64 CPU oracle of the gated delta rule (Gated DeltaNet token mixer).

TEST INFRASTRUCTURE ONLY: the test suite and the benchmark use this module to
compute expected values.  The GPU library never imports it, and it never
imports the GPU library.

The pages name Gated DeltaNet as the mixer they recommend ("systematic analysis
of hybrid linear attention", 2507.06457, findings on selective gating and
recommendations; "LT2" technical summary, 2605.20670, hybrid designs GDN+DSA and
Full+GDN) and describe its update only in words: an error-correcting (delta)
write into the state with controlled forgetting (gated decay).  They print no
formula, so this oracle takes the published Gated DeltaNet recurrence, per batch
row and head, with the state M (d_v x d_k) kept as value rows:

    k^ = k_t / sqrt(|k_t|^2 + eps),  q^ = q_t / sqrt(|q_t|^2 + eps),  eps = 1e-6
    M_t = alpha_t M_{t-1} (I - beta_t k^ k^T) + beta_t v_t k^T
    o_t = M_t q^

with alpha_t = exp(a_t) (a_t <= 0 the log-decay of token t, -inf allowed) and
beta_t in [0, 1] the write strength.  The delta reading: M_{t-1} k^ is what the
state currently returns for key k^; the write replaces beta_t of it with v_t.
Readings where the pages are silent: keys and queries are L2-normalised inside
the mixer with eps added to the squared norm, the readout carries no further
scale, a and beta are given per token and head (the caller applies its own
sigmoid or softplus), M_0 = 0 unless an initial state is given.

Everything is plain float64 numpy, one token at a time, vectorised over
(batch, head) only.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def l2_normalise(x):
    """x / sqrt(sum(x^2) + EPS) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)


def _step(M, q, k, v, a, beta):
    """One token for every (b, h): M [B,H,dv,dk], q/k [B,H,dk], v [B,H,dv],
    a/beta [B,H].  Returns (o [B,H,dv], new M)."""
    kh = l2_normalise(k)
    qh = l2_normalise(q)
    alpha = np.exp(a)[..., None, None]
    b = beta[..., None, None]
    # M (I - beta k^ k^T): remove beta of what the state returns for k^ ...
    recall = np.einsum("bhvk,bhk->bhv", M, kh)
    erased = M - b * np.einsum("bhv,bhk->bhvk", recall, kh)
    # ... decay, then write beta v k^T
    M = alpha * erased + b * np.einsum("bhv,bhk->bhvk", v, kh)
    o = np.einsum("bhvk,bhk->bhv", M, qh)
    return o, M


def gdn_fwd(q, k, v, a, beta, *, state_in=None, return_state=False):
    """Gated delta rule over whole sequences.

    q, k: [B,H,L,dk]; v: [B,H,L,dv]; a (log-decay <= 0), beta: [B,H,L];
    state_in: [B,H,dv,dk] or None (zeros).  Returns o [B,H,L,dv] (and the final
    state [B,H,dv,dk] when return_state)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    M = np.zeros((B, H, dv, dk)) if state_in is None else np.array(state_in, dtype=np.float64)
    o = np.zeros((B, H, L, dv))
    for t in range(L):
        o[:, :, t], M = _step(M, q[:, :, t], k[:, :, t], v[:, :, t], a[:, :, t], beta[:, :, t])
    return (o, M) if return_state else o


def gdn_decode_step(q, k, v, a, beta, state):
    """One generated token: q, k [B,H,dk], v [B,H,dv], a, beta [B,H], state
    [B,H,dv,dk].  Returns (o [B,H,dv], new state)."""
    return _step(np.asarray(state, dtype=np.float64), np.asarray(q, dtype=np.float64),
                 np.asarray(k, dtype=np.float64), np.asarray(v, dtype=np.float64),
                 np.asarray(a, dtype=np.float64), np.asarray(beta, dtype=np.float64))
