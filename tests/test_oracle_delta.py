"""Pins of the gated delta rule oracle (oracle/delta.py).

The pages describe Gated DeltaNet only in words (an error-correcting write with
gated forgetting: "systematic analysis of hybrid linear attention", findings and
recommendations; "LT2" technical summary, hybrid designs), so the oracle follows
the published recurrence.  None of these pins reuses its code: each checks a
consequence of the definition computed another way --

* orthonormal keys with alpha = 1, beta = 1: the delta write never erases, so
  the mixer is plain causal linear attention, sum_s (k^_s . q^_t) v_s;
* beta = 0: nothing is written, the initial state only decays;
* the same key written twice with beta = 1: the second value replaces the first
  (with the eps of the normalisation in closed form, at a key norm where eps
  matters);
* alpha = 0 (a = -inf): the state restarts from the token's own write;
* explicit transition matrices A_t = alpha_t (I - beta_t k^ k^T), multiplied
  out on tiny inputs;
* v = 0, alpha = 1: every step is a contraction (Frobenius norm never grows);
* state continuation and decode continuation;
* planted mistakes (test_delta_mutations_are_caught) each fail one of the above.
"""
import math
import types

import numpy as np
import pytest

from oracle import delta

EPS_DEF = 1e-6  # the normalisation's eps, restated here (not read from the oracle)


def nrm(x):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS_DEF)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def rand_case(seed, B=2, H=2, L=9, dk=8, dv=5):
    rng = np.random.default_rng(seed)
    return dict(q=rng.normal(size=(B, H, L, dk)), k=rng.normal(size=(B, H, L, dk)),
                v=rng.normal(size=(B, H, L, dv)), a=np.log(rng.uniform(0.3, 1.0, (B, H, L))),
                beta=rng.uniform(0.0, 1.0, (B, H, L)), s0=rng.normal(size=(B, H, dv, dk)))


# --- pins, each taking the oracle module so that planted mistakes can be run ---

def pin_orthonormal_is_linear_attention(m):
    rng = np.random.default_rng(1)
    B, H, L, dk, dv = 1, 2, 6, 8, 3
    k = np.zeros((B, H, L, dk))
    for h in range(H):
        Q, _ = np.linalg.qr(rng.normal(size=(dk, dk)))
        k[0, h] = Q[:L] * rng.uniform(0.5, 2.0, (L, 1))  # orthogonal rows, any norms
    q, v = rng.normal(size=(B, H, L, dk)), rng.normal(size=(B, H, L, dv))
    o = m.gdn_fwd(q, k, v, np.zeros((B, H, L)), np.ones((B, H, L)))
    kh, qh = nrm(k), nrm(q)
    exp = np.einsum("bhts,bhsv->bhtv", np.tril(np.einsum("bhtd,bhsd->bhts", qh, kh)), v)
    return rel(o, exp) < 1e-12


def pin_no_write_only_decays(m):
    c = rand_case(2)
    o, s = m.gdn_fwd(c["q"], c["k"], c["v"], c["a"], np.zeros_like(c["beta"]), state_in=c["s0"],
                     return_state=True)
    cum = np.cumsum(c["a"], axis=-1)
    exp = np.exp(cum)[..., None] * np.einsum("bhvk,bhtk->bhtv", c["s0"], nrm(c["q"]))
    return rel(o, exp) < 1e-12 and rel(s, np.exp(cum[..., -1])[..., None, None] * c["s0"]) < 1e-12


def pin_overwrite(m):
    rng = np.random.default_rng(3)
    dk, dv = 8, 4
    out = []
    for scale in (1.0, 1e-3):  # |k|^2 = scale^2 |u|^2 with |u| = 1: eps matters at 1e-3
        u = rng.normal(size=dk)
        u /= np.linalg.norm(u)
        kv = scale * u
        k = np.stack([kv, kv])[None, None]
        q = np.stack([rng.normal(size=dk), kv])[None, None]
        v = rng.normal(size=(1, 1, 2, dv))
        o = m.gdn_fwd(q, k, v, np.zeros((1, 1, 2)), np.ones((1, 1, 2)))
        n = scale ** 2 / (scale ** 2 + EPS_DEF)  # |k^|^2 = k^ . q^ for q = k
        exp = n * v[0, 0, 1] + n * (1.0 - n) * v[0, 0, 0]
        out.append(rel(o[0, 0, 1], exp) < 1e-12)
    return all(out)


def pin_alpha_zero_restarts(m):
    c = rand_case(4)
    a = c["a"].copy()
    a[:, :, 4] = -np.inf
    o = m.gdn_fwd(c["q"], c["k"], c["v"], a, c["beta"], state_in=c["s0"])
    M4 = c["beta"][:, :, 4, None, None] * np.einsum("bhv,bhk->bhvk", c["v"][:, :, 4], nrm(c["k"][:, :, 4]))
    return rel(o[:, :, 4], np.einsum("bhvk,bhk->bhv", M4, nrm(c["q"][:, :, 4]))) < 1e-12


def pin_transition_products(m):
    c = rand_case(5, B=1, H=2, L=7, dk=5, dv=3)
    o = m.gdn_fwd(c["q"], c["k"], c["v"], c["a"], c["beta"], state_in=c["s0"])
    kh, qh = nrm(c["k"]), nrm(c["q"])
    ok = True
    for h in range(2):
        A = [math.exp(c["a"][0, h, t]) * (np.eye(5) - c["beta"][0, h, t] * np.outer(kh[0, h, t], kh[0, h, t]))
             for t in range(7)]
        for t in range(7):
            P = np.eye(5)
            for r in range(t + 1):
                P = P @ A[r]
            M = c["s0"][0, h] @ P
            for s in range(t + 1):
                Ps = np.eye(5)
                for r in range(s + 1, t + 1):
                    Ps = Ps @ A[r]
                M = M + c["beta"][0, h, s] * np.outer(c["v"][0, h, s], kh[0, h, s]) @ Ps
            ok = ok and rel(o[0, h, t], M @ qh[0, h, t]) < 1e-11
    return ok


def pin_contraction(m):
    c = rand_case(6, L=12)
    norms = [np.linalg.norm(c["s0"], axis=(-2, -1))]
    s = c["s0"]
    for t in range(12):
        _, s = m.gdn_decode_step(c["q"][:, :, t], c["k"][:, :, t], np.zeros_like(c["v"][:, :, t]),
                                 np.zeros_like(c["a"][:, :, t]), c["beta"][:, :, t], s)
        norms.append(np.linalg.norm(s, axis=(-2, -1)))
    return all(np.all(norms[i + 1] <= norms[i] * (1 + 1e-14)) for i in range(12))


def pin_continuation(m):
    c = rand_case(7, L=11)
    o, s = m.gdn_fwd(c["q"], c["k"], c["v"], c["a"], c["beta"], state_in=c["s0"], return_state=True)
    o1, s1 = m.gdn_fwd(c["q"][:, :, :5], c["k"][:, :, :5], c["v"][:, :, :5], c["a"][:, :, :5],
                       c["beta"][:, :, :5], state_in=c["s0"], return_state=True)
    o2, s2 = m.gdn_fwd(c["q"][:, :, 5:10], c["k"][:, :, 5:10], c["v"][:, :, 5:10], c["a"][:, :, 5:10],
                       c["beta"][:, :, 5:10], state_in=s1, return_state=True)
    od, sd = m.gdn_decode_step(c["q"][:, :, 10], c["k"][:, :, 10], c["v"][:, :, 10], c["a"][:, :, 10],
                               c["beta"][:, :, 10], s2)
    return (rel(np.concatenate([o1, o2, od[:, :, None]], axis=2), o) < 1e-12 and rel(sd, s) < 1e-12)


PINS = [pin_orthonormal_is_linear_attention, pin_no_write_only_decays, pin_overwrite,
        pin_alpha_zero_restarts, pin_transition_products, pin_contraction, pin_continuation]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_delta_pin(pin):
    assert pin(delta)


MUTATIONS = [
    ("keys not normalised", "kh = l2_normalise(k)", "kh = np.asarray(k, dtype=np.float64)"),
    ("queries not normalised", "qh = l2_normalise(q)", "qh = np.asarray(q, dtype=np.float64)"),
    ("wrong eps", "EPS = 1e-6", "EPS = 1e-4"),
    ("eps outside the root", "np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)",
     "(np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + EPS)"),
    ("decay applied to the write", "M = alpha * erased + b * np.einsum(\"bhv,bhk->bhvk\", v, kh)",
     "M = alpha * (erased + b * np.einsum(\"bhv,bhk->bhvk\", v, kh))"),
    ("erase without beta", "erased = M - b * np.einsum", "erased = M - np.einsum"),
    ("write without beta", "+ b * np.einsum(\"bhv,bhk->bhvk\", v, kh)", "+ np.einsum(\"bhv,bhk->bhvk\", v, kh)"),
    ("readout before the write", "o = np.einsum(\"bhvk,bhk->bhv\", M, qh)",
     "o = np.einsum(\"bhvk,bhk->bhv\", erased, qh)"),
    ("readout with the key", "o = np.einsum(\"bhvk,bhk->bhv\", M, qh)", "o = np.einsum(\"bhvk,bhk->bhv\", M, kh)"),
    ("decay sign", "alpha = np.exp(a)[..., None, None]", "alpha = np.exp(-a)[..., None, None]"),
    ("recall with the query", "recall = np.einsum(\"bhvk,bhk->bhv\", M, kh)",
     "recall = np.einsum(\"bhvk,bhk->bhv\", M, qh)"),
    ("decay before the erase only", "M = alpha * erased + b", "M = erased + b"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_delta_mutations_are_caught(name, old, new):
    src = open(delta.__file__).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType("delta_mutant")
    exec(compile(src.replace(old, new), "delta_mutant", "exec"), mod.__dict__)
    caught = []
    for pin in PINS:
        with np.errstate(all="ignore"):
            try:
                caught.append(not pin(mod))
            except Exception:
                caught.append(True)
    assert any(caught), "planted mistake not caught: " + name
