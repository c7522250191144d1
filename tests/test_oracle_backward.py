"""Pins of the backward oracle (oracle/backward.py).

The gradient is checked against central finite differences of the independent
C oracle's forward (``oracle.c``), along random directions in every input, so
a dropped term, a wrong sign or a transposed operand anywhere in the autograd
forward shows up; and against a closed form: with Gamma = 1 and no window part
the layer is causal linear attention o = tril(phiQ phiK^T) V, whose value
gradient is tril(phiQ phiK^T)^T dO (Lizard technical summary, gist.science
2507.09025, Methodology A.1 with the gate at one)."""
import numpy as np
import pytest

import oracle
from oracle import backward as OB
from test_oracle import phi_ref, rand_case


def c_loss(c, parts, window, kind, s_in, dO, dS, scale=None):
    o, S = oracle.layer_fwd(c["q"], c["k"], c["v"], c["g"], c["wq"], c["wk"], c["meta"], window=window,
                            parts=parts, gate_kind=kind, state_in=s_in, return_state=True, scale=scale)
    val = float(np.sum(o * dO))
    if parts & OB.PART_GLA and dS is not None:
        val += float(np.sum(S * dS))
    return val


def gate_for(kind, c, rng):
    B, H, L, f = c["g"].shape
    if kind == OB.GATE_LOGITS:
        return c["g"]
    if kind == OB.GATE_LOG:
        return -np.abs(rng.normal(0.3, 0.3, (B, H, L, f)))
    if kind == OB.GATE_LOG_TOKEN:
        return -np.abs(rng.normal(0.3, 0.3, (B, H, L)))
    return -np.abs(rng.normal(0.3, 0.3, (H,)))


CASES = [
    (OB.PART_BOTH, OB.GATE_LOGITS, True),
    (OB.PART_BOTH, OB.GATE_LOG, False),
    (OB.PART_GLA, OB.GATE_LOG_TOKEN, True),
    (OB.PART_BOTH, OB.GATE_LOG_HEAD, True),
    (OB.PART_SWA, OB.GATE_LOGITS, False),
]


@pytest.mark.parametrize("parts,kind,with_state", CASES)
def test_gradient_matches_finite_differences_of_the_c_oracle(parts, kind, with_state):
    rng = np.random.default_rng(7 + 3 * parts + kind)
    c = rand_case(40 + kind, B=2, H=2, L=9, d=5, f=6, dv=4, M=2)
    c["g"] = gate_for(kind, c, rng)
    window = 3
    s_in = rng.normal(0, 1, (2, 2, 6, 4)) if with_state else None
    dO = rng.normal(0, 1, c["v"].shape)
    dS = rng.normal(0, 1, (2, 2, 6, 4)) if with_state else None
    grads = OB.layer_bwd(c["q"], c["k"], c["v"], c["g"], c["wq"], c["wk"], c["meta"], dO, window=window,
                         gate_kind=kind, parts=parts, state_in=s_in, dstate_out=dS)
    inputs = dict(q=c["q"], k=c["k"], v=c["v"], gate=c["g"], wq=c["wq"], wk=c["wk"], meta=c["meta"],
                  state_in=s_in)
    checked = 0
    for name, x in inputs.items():
        gr = grads[name]
        if x is None or gr is None:
            continue
        assert gr.shape == np.shape(x), name
        for trial in range(2):
            u = rng.normal(0, 1, np.shape(x))
            eps = 1e-5
            cp, cm = dict(c), dict(c)
            key = "g" if name == "gate" else name
            sp, sm = s_in, s_in
            if name == "state_in":
                sp, sm = s_in + eps * u, s_in - eps * u
            else:
                cp[key] = x + eps * u
                cm[key] = x - eps * u
            fd = (c_loss(cp, parts, window, kind, sp, dO, dS) - c_loss(cm, parts, window, kind, sm, dO, dS)) / (2 * eps)
            an = float(np.sum(gr * u))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)
            checked += 1
    assert checked >= 6


def test_unused_inputs_get_no_gradient():
    c = rand_case(3, B=1, H=2, L=5, d=4, f=4, dv=3, M=2)
    dO = np.ones(c["v"].shape)
    g = OB.layer_bwd(c["q"], c["k"], c["v"], c["g"], c["wq"], c["wk"], c["meta"], dO, window=2,
                     parts=OB.PART_SWA)
    assert g["gate"] is None and g["wq"] is None and g["wk"] is None
    g = OB.layer_bwd(c["q"], c["k"], c["v"], c["g"], c["wq"], c["wk"], c["meta"], dO, window=2,
                     parts=OB.PART_GLA)
    assert g["meta"] is None


def test_torch_forward_equals_the_c_oracle():
    c = rand_case(12, B=2, H=3, L=30, d=6, f=8, dv=5, M=3)
    s_in = np.random.default_rng(1).normal(0, 1, (2, 3, 8, 5))
    import torch
    T = {k: torch.as_tensor(v) for k, v in c.items()}
    o, S = OB.forward(T["q"], T["k"], T["v"], T["g"], T["wq"], T["wk"], T["meta"], window=4,
                      state_in=torch.as_tensor(s_in))
    oc, Sc = oracle.layer_fwd(c["q"], c["k"], c["v"], c["g"], c["wq"], c["wk"], c["meta"], window=4,
                              state_in=s_in, return_state=True)
    assert np.max(np.abs(o.numpy() - oc)) <= 1e-12 * max(1.0, np.max(np.abs(oc)))
    assert np.max(np.abs(S.numpy() - Sc)) <= 1e-12 * max(1.0, np.max(np.abs(Sc)))


def test_value_gradient_of_ungated_linear_attention_is_the_closed_form():
    """Gamma = 1 (log-gate 0), window part off: dV = tril(phiQ phiK^T)^T dO."""
    c = rand_case(21, B=1, H=2, L=12, d=5, f=6, dv=4)
    dO = np.random.default_rng(2).normal(0, 1, c["v"].shape)
    g = OB.layer_bwd(c["q"], c["k"], c["v"], np.zeros(c["g"].shape), c["wq"], c["wk"], None, dO,
                     window=1, gate_kind=OB.GATE_LOG, parts=OB.PART_GLA)
    for h in range(2):
        pq = phi_ref(c["q"][0, h], c["wq"][h])
        pk = phi_ref(c["k"][0, h], c["wk"][h])
        A = np.tril(pq @ pk.T)
        assert np.max(np.abs(g["v"][0, h] - A.T @ dO[0, h])) <= 1e-12
