"""Pins of the oracle's scalar-decay gate layouts (a per-token scalar as in
Mamba-2, a fixed per-head decay as in RetNet: "LT2" technical summary, 2.1
architecture variants; "systematic analysis of hybrid linear attention",
evaluated models).  Each is checked against an independent expansion: the
retention form sum_s gamma^(t-s) (phiq_t . phik_s) v_s for a fixed decay, and
explicit products of scalar gates for per-token gates."""
import math

import numpy as np

import oracle
from oracle import GATE_LOG_HEAD, GATE_LOG_TOKEN, PART_GLA
from test_oracle import phi_ref, rand_case, rel, RTOL


def test_fixed_head_decay_is_retention():
    """Fixed log-decay per head: o_t = sum_{s<=t} gamma_h^(t-s) (phiq_t . phik_s) v_s
    + gamma_h^(t+1) phiq_t S_in (the retention form, no recurrence)."""
    c = rand_case(31, B=2, H=3, L=17, d=6, f=8, dv=5)
    lg = np.log(np.array([0.9, 0.5, 0.99]))
    rng = np.random.default_rng(5)
    s_in = rng.normal(0, 1, (2, 3, 8, 5))
    o = oracle.layer_fwd(c["q"], c["k"], c["v"], lg, c["wq"], c["wk"], None, window=2,
                         parts=PART_GLA, gate_kind=GATE_LOG_HEAD, state_in=s_in)
    exp = np.zeros_like(o)
    for b in range(2):
        for h in range(3):
            pq = phi_ref(c["q"][b, h], c["wq"][h])
            pk = phi_ref(c["k"][b, h], c["wk"][h])
            gam = math.exp(lg[h])
            for t in range(17):
                exp[b, h, t] = gam ** (t + 1) * (pq[t] @ s_in[b, h])
                for s in range(t + 1):
                    exp[b, h, t] += gam ** (t - s) * float(pq[t] @ pk[s]) * c["v"][b, h, s]
    assert rel(o, exp) < RTOL


def test_token_scalar_gate_is_scalar_products():
    """Per-token scalar log-gates: o_t = sum_{s<=t} (prod_{r=s+1..t} Gamma_r)
    (phiq_t . phik_s) v_s, one factor shared by all features."""
    c = rand_case(32, B=2, H=2, L=15, d=6, f=10, dv=4)
    rng = np.random.default_rng(6)
    lg = np.log(rng.uniform(0.3, 1.0, (2, 2, 15)))
    o = oracle.layer_fwd(c["q"], c["k"], c["v"], lg, c["wq"], c["wk"], None, window=3,
                         parts=PART_GLA, gate_kind=GATE_LOG_TOKEN)
    exp = np.zeros_like(o)
    for b in range(2):
        for h in range(2):
            pq = phi_ref(c["q"][b, h], c["wq"][h])
            pk = phi_ref(c["k"][b, h], c["wk"][h])
            gam = np.exp(lg[b, h])
            for t in range(15):
                for s in range(t + 1):
                    dec = float(np.prod(gam[s + 1:t + 1]))
                    exp[b, h, t] += dec * float(pq[t] @ pk[s]) * c["v"][b, h, s]
    assert rel(o, exp) < RTOL


def test_scalar_gate_decode_continues_the_prefill():
    """Decode steps with scalar gates continue a scalar-gate prefill (both
    layouts): the state after L0 prefill tokens stepped L1 more times gives the
    prefill's outputs of those tokens."""
    c = rand_case(33, B=1, H=2, L=9, d=6, f=8, dv=4)
    rng = np.random.default_rng(7)
    for kind, lg in ((GATE_LOG_TOKEN, np.log(rng.uniform(0.4, 1.0, (1, 2, 9)))),
                     (GATE_LOG_HEAD, np.log(np.array([0.8, 0.6])))):
        full = oracle.layer_fwd(c["q"], c["k"], c["v"], lg, c["wq"], c["wk"], c["meta"], window=3,
                                gate_kind=kind)
        L0 = 5
        pre = (lambda a: a[:, :, :L0]) if kind == GATE_LOG_TOKEN else (lambda a: a)
        _, st = oracle.layer_fwd(c["q"][:, :, :L0], c["k"][:, :, :L0], c["v"][:, :, :L0], pre(lg),
                                 c["wq"], c["wk"], c["meta"], window=3, gate_kind=kind, return_state=True)
        state = np.ascontiguousarray(st)
        kc = np.zeros((1, 2, 3, 6))
        vc = np.zeros((1, 2, 3, 4))
        for p in range(L0):
            kc[:, :, p % 3] = c["k"][:, :, p]
            vc[:, :, p % 3] = c["v"][:, :, p]
        for t in range(L0, 9):
            gt = lg[:, :, t] if kind == GATE_LOG_TOKEN else lg
            o = oracle.decode_step(c["q"][:, :, t], c["k"][:, :, t], c["v"][:, :, t], gt, c["wq"], c["wk"],
                                   c["meta"], state, kc, vc, np.array([t]), window=3, gate_kind=kind)
            assert rel(o, full[:, :, t]) < 1e-10
