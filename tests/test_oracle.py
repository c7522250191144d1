"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a closed form,
an independent brute-force expansion, a library routine in a special case, or an
invariant of the layer.  The layer is Lizard's hybrid attention ("Lizard"
technical summary, gist.science 2507.09025, Methodology A.1 gated linear
attention, A.2 window attention with meta-memory sinks, C Hedgehog feature map).
The pages print no worked numeric example, so no page values are pinned.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import PART_BOTH, PART_GLA, PART_SWA

RTOL = 1e-12


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def rand_case(seed, B=1, H=2, L=20, d=8, f=12, dv=6, M=3, gate_mean=1.0, x_std=1.0):
    rng = np.random.default_rng(seed)
    return dict(
        q=rng.normal(0, x_std, (B, H, L, d)), k=rng.normal(0, x_std, (B, H, L, d)),
        v=rng.normal(0, 1, (B, H, L, dv)), g=rng.normal(gate_mean, 1.0, (B, H, L, f)),
        wq=rng.normal(0, 1 / math.sqrt(d), (H, d, f // 2)),
        wk=rng.normal(0, 1 / math.sqrt(d), (H, d, f // 2)),
        meta=rng.normal(0, 1, (H, M)),
    )


def phi_ref(x, W):
    """Hedgehog map via torch.softmax (library routine): [softmax(xW), softmax(-xW)]."""
    u = torch.from_numpy(x) @ torch.from_numpy(W)
    return torch.cat([torch.softmax(u, -1), torch.softmax(-u, -1)], -1).numpy()


def run(c, window, parts, gate_is_log=False, g=None, scale=None, meta="default", **kw):
    return oracle.layer_fwd(c["q"], c["k"], c["v"], c["g"] if g is None else g, c["wq"], c["wk"],
                            c["meta"] if isinstance(meta, str) else meta, window=window,
                            scale=scale, gate_is_log=gate_is_log, parts=parts, **kw)


# ---------------------------------------------------------------- gated linear part

def test_gla_matches_bruteforce_products():
    """Recurrence == explicit quadratic form with products of gates (no logs):
    o_t = sum_{s<=t} (sum_c phiq_tc phik_sc prod_{r=s+1..t} sigma(g_rc)) v_s."""
    c = rand_case(1, B=2, H=2, L=14, d=6, f=10, dv=5, gate_mean=0.5)
    o = run(c, window=4, parts=PART_GLA)
    B, H, L = c["q"].shape[:3]
    exp = np.zeros_like(o)
    for b in range(B):
        for h in range(H):
            pq = phi_ref(c["q"][b, h], c["wq"][h])
            pk = phi_ref(c["k"][b, h], c["wk"][h])
            gam = torch.sigmoid(torch.from_numpy(c["g"][b, h])).numpy()
            for t in range(L):
                for s in range(t + 1):
                    dec = np.ones(gam.shape[1])
                    for r in range(s + 1, t + 1):
                        dec = dec * gam[r]
                    w = float(np.sum(pq[t] * pk[s] * dec))
                    exp[b, h, t] += w * c["v"][b, h, s]
    assert rel(o, exp) < RTOL


def test_gate_one_is_ungated_causal_linear_attention():
    """log-gate 0 (Gamma = 1): o = (phiQ phiK^T * tril) V."""
    c = rand_case(2, L=24)
    o = run(c, window=3, parts=PART_GLA, gate_is_log=True, g=np.zeros_like(c["g"]))
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            pq = phi_ref(c["q"][b, h], c["wq"][h])
            pk = phi_ref(c["k"][b, h], c["wk"][h])
            exp = np.tril(pq @ pk.T) @ c["v"][b, h]
            assert rel(o[b, h], exp) < RTOL


def test_gate_zero_is_single_token_outer_product():
    """log-gate -inf (Gamma = 0): o_t = (phiq_t . phik_t) v_t."""
    c = rand_case(3, L=16)
    o = run(c, window=5, parts=PART_GLA, gate_is_log=True, g=np.full_like(c["g"], -np.inf))
    assert np.all(np.isfinite(o))
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            pq = phi_ref(c["q"][b, h], c["wq"][h])
            pk = phi_ref(c["k"][b, h], c["wk"][h])
            exp = np.sum(pq * pk, -1, keepdims=True) * c["v"][b, h]
            assert rel(o[b, h], exp) < RTOL


def test_constant_gate_closed_form():
    """Constant gate gamma: o_t = sum_{s<=t} gamma^(t-s) (phiq_t . phik_s) v_s."""
    c = rand_case(4, L=30)
    gamma = 0.8
    o = run(c, window=2, parts=PART_GLA, gate_is_log=True, g=np.full_like(c["g"], math.log(gamma)))
    L = c["q"].shape[2]
    t = np.arange(L)
    D = np.where(t[:, None] >= t[None, :], gamma ** (t[:, None] - t[None, :]).clip(min=0), 0.0)
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            pq = phi_ref(c["q"][b, h], c["wq"][h])
            pk = phi_ref(c["k"][b, h], c["wk"][h])
            assert rel(o[b, h], ((pq @ pk.T) * D) @ c["v"][b, h]) < RTOL


def test_logits_and_log_gate_modes_agree():
    """sigmoid of logits == exp of torch.nn.functional.logsigmoid(logits)."""
    c = rand_case(5, L=18, gate_mean=-1.0)
    a = F.logsigmoid(torch.from_numpy(c["g"])).numpy()
    o1 = run(c, window=4, parts=PART_BOTH)
    o2 = run(c, window=4, parts=PART_BOTH, gate_is_log=True, g=a)
    assert rel(o1, o2) < 1e-13


def test_extreme_gate_logits_reach_the_limits():
    """Logits +-30 are finite and sit within ~1e-12 of the gate=1 / gate=0 forms."""
    c = rand_case(6, L=12)
    hi = run(c, window=3, parts=PART_GLA, g=np.full_like(c["g"], 30.0))
    one = run(c, window=3, parts=PART_GLA, gate_is_log=True, g=np.zeros_like(c["g"]))
    lo = run(c, window=3, parts=PART_GLA, g=np.full_like(c["g"], -30.0))
    zero = run(c, window=3, parts=PART_GLA, gate_is_log=True, g=np.full_like(c["g"], -np.inf))
    assert np.all(np.isfinite(hi)) and np.all(np.isfinite(lo))
    assert rel(hi, one) < 1e-11 and rel(lo, zero) < 1e-11


def test_hedgehog_normalisation_with_zero_query():
    """q = 0 gives phi(q) = 2/f uniform; each half of phi(k) sums to 1, so with a
    single token o_0 = (2/f) * 2 * v_0 whatever k is."""
    c = rand_case(7, L=1, f=16)
    c["q"][:] = 0.0
    o = run(c, window=1, parts=PART_GLA)
    f = c["g"].shape[-1]
    assert rel(o[..., 0, :], (4.0 / f) * c["v"][..., 0, :]) < RTOL


def test_hedgehog_halves_are_distinct_softmaxes():
    """With one token and a one-hot value, the output is phiq . phik: check it
    against the library softmax of +u and -u (catches a sign or half mix-up)."""
    c = rand_case(8, L=1, d=5, f=8, dv=1)
    c["v"][:] = 1.0
    o = run(c, window=1, parts=PART_GLA)
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            pq = phi_ref(c["q"][b, h], c["wq"][h])[0]
            pk = phi_ref(c["k"][b, h], c["wk"][h])[0]
            assert abs(o[b, h, 0, 0] - np.dot(pq, pk)) < 1e-14
            # the map is not symmetric in its halves: swapping them changes the value
            sw = np.concatenate([pk[4:], pk[:4]])
            assert abs(np.dot(pq, sw) - np.dot(pq, pk)) > 1e-6


def test_state_continuation():
    """prefill(0:L1) -> state -> prefill(L1:L, state_in) == prefill(0:L) (gated part)."""
    c = rand_case(9, L=26)
    full, sfull = run(c, window=4, parts=PART_GLA, return_state=True)
    L1 = 11
    first = {k: (v[:, :, :L1] if v.ndim == 4 else v) for k, v in c.items()}
    rest = {k: (v[:, :, L1:] if v.ndim == 4 else v) for k, v in c.items()}
    o1, s1 = run(first, window=4, parts=PART_GLA, return_state=True)
    o2, s2 = run(rest, window=4, parts=PART_GLA, state_in=s1, return_state=True)
    assert rel(np.concatenate([o1, o2], 2), full) < RTOL
    assert rel(s2, sfull) < RTOL


# ---------------------------------------------------------------- window part

def sdpa_with_sinks(q, k, v, meta, window, scale):
    """torch scaled_dot_product_attention (fp64, CPU): the sinks are extra keys
    with zero key and value vectors whose additive mask entry is t_m."""
    L, d = q.shape
    M = 0 if meta is None else len(meta)
    kk = torch.cat([torch.from_numpy(k), torch.zeros(M, d, dtype=torch.float64)])
    vv = torch.cat([torch.from_numpy(v), torch.zeros(M, v.shape[1], dtype=torch.float64)])
    mask = torch.full((L, L + M), float("-inf"), dtype=torch.float64)
    for t in range(L):
        mask[t, max(0, t - window + 1):t + 1] = 0.0
        if M:
            mask[t, L:] = torch.from_numpy(meta)
    out = F.scaled_dot_product_attention(torch.from_numpy(q)[None], kk[None], vv[None],
                                         attn_mask=mask[None], scale=scale)
    return out[0].numpy()


@pytest.mark.parametrize("window", [1, 3, 7, 64])
def test_window_matches_sdpa_with_sinks(window):
    c = rand_case(10, L=21, x_std=1.5)
    o = run(c, window=window, parts=PART_SWA, scale=0.7)
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            exp = sdpa_with_sinks(c["q"][b, h], c["k"][b, h], c["v"][b, h], c["meta"][h], window, 0.7)
            assert rel(o[b, h], exp) < 1e-12


def test_window_without_sinks_is_causal_softmax():
    """No sinks and window >= L: textbook causal softmax attention (is_causal)."""
    c = rand_case(11, L=17, x_std=1.5)
    o = oracle.layer_fwd(c["q"], c["k"], c["v"], None, None, None, None, window=100,
                         parts=PART_SWA)
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            exp = F.scaled_dot_product_attention(torch.from_numpy(c["q"][b, h])[None],
                                                 torch.from_numpy(c["k"][b, h])[None],
                                                 torch.from_numpy(c["v"][b, h])[None],
                                                 is_causal=True)[0].numpy()
            assert rel(o[b, h], exp) < 1e-12


def test_window_one_closed_form():
    """w = 1: o_t = e^{s_tt} v_t / (e^{s_tt} + sum_m e^{t_m})."""
    c = rand_case(12, L=9)
    scale = 0.3
    o = run(c, window=1, parts=PART_SWA, scale=scale)
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            s = scale * np.sum(c["q"][b, h] * c["k"][b, h], -1, keepdims=True)
            den = np.exp(s) + np.sum(np.exp(c["meta"][h]))
            assert rel(o[b, h], np.exp(s) * c["v"][b, h] / den) < RTOL


def test_default_scale_is_inverse_sqrt_d():
    c = rand_case(13, L=10, d=9)
    assert rel(run(c, window=4, parts=PART_SWA), run(c, window=4, parts=PART_SWA, scale=1 / 3.0)) < 1e-15


# ---------------------------------------------------------------- the hybrid

def test_single_token_is_sum_of_closed_forms():
    """L = 1: o_0 = (phiq_0 . phik_0) v_0 + e^{s} v_0 / (e^{s} + sum e^{t_m})."""
    c = rand_case(14, L=1)
    o = run(c, window=8, parts=PART_BOTH, scale=0.5)
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            pq = phi_ref(c["q"][b, h], c["wq"][h])[0]
            pk = phi_ref(c["k"][b, h], c["wk"][h])[0]
            s = 0.5 * np.dot(c["q"][b, h, 0], c["k"][b, h, 0])
            sw = np.exp(s) / (np.exp(s) + np.sum(np.exp(c["meta"][h])))
            assert rel(o[b, h, 0], (np.dot(pq, pk) + sw) * c["v"][b, h, 0]) < RTOL


def test_hybrid_is_sum_of_parts():
    c = rand_case(15, L=19)
    both = run(c, window=5, parts=PART_BOTH)
    assert rel(both, run(c, window=5, parts=PART_GLA) + run(c, window=5, parts=PART_SWA)) < 1e-14


def test_linear_in_values():
    c = rand_case(16, L=15)
    c2 = dict(c, v=np.random.default_rng(99).normal(size=c["v"].shape))
    mix = dict(c, v=2.0 * c["v"] - 0.5 * c2["v"])
    o = run(mix, window=4, parts=PART_BOTH)
    assert rel(o, 2.0 * run(c, window=4, parts=PART_BOTH) - 0.5 * run(c2, window=4, parts=PART_BOTH)) < 1e-13


def test_heads_and_batches_are_independent():
    c = rand_case(17, B=2, H=3, L=12)
    o = run(c, window=4, parts=PART_BOTH)
    for b in range(2):
        for h in range(3):
            one = {k: (v[b:b + 1, h:h + 1] if v.ndim == 4 else v[h:h + 1]) for k, v in c.items()}
            assert rel(run(one, window=4, parts=PART_BOTH)[0, 0], o[b, h]) < 1e-15


# ---------------------------------------------------------------- decode

@pytest.mark.parametrize("window,L0", [(4, 9), (6, 3), (1, 5)])
def test_decode_steps_continue_the_prefill(window, L0):
    """prefill(0:L0) then decode steps L0..L-1 (ring from the last w tokens) ==
    prefill(0:L), outputs and final state."""
    c = rand_case(18, B=2, H=2, L=L0 + 7)
    full, sfull = run(c, window=window, parts=PART_BOTH, return_state=True)
    first = {k: (v[:, :, :L0] if v.ndim == 4 else v) for k, v in c.items()}
    _, st = run(first, window=window, parts=PART_BOTH, return_state=True)
    B, H, L, d = c["q"].shape
    dv = c["v"].shape[-1]
    kc = np.zeros((B, H, window, d))
    vc = np.zeros((B, H, window, dv))
    for p in range(max(0, L0 - window), L0):
        kc[:, :, p % window] = c["k"][:, :, p]
        vc[:, :, p % window] = c["v"][:, :, p]
    st = np.ascontiguousarray(st)
    for t in range(L0, L):
        o = oracle.decode_step(c["q"][:, :, t], c["k"][:, :, t], c["v"][:, :, t], c["g"][:, :, t],
                               c["wq"], c["wk"], c["meta"], st, kc, vc, np.full(B, t),
                               window=window)
        assert rel(o, full[:, :, t]) < RTOL
    assert rel(st, sfull) < RTOL


def test_decode_from_empty_ring():
    """pos = 0 with an empty (garbage) ring: only the new token is attended."""
    c = rand_case(19, B=1, H=2, L=1)
    o_ref = run(c, window=4, parts=PART_BOTH)
    B, H, _, d = c["q"].shape
    st = np.zeros((B, H, c["g"].shape[-1], c["v"].shape[-1]))
    kc = np.full((B, H, 4, d), 1e3)
    vc = np.full((B, H, 4, c["v"].shape[-1]), -7.0)
    o = oracle.decode_step(c["q"][:, :, 0], c["k"][:, :, 0], c["v"][:, :, 0], c["g"][:, :, 0],
                           c["wq"], c["wk"], c["meta"], st, kc, vc, np.zeros(B), window=4)
    assert rel(o, o_ref[:, :, 0]) < RTOL


def test_golden_regression_fixture():
    """tests/golden/tiny_hybrid.json was written by tests/golden/make_golden.py from
    the oracle; a change of the oracle's arithmetic shows up here."""
    import json
    import os
    import sys
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    sys.path.insert(0, here)
    try:
        import make_golden
    finally:
        sys.path.remove(here)
    c = make_golden.fixed_inputs()
    ref = json.load(open(os.path.join(here, "tiny_hybrid.json")))
    o, st = oracle.layer_fwd(c["q"], c["k"], c["v"], c["g"], c["wq"], c["wk"], c["meta"],
                             window=ref["window"], scale=ref["scale"], return_state=True)
    assert rel(o, np.array(ref["o"])) < 1e-14
    assert rel(st, np.array(ref["state"])) < 1e-14
