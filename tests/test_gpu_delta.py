"""GPU parity of the gated delta rule (gdn_prefill, gdn_decode_step) against the
fp64 oracle (oracle/delta.py) on the same seeded inputs, through the C ABI.

Tolerances: max row-normwise relative error <= 1e-4 for fp32 I/O, <= 2e-2 for
bf16 I/O (fp32 state and arithmetic in both)."""
import sys

import numpy as np
import pytest
import torch

from oracle import delta as D
from gated_linear_attention_hybrid_amd import binding as G
from gated_linear_attention_hybrid_amd.inputs import WORKLOADS, make_delta, make_delta_token, to_f64
from parity import TOL_BF16, TOL_F32, assert_finite, gpu_f64, row_rel_err, seeded_randn

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def say(msg):
    print("[gdn]", msg, flush=True)
    sys.stdout.flush()


def oracle_fwd(x, state_in=None, heads=None):
    f = {k: to_f64(v) for k, v in x.items()}
    if heads is not None:
        f = {k: np.stack([f[k][b, h] for b, h in heads])[None] for k in f}
        if state_in is not None:
            state_in = np.stack([state_in[b, h] for b, h in heads])[None]
    return D.gdn_fwd(f["q"], f["k"], f["v"], f["log_alpha"], f["beta"], state_in=state_in, return_state=True)


def run(x, **kw):
    return G.gdn_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], **kw)


@pytest.mark.parametrize("with_state", [False, True])
def test_tiny_fp32(with_state):
    wl = WORKLOADS["tiny_fp32"]
    say("tiny fp32 B=1 H=2 L=256 d=64 state_in=%s" % with_state)
    x = make_delta(wl, DEV)
    s_in = None
    if with_state:
        g = torch.Generator(device="cpu").manual_seed(77)
        s_in = (torch.randn((wl.B, wl.H, wl.dv, wl.d), generator=g) * 0.3).to(DEV)
    s_out = torch.empty((wl.B, wl.H, wl.dv, wl.d), device=DEV)
    o = run(x, state_in=s_in, state_out=s_out)
    ref, ref_s = oracle_fwd(x, None if s_in is None else to_f64(s_in))
    assert row_rel_err(gpu_f64(o), ref) <= TOL_F32
    assert row_rel_err(gpu_f64(s_out), ref_s) <= TOL_F32


@pytest.mark.parametrize("decay_mean", [None, 6.0])
def test_prefill_2k_bf16(decay_mean):
    wl = WORKLOADS["prefill_2k"]
    say("bf16 B=1 H=32 L=2048 d=128 decay logits mean %s" % decay_mean)
    x = make_delta(wl, DEV, decay_mean=decay_mean)
    s_out = torch.empty((wl.B, wl.H, wl.dv, wl.d), device=DEV)
    o = run(x, state_out=s_out)
    assert_finite(o, "o")
    ref, ref_s = oracle_fwd(x)
    assert row_rel_err(gpu_f64(o), ref) <= TOL_BF16
    assert row_rel_err(gpu_f64(s_out), ref_s) <= TOL_BF16


def test_prefill_32k_sampled_heads():
    wl = WORKLOADS["prefill_32k"]
    say("bf16 B=1 H=32 L=32768 d=128, oracle on 2 sampled heads")
    x = make_delta(wl, DEV)
    o = run(x)
    assert_finite(o, "o")
    heads = [(0, 5), (0, 30)]
    ref, _ = oracle_fwd(x, heads=heads)
    got = gpu_f64(o)
    assert row_rel_err(np.stack([got[b, h] for b, h in heads])[None], ref) <= TOL_BF16


@pytest.mark.parametrize("d,dv,L,dtype", [(32, 40, 17, "bf16"), (64, 5, 1, "f32"), (128, 24, 9, "bf16"),
                                          (32, 16, 100, "f32")])
def test_ragged_shapes(d, dv, L, dtype):
    wl = WORKLOADS["tiny_fp32"].with_(B=2, H=3, L=L, d=d, dv=dv, dtype=dtype)
    say("ragged d=%d dv=%d L=%d %s" % (d, dv, L, dtype))
    x = make_delta(wl, DEV)
    s_out = torch.empty((wl.B, wl.H, dv, d), device=DEV)
    o = run(x, state_out=s_out)
    ref, ref_s = oracle_fwd(x)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert row_rel_err(gpu_f64(o), ref) <= tol
    assert row_rel_err(gpu_f64(s_out), ref_s) <= tol


def test_extreme_decay_and_strength():
    wl = WORKLOADS["tiny_fp32"].with_(L=64)
    say("alpha = 0 (log-decay -inf), alpha = 1, beta = 0 and 1")
    x = make_delta(wl, DEV)
    x["log_alpha"][:, :, 10] = -float("inf")
    x["log_alpha"][:, :, 20:30] = 0.0
    x["beta"][:, :, 30:35] = 0.0
    x["beta"][:, :, 40:50] = 1.0
    o = run(x)
    assert_finite(o, "o")
    ref, _ = oracle_fwd(x)
    assert row_rel_err(gpu_f64(o), ref) <= TOL_F32


def test_empty_sequence_passes_state_through():
    wl = WORKLOADS["tiny_fp32"].with_(L=0)
    x = make_delta(wl, DEV)
    s_in = seeded_randn((wl.B, wl.H, wl.dv, wl.d), 42, DEV)
    s_out = torch.full_like(s_in, 7.0)
    run(x, state_in=s_in, state_out=s_out)
    torch.cuda.synchronize()
    assert torch.equal(s_out, s_in)
    run(x, state_out=s_out)
    torch.cuda.synchronize()
    assert not bool(s_out.any())


def test_continuation_and_determinism():
    wl = WORKLOADS["prefill_2k"].with_(H=4, L=300)
    say("split 300 = 128 + 172 through state_in, bitwise repeatability")
    x = make_delta(wl, DEV)
    s_full = torch.empty((wl.B, wl.H, wl.dv, wl.d), device=DEV)
    o = run(x, state_out=s_full)
    o2 = run(x)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    a = {k: v[:, :, :128].contiguous() for k, v in x.items()}
    b = {k: v[:, :, 128:].contiguous() for k, v in x.items()}
    s_mid = torch.empty_like(s_full)
    oa = run(a, state_out=s_mid)
    s_end = torch.empty_like(s_full)
    ob = run(b, state_in=s_mid, state_out=s_end)
    torch.cuda.synchronize()
    # the same per-row operations in the same order: identical bits
    assert torch.equal(torch.cat([oa, ob], dim=2), o)
    assert torch.equal(s_end, s_full)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_decode_continues_prefill(dtype, d):
    wl = WORKLOADS["decode_b8"].with_(L=96, d=d, dv=d, dtype=dtype)
    say("decode B=8 H=32 d=%d %s: 3 steps after a 96-token prefill" % (d, dtype))
    x = make_delta(wl, DEV)
    st = torch.empty((wl.B, wl.H, wl.dv, wl.d), device=DEV)
    run(x, state_out=st)
    _, ref_s = oracle_fwd(x)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    for step in range(3):
        t = make_delta_token(wl, step, DEV)
        o = G.gdn_decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], st)
        f = {k: to_f64(v) for k, v in t.items()}
        ref_o, ref_s = D.gdn_decode_step(f["q"], f["k"], f["v"], f["log_alpha"], f["beta"], ref_s)
        assert row_rel_err(gpu_f64(o), ref_o) <= tol
    assert row_rel_err(gpu_f64(st), ref_s) <= tol


def test_decode_equals_prefill_token():
    """A decode step from state S gives what a one-token prefill from S gives."""
    wl = WORKLOADS["decode_b8"].with_(L=1, B=2, H=8)
    x = make_delta(wl, DEV)
    gen = torch.Generator(device="cpu").manual_seed(31)
    s0 = (torch.randn((wl.B, wl.H, wl.dv, wl.d), generator=gen) * 0.1).to(DEV)
    s_pre = torch.empty_like(s0)
    o_pre = run(x, state_in=s0, state_out=s_pre)
    s_dec = s0.clone()
    o_dec = G.gdn_decode_step(x["q"][:, :, 0].contiguous(), x["k"][:, :, 0].contiguous(),
                              x["v"][:, :, 0].contiguous(), x["log_alpha"][:, :, 0].contiguous(),
                              x["beta"][:, :, 0].contiguous(), s_dec)
    torch.cuda.synchronize()
    # the two kernels reduce the dot products in different orders, so their fp32
    # results differ by a few fp32 ulps and the bf16 output may round one bf16
    # ulp (at most 2^-7 relative) apart; the fp32 states agree to 1e-5
    assert torch.allclose(o_pre[:, :, 0].float(), o_dec.float(), rtol=2.0 ** -7, atol=1e-6)
    assert torch.allclose(s_pre, s_dec, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("d,dv,dtype", [(32, 40, "bf16"), (64, 5, "f32"), (128, 48, "bf16")])
def test_decode_ragged_value_rows(d, dv, dtype):
    """Value-row counts that fill no whole block of the decode step."""
    wl = WORKLOADS["decode_b8"].with_(B=3, H=5, L=20, d=d, dv=dv, dtype=dtype)
    say("decode ragged d=%d dv=%d %s" % (d, dv, dtype))
    x = make_delta(wl, DEV)
    st = torch.empty((wl.B, wl.H, dv, d), device=DEV)
    run(x, state_out=st)
    _, ref_s = oracle_fwd(x)
    t = make_delta_token(wl, 0, DEV)
    o = G.gdn_decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], st)
    f = {k: to_f64(v) for k, v in t.items()}
    ref_o, ref_s = D.gdn_decode_step(f["q"], f["k"], f["v"], f["log_alpha"], f["beta"], ref_s)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert row_rel_err(gpu_f64(o), ref_o) <= tol
    assert row_rel_err(gpu_f64(st), ref_s) <= tol
