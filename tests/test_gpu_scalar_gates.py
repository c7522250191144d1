"""GPU parity of the scalar-decay gate layouts against the fp64 oracle: one
log-gate per token (Mamba-2 style) and one fixed log-decay per head (RetNet
style), broadcast over the features by the same kernels ("LT2" technical
summary, 2.1 architecture variants; "systematic analysis of hybrid linear
attention", evaluated models).  Chunkwise MFMA prefill (bf16, d = 128), the
token-recurrent path (fp32), and both decode kernels."""
import numpy as np
import pytest
import torch

import oracle
from gated_linear_attention_hybrid_amd import binding as G
from gated_linear_attention_hybrid_amd.inputs import WORKLOADS, make_decode_token, make_prefill, to_f64
from parity import TOL_BF16, TOL_F32, assert_finite, gpu_f64, row_rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"
KINDS = {"token": (G.GLAH_GATE_LOG_TOKEN, oracle.GATE_LOG_TOKEN),
         "head": (G.GLAH_GATE_LOG_HEAD, oracle.GATE_LOG_HEAD)}


def say(msg):
    print("[case]", msg, flush=True)


def scalar_gates(kind, B, H, L, dtype, seed=11):
    """Seeded log-gates: per token in [log 0.5, 0], or a fixed decay per head."""
    gen = torch.Generator().manual_seed(seed)
    if kind == "token":
        g = torch.log(torch.rand((B, H, L), generator=gen) * 0.5 + 0.5)
    else:
        g = torch.log(torch.rand((H,), generator=gen) * 0.2 + 0.8)
    return g.to(dtype).to(DEV)


def oracle_fwd(x, g, wl, okind, **kw):
    h = {k: to_f64(v) for k, v in x.items() if k != "gate"}
    return oracle.layer_fwd(h["q"], h["k"], h["v"], to_f64(g), h["wq"], h["wk"], h["meta"],
                            window=wl.window, gate_kind=okind, **kw)


@pytest.mark.parametrize("kind", ["token", "head"])
@pytest.mark.parametrize("L", [700, 1000])
def test_chunked_prefill_scalar_gates(kind, L):
    wl = WORKLOADS["prefill_2k"].with_(H=4, L=L)
    say("chunked prefill, %s gates, L=%d" % (kind, L))
    x = make_prefill(wl, DEV)
    g = scalar_gates(kind, wl.B, wl.H, wl.L, torch.bfloat16)
    gk, ok = KINDS[kind]
    st = torch.empty((wl.B, wl.H, wl.f, wl.dv), device=DEV)
    o = G.hybrid_layer_fwd(x["q"], x["k"], x["v"], g, x["wq"], x["wk"], x["meta"], window=wl.window,
                           gate_kind=gk, state_out=st)
    assert_finite(o, "o")
    ref, sref = oracle_fwd(x, g, wl, ok, return_state=True)
    assert row_rel_err(gpu_f64(o), ref) <= TOL_BF16
    assert row_rel_err(gpu_f64(st).reshape(-1, wl.dv), sref.reshape(-1, wl.dv)) <= TOL_BF16
    o2 = G.gla_prefill(x["q"], x["k"], x["v"], g, x["wq"], x["wk"], gate_kind=gk)
    ref2 = oracle_fwd(x, g, wl, ok, parts=oracle.PART_GLA)
    assert row_rel_err(gpu_f64(o2), ref2) <= TOL_BF16


@pytest.mark.parametrize("kind", ["token", "head"])
def test_recurrent_prefill_scalar_gates_fp32(kind):
    wl = WORKLOADS["tiny_fp32"].with_(H=3, B=2, L=77)
    say("fp32 recurrent prefill, %s gates" % kind)
    x = make_prefill(wl, DEV)
    g = scalar_gates(kind, wl.B, wl.H, wl.L, torch.float32)
    gk, ok = KINDS[kind]
    o = G.hybrid_layer_fwd(x["q"], x["k"], x["v"], g, x["wq"], x["wk"], x["meta"], window=wl.window,
                           gate_kind=gk)
    assert row_rel_err(gpu_f64(o), oracle_fwd(x, g, wl, ok)) <= TOL_F32


@pytest.mark.parametrize("kind", ["token", "head"])
@pytest.mark.parametrize("shape", ["d128_bf16", "d128_f32", "d64_f32"])
def test_decode_scalar_gates(kind, shape):
    """Decode steps after a prefill, both sides starting from their own prefix
    (d = 128 runs the per-head decode kernel, d = 64 the general one)."""
    if shape == "d64_f32":
        wl = WORKLOADS["tiny_fp32"].with_(B=2, H=3)
    else:
        wl = WORKLOADS["decode_b8"].with_(B=2, H=4, dtype=shape[-4:].lstrip("_"))
    say("decode, %s gates, %s" % (kind, shape))
    L0, steps = 40, 6
    x = make_prefill(wl.with_(L=L0), DEV)
    gk, ok = KINDS[kind]
    tdt = wl.torch_dtype
    g0 = scalar_gates(kind, wl.B, wl.H, L0, tdt)
    B, H = wl.B, wl.H
    st = torch.empty((B, H, wl.f, wl.dv), device=DEV)
    kc = torch.empty((B, H, wl.window, wl.d), device=DEV, dtype=tdt)
    vc = torch.empty((B, H, wl.window, wl.dv), device=DEV, dtype=tdt)
    G.hybrid_layer_fwd(x["q"], x["k"], x["v"], g0, x["wq"], x["wk"], x["meta"], window=wl.window,
                       gate_kind=gk, state_out=st, kcache_out=kc, vcache_out=vc)
    ox = {k: to_f64(v) for k, v in x.items()}
    _, ost = oracle_fwd(x, g0, wl, ok, return_state=True)
    ost = np.ascontiguousarray(ost)
    okc = np.zeros((B, H, wl.window, wl.d))
    ovc = np.zeros((B, H, wl.window, wl.dv))
    for p in range(max(0, L0 - wl.window), L0):
        okc[:, :, p % wl.window] = ox["k"][:, :, p]
        ovc[:, :, p % wl.window] = ox["v"][:, :, p]
    tol = TOL_BF16 if tdt == torch.bfloat16 else TOL_F32
    for s in range(steps):
        t = make_decode_token(wl, s, DEV)
        gt = scalar_gates(kind, B, H, 1, tdt, seed=100 + s)
        gt = gt[:, :, 0].contiguous() if kind == "token" else gt
        pos = torch.full((B,), L0 + s, dtype=torch.int32, device=DEV)
        o = G.gla_decode_step(t["q"], t["k"], t["v"], gt, x["wq"], x["wk"], x["meta"], st, kc, vc, pos,
                              window=wl.window, gate_kind=gk)
        ot = {k: to_f64(v) for k, v in t.items()}
        oref = oracle.decode_step(ot["q"], ot["k"], ot["v"], to_f64(gt), ox["wq"], ox["wk"], ox["meta"],
                                  ost, okc, ovc, np.full(B, L0 + s), window=wl.window, gate_kind=ok)
        assert row_rel_err(gpu_f64(o), oref) <= tol, s
    assert_finite(st, "state")
    assert row_rel_err(gpu_f64(st).reshape(-1, wl.dv), ost.reshape(-1, wl.dv)) <= tol
