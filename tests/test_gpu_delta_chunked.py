"""GPU parity of the chunkwise gated delta rule prefill (bf16, d_qk = 128, d_v a
multiple of 16, L >= 64: the prep and recurrence kernels of delta_chunk.hip)
against the fp64 oracle (oracle/delta.py), through the C ABI, on shapes and
values that stress the chunk form: ragged lengths with a given initial state,
narrow and wide value tiles, extreme decays and write strengths, a key repeated
over a whole chunk with full write strength (the unit lower-triangular system
at its least well conditioned), zero keys and queries, and the caller's
workspace.

Tolerance: max row-normwise relative error <= 2e-2 (bf16 I/O, fp32 state)."""
import sys

import numpy as np
import pytest
import torch

from oracle import delta as D
from gated_linear_attention_hybrid_amd import binding as G
from gated_linear_attention_hybrid_amd.inputs import WORKLOADS, make_delta, to_f64
from parity import TOL_BF16, assert_finite, gpu_f64, row_rel_err, seeded_randn

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
BASE = WORKLOADS["prefill_2k"]


def say(msg):
    print("[gdn-chunk]", msg, flush=True)
    sys.stdout.flush()


def oracle_fwd(x, state_in=None):
    f = {k: to_f64(v) for k, v in x.items()}
    return D.gdn_fwd(f["q"], f["k"], f["v"], f["log_alpha"], f["beta"], state_in=state_in, return_state=True)


def run(x, **kw):
    return G.gdn_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], **kw)


def check(x, s_in=None, tag=""):
    B, H, L, dv = x["v"].shape
    d = x["q"].shape[-1]
    s_out = torch.empty((B, H, dv, d), device=DEV)
    o = run(x, state_in=s_in, state_out=s_out)
    assert_finite(o, "o")
    ref, ref_s = oracle_fwd(x, None if s_in is None else to_f64(s_in))
    eo, es = row_rel_err(gpu_f64(o), ref), row_rel_err(gpu_f64(s_out), ref_s)
    say("%s: o err %.3e, state err %.3e" % (tag, eo, es))
    assert eo <= TOL_BF16
    assert es <= TOL_BF16
    return o


def test_path_is_chunked():
    # the shapes below take the chunkwise path: it is the one that needs a workspace
    desc = G.make_desc(2, 3, 65, 128, 16, 128, dtype=G.GLAH_BF16)
    assert G.gdn_workspace_bytes(desc) == 2 * 3 * 2 * 13568


@pytest.mark.parametrize("L", [64, 65, 127, 200, 1000])
def test_ragged_lengths_with_state(L):
    wl = BASE.with_(B=2, H=3, L=L)
    say("B=2 H=3 L=%d d=d_v=128, state_in given" % L)
    x = make_delta(wl, DEV)
    s_in = seeded_randn((wl.B, wl.H, wl.dv, wl.d), 1000 + L, DEV) * 0.3
    check(x, s_in, "L=%d" % L)


@pytest.mark.parametrize("dv", [16, 48, 80, 256])
def test_value_tiles(dv):
    wl = BASE.with_(B=1, H=2, L=200, dv=dv)
    say("d_v=%d (%d tiles of 16), L=200" % (dv, dv // 16))
    check(make_delta(wl, DEV), tag="dv=%d" % dv)


def test_extreme_decay_and_strength():
    wl = BASE.with_(B=1, H=4, L=256)
    say("alpha = 0, alpha = 1 across a chunk boundary, log-decay -1000, beta = 0 and 1")
    x = make_delta(wl, DEV)
    x["log_alpha"][:, :, 10] = -float("inf")
    x["log_alpha"][:, :, 20:90] = 0.0
    x["log_alpha"][:, :, 100] = -1000.0
    x["beta"][:, :, 30:35] = 0.0
    x["beta"][:, :, 40:130] = 1.0
    check(x, tag="extreme gates")


def test_repeated_and_zero_keys():
    wl = BASE.with_(B=1, H=4, L=320)
    say("one key over a whole chunk with beta = 1, zero keys, zero queries")
    x = make_delta(wl, DEV)
    x["k"][:, :, 64:128] = x["k"][:, :, 64:65]
    x["beta"][:, :, 64:128] = 1.0
    x["log_alpha"][:, :, 64:128] = 0.0
    x["k"][:, :, 200:210] = 0.0
    x["q"][:, :, 220:230] = 0.0
    o = check(x, tag="repeated/zero keys")
    torch.cuda.synchronize()
    assert not bool(o[:, :, 220:230].any()), "a zero query reads nothing"


def test_workspace_given_and_reused():
    wl = BASE.with_(B=1, H=4, L=300)
    say("explicit workspace, reused across calls; too small a workspace is refused")
    x = make_delta(wl, DEV)
    desc = G.make_desc(wl.B, wl.H, wl.L, wl.d, wl.dv, wl.d, dtype=G.GLAH_BF16)
    need = G.gdn_workspace_bytes(desc)
    assert need == wl.B * wl.H * 5 * 13568
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    o_fresh = run(x)
    y = make_delta(wl.with_(seed=wl.seed + 1), DEV)
    run(y, ws=ws)  # leaves other records in the workspace
    o_ws = run(x, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(o_ws, o_fresh)
    with pytest.raises(G.GlahError):
        run(x, ws=ws[:need - 1])
