"""The no-allocation entry point (hybrid_layer_fwd_noalloc) gives what
hybrid_layer_fwd gives with a caller workspace: two calls in a row through the
C ABI, the second with a smaller input (the scratch array then still holds the
first call's segment states), compared bitwise (the same kernels run on the
same inputs) on the output, the final state and the window ring.  A third call
checks a size that needs no segment states at all."""
import pytest
import torch

from gated_linear_attention_hybrid_amd import binding as G
from gated_linear_attention_hybrid_amd.inputs import WORKLOADS, make_prefill
from parity import seeded_randn

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _both(wl, with_state_in):
    x = make_prefill(wl, DEV)
    B, H = wl.B, wl.H
    sin = seeded_randn((B, H, wl.f, wl.dv), 44, DEV) if with_state_in else None
    outs = []
    for noalloc in (True, False):
        st = torch.empty((B, H, wl.f, wl.dv), device=DEV)
        kc = torch.empty((B, H, wl.window, wl.d), device=DEV, dtype=wl.torch_dtype)
        vc = torch.empty((B, H, wl.window, wl.dv), device=DEV, dtype=wl.torch_dtype)
        o = torch.empty((B, H, wl.L, wl.dv), device=DEV, dtype=wl.torch_dtype)
        kw = dict(window=wl.window, state_in=sin, state_out=st, kcache_out=kc, vcache_out=vc)
        if noalloc:
            G.hybrid_layer_fwd_noalloc(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"], o, **kw)
        else:
            G.hybrid_layer_fwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"], o=o, **kw)
        torch.cuda.synchronize()
        outs.append((o, st, kc, vc))
    return outs


def test_noalloc_matches_workspace_call():
    wl_big = WORKLOADS["prefill_32k"]  # the largest workspace: 32 heads x 14 state slices
    wl_small = WORKLOADS["prefill_2k"].with_(H=4, L=1000, gate_mean=6.0)
    wl_none = WORKLOADS["prefill_2k"].with_(B=8, H=32, L=640)  # one segment per head: no states
    for name, wl, sin in (("32k", wl_big, False), ("small, state in", wl_small, True),
                          ("no segment states", wl_none, False)):
        print("[case] noalloc", name, flush=True)
        desc = G.make_desc(wl.B, wl.H, wl.L, wl.d, wl.dv, wl.f, window=wl.window, n_meta=wl.n_meta)
        assert G.workspace_bytes(desc) <= 40 << 20
        a, b = _both(wl, sin)
        for x, y, what in zip(a, b, ("o", "state", "kcache", "vcache")):
            assert torch.equal(x, y), (name, what)
