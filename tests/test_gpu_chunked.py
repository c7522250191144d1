"""GPU parity of the chunkwise MFMA path (bf16, d = f = d_v = 128, 64-token
chunks) against the fp64 oracle on the same seeded inputs.

The base workloads (2K and 32K-token LLaMA-3-8B-shaped layers, the batch-8
strong-decay layer) barely exercise the inter-chunk state pass, because their
gates decay the state within a few chunks; the slow-decay, gate=1 and
state-continuation cases make the state pass carry real signal, and the peaked
case makes the window softmax far from uniform."""
import numpy as np
import pytest
import torch

import oracle
from gated_linear_attention_hybrid_amd import binding as G
from gated_linear_attention_hybrid_amd.inputs import WORKLOADS, make_prefill, to_f64
from parity import TOL_BF16, assert_finite, gpu_f64, row_rel_err, seeded_randn

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print("[case]", msg, flush=True)


def run_hybrid(x, wl, gate_is_log=False, **kw):
    return G.hybrid_layer_fwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"],
                              window=wl.window, chunk=64, gate_is_log=gate_is_log, **kw)


def ref(x, wl, parts=oracle.PART_BOTH, gate_is_log=False, heads=None, **kw):
    """Oracle output; ``heads`` = list of (b, h) pairs restricts it to those heads."""
    if heads is None:
        o = {k: to_f64(v) for k, v in x.items()}
        return oracle.layer_fwd(o["q"], o["k"], o["v"], o["gate"], o["wq"], o["wk"], o["meta"],
                                window=wl.window, gate_is_log=gate_is_log, parts=parts, **kw)
    outs = []
    for b, h in heads:
        o = {k: to_f64(v[b:b + 1, h:h + 1]) for k, v in x.items() if v.dim() == 4}
        w = {k: to_f64(x[k][h:h + 1]) for k in ("wq", "wk", "meta")}
        outs.append(oracle.layer_fwd(o["q"], o["k"], o["v"], o["gate"], w["wq"], w["wk"], w["meta"],
                                     window=wl.window, gate_is_log=gate_is_log, parts=parts)[0, 0])
    return np.stack(outs)


def ref_states(x, wl, heads):
    """Oracle outputs and final states of the sampled (b, h) heads, run as one
    batch row of len(heads) heads (OpenMP over heads)."""
    tok = {k: np.stack([to_f64(x[k][b, h]) for b, h in heads])[None] for k in ("q", "k", "v", "gate")}
    w = {k: np.stack([to_f64(x[k][h]) for _, h in heads]) for k in ("wq", "wk", "meta")}
    o, s = oracle.layer_fwd(tok["q"], tok["k"], tok["v"], tok["gate"], w["wq"], w["wk"], w["meta"],
                            window=wl.window, return_state=True)
    return o[0], s[0]


def base(H=4, **kw):
    return WORKLOADS["prefill_2k"].with_(H=H, **kw)


def test_prefill_2k_full():
    wl = WORKLOADS["prefill_2k"]
    say("hybrid prefill_2k all 32 heads")
    x = make_prefill(wl, DEV)
    o = run_hybrid(x, wl)
    assert_finite(o, "o")
    assert row_rel_err(gpu_f64(o), ref(x, wl)) <= TOL_BF16


@pytest.mark.parametrize("variant", ["slow_decay", "gate_one", "peaked", "strong_decay"])
def test_hybrid_variants(variant):
    wl = base(L=1024)
    gate_is_log = False
    if variant == "slow_decay":
        wl = wl.with_(gate_mean=6.0)
    elif variant == "peaked":
        wl = wl.with_(x_std=1.0, w_std=1.0 / np.sqrt(128.0))
    elif variant == "strong_decay":
        wl = wl.with_(gate_mean=-2.0, gate_std=1.5)
    say("hybrid variant %s" % variant)
    x = make_prefill(wl, DEV, gate_log_zero=(variant == "gate_one"))
    gate_is_log = variant == "gate_one"
    o = run_hybrid(x, wl, gate_is_log=gate_is_log)
    assert_finite(o, "o")
    assert row_rel_err(gpu_f64(o), ref(x, wl, gate_is_log=gate_is_log)) <= TOL_BF16


@pytest.mark.parametrize("extreme", ["logits_plus30", "logits_minus30", "log_minus_inf", "mixed"])
def test_extreme_gates(extreme):
    wl = base(H=2, L=300)
    say("extreme gates %s" % extreme)
    x = make_prefill(wl, DEV)
    gate_is_log = False
    g = x["gate"]
    if extreme == "logits_plus30":
        g = torch.full_like(g, 30.0)
    elif extreme == "logits_minus30":
        g = torch.full_like(g, -30.0)
    elif extreme == "log_minus_inf":
        gate_is_log = True
        g = torch.full_like(g, float("-inf"))
    else:  # random mix of open, shut and ordinary gates
        gen = torch.Generator(device=DEV).manual_seed(7)
        r = torch.rand(g.shape, generator=gen, device=DEV)
        g = torch.where(r < 0.1, torch.full_like(g, -30.0), torch.where(r > 0.8, torch.full_like(g, 30.0), g))
    x = dict(x, gate=g.contiguous())
    o = run_hybrid(x, wl, gate_is_log=gate_is_log)
    assert_finite(o, "o")
    assert row_rel_err(gpu_f64(o), ref(x, wl, gate_is_log=gate_is_log)) <= TOL_BF16


def test_gla_and_swa_parts():
    wl = base(L=700, gate_mean=5.0)
    say("gla_prefill and swa_meta_attn (MFMA)")
    x = make_prefill(wl, DEV)
    o = G.gla_prefill(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], chunk=64)
    assert row_rel_err(gpu_f64(o), ref(x, wl, parts=oracle.PART_GLA)) <= TOL_BF16
    o = G.swa_meta_attn(x["q"], x["k"], x["v"], x["meta"], window=wl.window)
    assert row_rel_err(gpu_f64(o), ref(x, wl, parts=oracle.PART_SWA)) <= TOL_BF16


@pytest.mark.parametrize("L", [1, 15, 63, 64, 65, 200, 1000])
def test_ragged_lengths(L):
    wl = base(H=3, B=2, L=L, gate_mean=4.0)
    say("ragged L=%d" % L)
    x = make_prefill(wl, DEV)
    o = run_hybrid(x, wl)
    assert row_rel_err(gpu_f64(o), ref(x, wl)) <= TOL_BF16


@pytest.mark.parametrize("window", [1, 2, 17, 63])
def test_windows(window):
    wl = base(H=2, L=333, window=window, x_std=0.5)
    say("window %d" % window)
    x = make_prefill(wl, DEV)
    o = run_hybrid(x, wl)
    assert row_rel_err(gpu_f64(o), ref(x, wl)) <= TOL_BF16


def test_no_sinks():
    wl = base(H=2, L=256, n_meta=0)
    say("no meta sinks")
    x = make_prefill(wl, DEV)
    x["meta"] = torch.zeros((wl.H, 0), device=DEV)
    o = G.hybrid_layer_fwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], None,
                           window=wl.window)
    assert row_rel_err(gpu_f64(o), ref(x, wl)) <= TOL_BF16


@pytest.mark.parametrize("H", [1, 8, 40])
def test_segment_splits(H):
    # the number of heads changes how many sequence segments run in parallel
    wl = base(H=H, L=1536, gate_mean=6.0)
    say("segment split H=%d" % H)
    x = make_prefill(wl, DEV)
    o = run_hybrid(x, wl)
    heads = [(0, h) for h in sorted(set([0, H // 2, H - 1]))]
    got = gpu_f64(o)
    assert row_rel_err(np.stack([got[b, h] for b, h in heads]), ref(x, wl, heads=heads)) <= TOL_BF16


def test_state_slices_with_empty_slice():
    # 128 sequences of 18 chunks on 256 compute units: 2 output segments of 9
    # chunks, and the state pass cuts segment 0 into 4 slices of 3 chunks, the
    # last of which is empty (zero state, zero decay)
    wl = base(B=2, H=64, L=18 * 64, gate_mean=6.0)
    say("state slices B=2 H=64 L=1152")
    x = make_prefill(wl, DEV)
    st = torch.empty((wl.B, wl.H, wl.f, wl.dv), device=DEV)
    o = run_hybrid(x, wl, state_out=st)
    heads = [(0, 0), (0, 37), (1, 63)]
    got = gpu_f64(o)
    want, wst = [], []
    for b, h in heads:
        oo = {k: to_f64(v[b:b + 1, h:h + 1]) for k, v in x.items() if v.dim() == 4}
        w = {k: to_f64(x[k][h:h + 1]) for k in ("wq", "wk", "meta")}
        r, s = oracle.layer_fwd(oo["q"], oo["k"], oo["v"], oo["gate"], w["wq"], w["wk"], w["meta"],
                                window=wl.window, return_state=True)
        want.append(r[0, 0])
        wst.append(s[0, 0])
    assert row_rel_err(np.stack([got[b, h] for b, h in heads]), np.stack(want)) <= TOL_BF16
    sg = gpu_f64(st)
    assert row_rel_err(np.stack([sg[b, h] for b, h in heads]).reshape(-1, wl.dv),
                       np.stack(wst).reshape(-1, wl.dv)) <= TOL_BF16


def test_state_in_out_continuation():
    wl = base(H=4, L=1280, gate_mean=6.0)
    say("state continuation")
    x = make_prefill(wl, DEV)
    L1 = 512
    first = {k: (v[:, :, :L1].contiguous() if v.dim() == 4 else v) for k, v in x.items()}
    rest = {k: (v[:, :, L1:].contiguous() if v.dim() == 4 else v) for k, v in x.items()}
    st = torch.empty((wl.B, wl.H, wl.f, wl.dv), device=DEV)
    G.gla_prefill(first["q"], first["k"], first["v"], first["gate"], first["wq"], first["wk"],
                  state_out=st)
    o2 = G.gla_prefill(rest["q"], rest["k"], rest["v"], rest["gate"], rest["wq"], rest["wk"],
                       state_in=st, state_out=st)
    full, sfull = ref(x, wl, parts=oracle.PART_GLA, return_state=True)
    assert row_rel_err(gpu_f64(o2), full[:, :, L1:]) <= TOL_BF16
    assert row_rel_err(gpu_f64(st).reshape(-1, wl.dv), sfull.reshape(-1, wl.dv)) <= TOL_BF16


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_empty_sequence_passes_the_state(dtype):
    """L = 0: state_out is the state before the sequence (state_in, or zeros
    without one) and the returned ring is all zeros, on both entry points."""
    wl = base(H=3, L=0)
    say("empty sequence, %s" % dtype)
    x = make_prefill(wl.with_(L=64), DEV)
    x = {k: (v[:, :, :0].to(dtype).contiguous() if v.dim() == 4 else v.to(dtype) if k in ("wq", "wk") else v)
         for k, v in x.items()}
    sin = seeded_randn((wl.B, wl.H, wl.f, wl.dv), 41, DEV)
    for with_in in (True, False):
        sout = torch.full_like(sin, 7.0)
        G.gla_prefill(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"],
                      state_in=sin if with_in else None, state_out=sout)
        torch.cuda.synchronize()
        assert torch.equal(sout, sin if with_in else torch.zeros_like(sin))
        sout = torch.full_like(sin, 7.0)
        kc = torch.full((wl.B, wl.H, wl.window, wl.d), 3.0, device=DEV, dtype=dtype)
        vc = torch.full((wl.B, wl.H, wl.window, wl.dv), 3.0, device=DEV, dtype=dtype)
        run_hybrid(x, wl, state_in=sin if with_in else None, state_out=sout, kcache_out=kc, vcache_out=vc)
        torch.cuda.synchronize()
        assert torch.equal(sout, sin if with_in else torch.zeros_like(sin))
        assert not kc.any() and not vc.any()


@pytest.mark.parametrize("L", [200, 40, 2000])
def test_window_cache_out_mfma(L):
    """The decode ring written by each head's last output-pass block: one segment
    (L = 200), fewer tokens than the window (slots of tokens before 0 are
    zeros), and seven segments (L = 2000)."""
    wl = base(H=2, L=L)
    say("window cache out (MFMA path), L=%d" % L)
    x = make_prefill(wl, DEV)
    kc = torch.full((wl.B, wl.H, wl.window, wl.d), 3.0, device=DEV, dtype=torch.bfloat16)
    vc = torch.full((wl.B, wl.H, wl.window, wl.dv), 3.0, device=DEV, dtype=torch.bfloat16)
    run_hybrid(x, wl, kcache_out=kc, vcache_out=vc)
    torch.cuda.synchronize()
    for p in range(wl.L - wl.window, wl.L):
        if p < 0:
            assert not kc[:, :, p % wl.window].any() and not vc[:, :, p % wl.window].any()
        else:
            assert torch.equal(kc[:, :, p % wl.window], x["k"][:, :, p])
            assert torch.equal(vc[:, :, p % wl.window], x["v"][:, :, p])


def test_deterministic():
    wl = base(H=4, L=640)
    say("bitwise determinism")
    x = make_prefill(wl, DEV)
    a = run_hybrid(x, wl).clone()
    b = run_hybrid(x, wl)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_prefill_32k_sampled_heads():
    wl = WORKLOADS["prefill_32k"]
    say("hybrid prefill_32k, oracle on 3 sampled heads")
    x = make_prefill(wl, DEV)
    st = torch.empty((wl.B, wl.H, wl.f, wl.dv), device=DEV)
    o = run_hybrid(x, wl, state_out=st)
    assert_finite(o, "o")
    heads = [(0, 0), (0, 17), (0, 31)]
    got = gpu_f64(o)
    exp, sexp = ref_states(x, wl, heads)
    assert row_rel_err(np.stack([got[b, h] for b, h in heads]), exp) <= TOL_BF16
    # the final state (what a decode continuing this prefill starts from)
    assert_finite(st, "state_out")
    sg = gpu_f64(st)
    assert row_rel_err(np.stack([sg[b, h] for b, h in heads]).reshape(-1, wl.dv),
                       sexp.reshape(-1, wl.dv)) <= TOL_BF16


def test_strong_decay_8k_sampled_heads():
    wl = WORKLOADS["strong_decay_8k"]
    say("strong decay B=8 L=8192, oracle on 4 sampled heads")
    x = make_prefill(wl, DEV)
    # the workload names 128-token chunks; the MFMA path serves that request with
    # its 64-token blocking, so it must give exactly what a 64-token request gives
    st = torch.empty((wl.B, wl.H, wl.f, wl.dv), device=DEV)
    o = G.hybrid_layer_fwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"],
                           window=wl.window, chunk=wl.chunk, state_out=st)
    o64 = G.hybrid_layer_fwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"],
                             window=wl.window, chunk=64)
    assert wl.chunk == 128 and torch.equal(o, o64)
    assert_finite(o, "o")
    assert_finite(st, "state_out")
    heads = [(0, 0), (3, 9), (5, 20), (7, 31)]
    got = gpu_f64(o)
    exp, sexp = ref_states(x, wl, heads)
    assert row_rel_err(np.stack([got[b, h] for b, h in heads]), exp) <= TOL_BF16
    sg = gpu_f64(st)
    assert row_rel_err(np.stack([sg[b, h] for b, h in heads]).reshape(-1, wl.dv),
                       sexp.reshape(-1, wl.dv)) <= TOL_BF16


def test_inter_chunk_readout_margin():
    """The inter-chunk readout q-bar S takes the fp32 state rounded once to bf16
    as its matrix-core operand (as q-bar itself is).  With gate = 1 nothing
    decays, so every row past the first chunk carries the readout of a state
    built from all earlier tokens.  Each bf16 operand rounding is at most 2^-9
    relative per term, as is the rounding of the output itself; the typical
    row (the median past the first chunk) must stay below two such roundings,
    2^-8, and the worst row within the bf16 tolerance."""
    wl = WORKLOADS["prefill_2k"]
    say("gate = 1, 2K x 32 heads, gated part: readout precision margin")
    x = make_prefill(wl, DEV, gate_log_zero=True)
    o = G.gla_prefill(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], gate_is_log=True)
    got = gpu_f64(o)
    exp = ref(x, wl, parts=oracle.PART_GLA, gate_is_log=True)
    assert row_rel_err(got, exp) <= TOL_BF16
    g2, r2 = got[:, :, 64:].reshape(-1, wl.dv), exp[:, :, 64:].reshape(-1, wl.dv)
    rows = np.max(np.abs(g2 - r2), axis=-1) / np.max(np.abs(r2), axis=-1)
    assert float(np.median(rows)) <= 2.0 ** -8, float(np.median(rows))


@pytest.mark.parametrize("window", [65, 100, 200, 700, 5000])
def test_wide_windows(window):
    """Windows wider than one 64-token chunk: the window part runs with an online
    softmax over key chunks (swa_meta_attn alone, and after the chunked gated
    part in the hybrid layer, which adds it to o); 5000 >= L is the full causal
    softmax with sinks.  Ragged length, peaked scores, two batch rows."""
    wl = base(B=2, H=2, L=1000, window=window, x_std=0.5)
    say("wide window %d" % window)
    x = make_prefill(wl, DEV)
    o = G.swa_meta_attn(x["q"], x["k"], x["v"], x["meta"], window=window)
    assert_finite(o, "o_swa")
    assert row_rel_err(gpu_f64(o), ref(x, wl, parts=oracle.PART_SWA)) <= TOL_BF16
    st = torch.empty((wl.B, wl.H, wl.f, wl.dv), device=DEV)
    kc = torch.full((wl.B, wl.H, window, wl.d), 3.0, device=DEV, dtype=torch.bfloat16)
    vc = torch.full((wl.B, wl.H, window, wl.dv), 3.0, device=DEV, dtype=torch.bfloat16)
    o = G.hybrid_layer_fwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"], window=window,
                           state_out=st, kcache_out=kc, vcache_out=vc)
    assert_finite(o, "o")
    exp, sexp = ref(x, wl, return_state=True)
    assert row_rel_err(gpu_f64(o), exp) <= TOL_BF16
    assert row_rel_err(gpu_f64(st).reshape(-1, wl.dv), sexp.reshape(-1, wl.dv)) <= TOL_BF16
    torch.cuda.synchronize()
    for p in range(max(0, wl.L - window), wl.L):  # ring slot p % window holds token p
        assert torch.equal(kc[:, :, p % window], x["k"][:, :, p])
        assert torch.equal(vc[:, :, p % window], x["v"][:, :, p])
    if window > wl.L:  # slots of tokens before 0 are zero-filled
        assert not kc[:, :, wl.L:].any() and not vc[:, :, wl.L:].any()


def test_wide_window_no_sinks_and_short():
    """No sinks, and sequences shorter than the window (the first chunk alone)."""
    for L, window in ((300, 129), (40, 100)):
        wl = base(H=3, L=L, window=window, n_meta=0, x_std=0.7)
        say("wide window %d, L %d, no sinks" % (window, L))
        x = make_prefill(wl, DEV)
        o = G.hybrid_layer_fwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], None, window=window)
        x["meta"] = torch.zeros((wl.H, 0), device=DEV)
        assert row_rel_err(gpu_f64(o), ref(x, wl)) <= TOL_BF16
