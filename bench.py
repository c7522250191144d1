"""Benchmark of the hybrid gated-linear + window attention layer on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one hybrid_layer_fwd over the 32K-token LLaMA-3-8B-shaped layer
(B=1, H=32, L=32768, d = f = d_v = 128, window 64, 4 meta sinks, bf16 inputs,
fp32 state), writing o, the final state and the window cache.  Inputs are
seeded synthetic tensors already resident in HBM.  Prints one JSON line with
tokens/s, the live roofline of the call (HIP events on the stream the library
launches on), a decode leg (batch 8, 32 heads, 256 graph-captured steps rotating
over 12 state sets so the 256 MB last-level cache cannot hold them) and the fp64
oracle timed on the host cores on a bounded sample of the same workload.

The other legs (device ceilings, decode, the 2K-token prefill with the
last-level cache flushed, the batch-8 8K strong-decay prefill, backward, gated
delta rule, serving pieces) run before the headline call, which is then timed
at the clocks the GPU settles to under sustained work; its per-call spread
(min, median, max, first and last five) is part of the line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA

# algorithmic counts per token-head at d = f = d_v = 128, 64-token chunks, w = 64:
#   bytes: q, k, v, gate read once (4 x 256 B) + o written once (256 B)
#   MACs:  Hedgehog 2*128*64 + intra (64+1)/2*(128+128) + inter 128*128
#          + state 128*128 + window 64*(128+128)
PREFILL_BYTES_PER_TOKEN_HEAD = 1280
PREFILL_FLOPS_PER_TOKEN_HEAD = 2 * (2 * 128 * 64 + 65 * 128 + 128 * 128 + 128 * 128 + 64 * 256)
# MFMA work the kernels execute per token-head at the 32K workload (16x16x32 bf16
# MFMAs of 16384 flops).  Output pass, per 64-token chunk of a head: readout 128,
# weights x V 96, state update 128, the two projections 128, window bands 80,
# intra tiles 40 = 600 MFMAs; state pass (7/8 of the tokens): projection 64 +
# update 128 = 192 per chunk.  Transposes on the matrix core (0/1 selection
# operands, no arithmetic work) are counted apart: 32 per output-pass chunk, 32
# per state-pass chunk (the k-hat^T fragments).
PREFILL_EXECUTED_FLOPS_PER_TOKEN_HEAD = (600 * 16384 + 192 * 16384 * 7 // 8) // 64
PREFILL_TRANSPOSE_FLOPS_PER_TOKEN_HEAD = (32 * 16384 + 32 * 16384 * 7 // 8) // 64


# backward at d = f = d_v = 128 (bf16): q, k, v, gate and dO read once, dq, dk,
# dv and dgate written once (9 x 256 B); the projections and sinks are per head
BACKWARD_BYTES_PER_TOKEN_HEAD = 9 * 256


def decode_bytes_per_step(B, H, d, f, dv, w, bpe=2):
    state = B * H * f * dv * 4 * 2          # fp32 state read + written
    ring = B * H * w * (d + dv) * bpe       # window keys and values read
    wphi = H * d * (f // 2) * bpe * 2       # two Hedgehog projections
    io = B * H * (d + d + dv + f + dv) * bpe  # q, k, v, gate in; o out
    return state + ring + wphi + io


# Sources of the kernels and host dispatch of one hybrid_layer_fwd prefill call:
# the stored HBM traffic of that call stays valid while these are unchanged.
PREFILL_SOURCES = ("capi.cpp", "chunk_common.hpp", "chunk_out.hip", "chunked.hip", "device_common.hpp",
                   "launch.hpp")


def source_hash(names=None):
    """Hash of the named csrc files (all of them by default)."""
    h = hashlib.sha256()
    cs = os.path.join(ROOT, "gated_linear_attention_hybrid_amd", "csrc")
    for name in sorted(names if names is not None else os.listdir(cs)):
        with open(os.path.join(cs, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(key):
    """HBM traffic per launch from the committed rocprofv3 counter summary, only
    when the sources it was taken on (the entry's file list) are unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = rec.get(key)
    if not ent or ent.get("source_hash") != source_hash(ent.get("sources")):
        return None
    return ent.get("bytes_per_launch")


def bench_prefill(G, wl, steps, warmup, torch):
    from gated_linear_attention_hybrid_amd.inputs import make_prefill
    dev = torch.device("cuda")
    x = make_prefill(wl, dev)
    o = torch.empty((wl.B, wl.H, wl.L, wl.dv), dtype=wl.torch_dtype, device=dev)
    st = torch.empty((wl.B, wl.H, wl.f, wl.dv), dtype=torch.float32, device=dev)
    kc = torch.empty((wl.B, wl.H, wl.window, wl.d), dtype=wl.torch_dtype, device=dev)
    vc = torch.empty((wl.B, wl.H, wl.window, wl.dv), dtype=wl.torch_dtype, device=dev)
    desc = G.make_desc(wl.B, wl.H, wl.L, wl.d, wl.dv, wl.f, window=wl.window, n_meta=wl.n_meta,
                       chunk=wl.chunk, dtype=G.GLAH_BF16)
    ws = torch.empty(max(1, G.workspace_bytes(desc)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        G.hybrid_layer_fwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"],
                           window=wl.window, chunk=wl.chunk, state_out=st, kcache_out=kc,
                           vcache_out=vc, o=o, ws=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    calls = [a.elapsed_time(b) for a, b in ev]
    bad = int((~torch.isfinite(o.float())).sum().item())
    del x
    return wall / steps * 1e3, calls, bad


def spread_us(calls_ms):
    """Per-call spread of HIP-event times (microseconds): min, median, max, and
    the mean of the first and of the last five calls (clock ramp shows as a
    first-five mean above the last-five one)."""
    s = sorted(calls_ms)
    k = min(5, len(calls_ms))
    return {"min": round(s[0] * 1e3, 2), "median": round(s[len(s) // 2] * 1e3, 2), "max": round(s[-1] * 1e3, 2),
            "first5_mean": round(sum(calls_ms[:k]) / k * 1e3, 2),
            "last5_mean": round(sum(calls_ms[-k:]) / k * 1e3, 2), "calls": len(calls_ms)}


def bench_prefill_config(G, torch, wl, reps=30, warmup=3, flush=False):
    """One hybrid_layer_fwd over a further prefill workload (parity-test shapes
    of the pages' setting), timed per call with HIP events on the launch stream;
    with ``flush`` a 1 GiB buffer is written before every call (outside the
    events), so inputs smaller than the 256 MB last-level cache come from HBM."""
    from gated_linear_attention_hybrid_amd.inputs import make_prefill
    dev = torch.device("cuda")
    x = make_prefill(wl, dev)
    o = torch.empty((wl.B, wl.H, wl.L, wl.dv), dtype=wl.torch_dtype, device=dev)
    st = torch.empty((wl.B, wl.H, wl.f, wl.dv), dtype=torch.float32, device=dev)
    desc = G.make_desc(wl.B, wl.H, wl.L, wl.d, wl.dv, wl.f, window=wl.window, n_meta=wl.n_meta,
                       chunk=wl.chunk, dtype=G.GLAH_BF16)
    ws = torch.empty(max(1, G.workspace_bytes(desc)), dtype=torch.uint8, device=dev)
    junk = torch.empty(1 << 28, dtype=torch.float32, device=dev) if flush else None
    stream = torch.cuda.current_stream()

    def call():
        G.hybrid_layer_fwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"], window=wl.window,
                           chunk=wl.chunk, state_out=st, o=o, ws=ws, stream=stream)

    for _ in range(warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        if flush:
            junk.fill_(float(i))
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    calls = [a.elapsed_time(b) for a, b in ev]
    ms = sorted(calls)[reps // 2]
    th = wl.B * wl.H * wl.L
    nbytes, nflops = PREFILL_BYTES_PER_TOKEN_HEAD * th, PREFILL_FLOPS_PER_TOKEN_HEAD * th
    achieved = nbytes / (ms * 1e-3) / 1e9
    bad = int((~torch.isfinite(o.float())).sum().item())
    del x, o, st, ws, junk
    return {"workload": "%s: B=%d H=%d L=%d d=f=d_v=%d chunk %d window %d, %d sinks, bf16, gate logits~N(%g,%g)%s"
                        % (wl.name, wl.B, wl.H, wl.L, wl.d, wl.chunk, wl.window, wl.n_meta, wl.gate_mean,
                           wl.gate_std, ", last-level cache flushed before each call" if flush else ""),
            "us_per_call": round(ms * 1e3, 2), "tokens_per_s": round(wl.B * wl.L / (ms * 1e-3), 1),
            "spread_us": spread_us(calls),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": nbytes,
                         "hbm_floor_us": round(nbytes / (HBM_PEAK_GBS * 1e9) * 1e6, 1),
                         "mfma_frac": round(nflops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
            "nonfinite_outputs": bad}


def bench_decode(G, torch, steps=256, sets=12, prefix=32768):
    from gated_linear_attention_hybrid_amd.inputs import WORKLOADS, make_decode_token, make_prefill
    wl = WORKLOADS["decode_b8"]
    dev = torch.device("cuda")
    B, H = wl.B, wl.H
    # state and ring from a seeded 32K-token prefill of the whole batch
    x = make_prefill(wl.with_(L=prefix), dev)
    st = torch.empty((B, H, wl.f, wl.dv), dtype=torch.float32, device=dev)
    kc = torch.empty((B, H, wl.window, wl.d), dtype=wl.torch_dtype, device=dev)
    vc = torch.empty((B, H, wl.window, wl.dv), dtype=wl.torch_dtype, device=dev)
    desc = G.make_desc(B, H, prefix, wl.d, wl.dv, wl.f, window=wl.window, n_meta=wl.n_meta,
                       chunk=64, dtype=G.GLAH_BF16)
    ws = torch.empty(max(1, G.workspace_bytes(desc)), dtype=torch.uint8, device=dev)
    G.hybrid_layer_fwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"],
                       window=wl.window, state_out=st, kcache_out=kc, vcache_out=vc, ws=ws)
    wq, wk, meta = x["wq"], x["wk"], x["meta"]
    torch.cuda.synchronize()
    del x, ws
    # independent state/ring sets (a stack of layers), each a copy of the prefill
    states = [st.clone() for _ in range(sets)]
    kcs = [kc.clone() for _ in range(sets)]
    vcs = [vc.clone() for _ in range(sets)]
    toks = [make_decode_token(wl, s, dev) for s in range(steps)]
    pos = [torch.full((B,), prefix + s // sets, dtype=torch.int32, device=dev) for s in range(steps)]
    outs = [torch.empty((B, H, wl.dv), dtype=wl.torch_dtype, device=dev) for _ in range(steps)]

    def run_all(stream):
        for s in range(steps):
            t = toks[s]
            j = s % sets
            G.gla_decode_step(t["q"], t["k"], t["v"], t["gate"], wq, wk, meta, states[j], kcs[j],
                              vcs[j], pos[s], window=wl.window, o=outs[s], stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all(side)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_all(torch.cuda.current_stream())
    for _ in range(3):  # untimed replays
        graph.replay()
    torch.cuda.synchronize()
    reps = 5
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record()
        graph.replay()
        ev[i][1].record()
    torch.cuda.synchronize()
    per_rep = [a.elapsed_time(b) / steps for a, b in ev]  # ms per step of each replay
    ms_step = sum(per_rep) / reps
    bad = int((~torch.isfinite(outs[-1].float())).sum().item())
    nbytes = decode_bytes_per_step(B, H, wl.d, wl.f, wl.dv, wl.window)
    return {
        "workload": "decode_b8: B=8 H=32 state 128x128 fp32, window 64, 4 sinks, prefix %d" % prefix,
        "steps_per_graph": steps, "state_sets": sets,
        "us_per_step": round(ms_step * 1e3, 3),
        "us_per_step_by_replay": [round(t * 1e3, 3) for t in per_rep],
        "tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (ms_step * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_step": nbytes},
        "nonfinite_outputs": bad,
    }


def bench_backward(G, torch, wl, reps=5, warmup=2):
    """hybrid_layer_bwd over one prefill workload: gradients of every input for a
    seeded upstream gradient dO, timed with HIP events on the launch stream."""
    from gated_linear_attention_hybrid_amd.inputs import make_prefill
    dev = torch.device("cuda")
    x = make_prefill(wl, dev)
    gen = torch.Generator(device=dev).manual_seed(wl.seed + 77)
    dO = torch.randn((wl.B, wl.H, wl.L, wl.dv), generator=gen, device=dev).to(wl.torch_dtype)
    desc = G.make_desc(wl.B, wl.H, wl.L, wl.d, wl.dv, wl.f, window=wl.window, n_meta=wl.n_meta,
                       dtype=G.GLAH_BF16)
    stream = torch.cuda.current_stream()

    def timed(ws):
        def call():
            return G.hybrid_layer_bwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"], dO,
                                      window=wl.window, ws=ws, stream=stream)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            ev[i][0].record(stream)
            g = call()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)[reps // 2], g

    # the workspace the library reports (a call above 1.5e9 bytes runs as
    # sub-problems of whole heads), and the whole call's for comparison
    ws_bytes = max(1, G.bwd_workspace_bytes(desc))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ms, g = timed(ws)
    bad = sum(int((~torch.isfinite(t.float())).sum().item()) for t in g.values() if t is not None)
    del ws, g
    whole = None
    whole_bytes = G.bwd_workspace_bytes_whole(desc)
    if whole_bytes > ws_bytes:
        wsw = torch.empty(whole_bytes, dtype=torch.uint8, device=dev)
        msw, g = timed(wsw)
        whole = {"ms_per_call": round(msw, 3), "workspace_bytes": whole_bytes}
        del wsw, g
    nbytes = BACKWARD_BYTES_PER_TOKEN_HEAD * wl.B * wl.H * wl.L
    achieved = nbytes / (ms * 1e-3) / 1e9
    del x, dO
    return {"workload": "%s: B=%d H=%d L=%d d=f=d_v=%d window %d, %d sinks, bf16"
                        % (wl.name, wl.B, wl.H, wl.L, wl.d, wl.window, wl.n_meta),
            "ms_per_call": round(ms, 3), "tokens_per_s": round(wl.B * wl.L / (ms * 1e-3), 1),
            "workspace_bytes": ws_bytes, "whole_call_workspace": whole,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": nbytes},
            "nonfinite_outputs": bad}


# gated delta rule at d = d_v = 128, bf16: q, k, v read and o written once
# (4 x 256 B) plus the log-decay and write strength (2 x 2 B) per token-head
DELTA_BYTES_PER_TOKEN_HEAD = 4 * 256 + 2 * 2


def bench_delta(G, torch, reps=5, warmup=2, steps=256, sets=12):
    """gdn_prefill over the 32K-token shape (32 heads of 128) and the gdn_decode_step
    at batch 8 (256 graph-captured steps rotating over 12 state sets), each against
    the HBM roofline of its algorithmic bytes."""
    from gated_linear_attention_hybrid_amd.inputs import WORKLOADS, make_delta, make_delta_token
    dev = torch.device("cuda")
    wl = WORKLOADS["prefill_32k"]
    x = make_delta(wl, dev)
    st = torch.empty((wl.B, wl.H, wl.dv, wl.d), device=dev)
    o = torch.empty((wl.B, wl.H, wl.L, wl.dv), dtype=wl.torch_dtype, device=dev)
    desc = G.make_desc(wl.B, wl.H, wl.L, wl.d, wl.dv, wl.d, dtype=G.GLAH_BF16)
    ws = torch.empty(max(1, G.gdn_workspace_bytes(desc)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        G.gdn_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], state_out=st, o=o, ws=ws, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    nbytes = DELTA_BYTES_PER_TOKEN_HEAD * wl.B * wl.H * wl.L
    pre = {"workload": "gdn prefill: B=%d H=%d L=%d d=d_v=%d bf16, fp32 state" % (wl.B, wl.H, wl.L, wl.d),
           "ms_per_call": round(ms, 3), "tokens_per_s": round(wl.B * wl.L / (ms * 1e-3), 1),
           "roofline": {"bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "algorithmic_bytes_per_launch": nbytes},
           "workspace_bytes": ws.numel(),
           "nonfinite_outputs": int((~torch.isfinite(o.float())).sum().item())}
    del x, o, ws
    wd = WORKLOADS["decode_b8"]
    B, H = wd.B, wd.H
    x = make_delta(wd.with_(L=64), dev)
    st0 = torch.empty((B, H, wd.dv, wd.d), device=dev)
    G.gdn_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], state_out=st0)
    states = [st0.clone() for _ in range(sets)]
    toks = [make_delta_token(wd, s, dev) for s in range(steps)]
    outs = [torch.empty((B, H, wd.dv), dtype=wd.torch_dtype, device=dev) for _ in range(steps)]

    def run_all(strm):
        for s in range(steps):
            t = toks[s]
            G.gdn_decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], states[s % sets],
                              o=outs[s], stream=strm)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_all(torch.cuda.current_stream())
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (5 * steps)
    dbytes = B * H * wd.dv * wd.d * 4 * 2 + B * H * (3 * wd.d + wd.dv + 2) * 2
    dec = {"workload": "gdn decode: B=%d H=%d state %dx%d fp32, bf16 I/O" % (B, H, wd.dv, wd.d),
           "steps_per_graph": steps, "state_sets": sets, "us_per_step": round(us, 3),
           "tokens_per_s": round(B / (us * 1e-6), 1),
           "roofline": {"bound": "hbm", "achieved": round(dbytes / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(dbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "algorithmic_bytes_per_step": dbytes},
           "nonfinite_outputs": int((~torch.isfinite(outs[-1].float())).sum().item())}
    return {"prefill": pre, "decode": dec}


def bench_serving(G, torch, reps=20):
    """Serving pieces at the 32K layer shape: the output-gate epilogue over the
    whole output (HBM roofline: o read and written, g read, 3 x 256 B per
    token-head) and a 2048-token continuation prefill at position 30720 (state
    and window ring of the previous 30720 tokens in and out)."""
    from gated_linear_attention_hybrid_amd.inputs import WORKLOADS, make_prefill
    dev = torch.device("cuda")
    wl = WORKLOADS["prefill_32k"]
    gen = torch.Generator(device=dev).manual_seed(wl.seed + 91)
    o = torch.randn((wl.B, wl.H, wl.L, wl.dv), generator=gen, device=dev).to(wl.torch_dtype)
    g = torch.randn((wl.B, wl.H, wl.L, wl.dv), generator=gen, device=dev).to(wl.torch_dtype)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]

    ms = timed(lambda: G.output_gate(o, g, stream=stream))
    nbytes = 3 * o.numel() * o.element_size()
    gate = {"workload": "output gate o * sigmoid(g), [1,32,32768,128] bf16", "us_per_call": round(ms * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": nbytes}}
    del o, g
    pw = wl.with_(L=2048)
    x = make_prefill(pw, dev)
    start = 30720
    st = torch.randn((pw.B, pw.H, pw.f, pw.dv), generator=gen, device=dev) * 0.01
    kc = torch.randn((pw.B, pw.H, pw.window, pw.d), generator=gen, device=dev).to(pw.torch_dtype)
    vc = torch.randn((pw.B, pw.H, pw.window, pw.dv), generator=gen, device=dev).to(pw.torch_dtype)
    st_out, kco, vco = torch.empty_like(st), torch.empty_like(kc), torch.empty_like(vc)
    oo = torch.empty((pw.B, pw.H, pw.L, pw.dv), dtype=pw.torch_dtype, device=dev)
    desc = G.make_desc(pw.B, pw.H, pw.L, pw.d, pw.dv, pw.f, window=pw.window, n_meta=pw.n_meta, dtype=G.GLAH_BF16)
    ws = torch.empty(max(1, G.workspace_bytes(desc)), dtype=torch.uint8, device=dev)

    def cont():
        G.hybrid_layer_fwd_cont(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"], window=pw.window,
                                start=start, state_in=st, kcache_in=kc, vcache_in=vc, state_out=st_out,
                                kcache_out=kco, vcache_out=vco, o=oo, ws=ws, stream=stream)

    def whole():
        G.hybrid_layer_fwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"], window=pw.window,
                           state_in=st, state_out=st_out, kcache_out=kco, vcache_out=vco, o=oo, ws=ws,
                           stream=stream)

    ms_c, ms_w = timed(cont), timed(whole)
    contd = {"workload": "continuation prefill: 2048 tokens at position 30720, B=1 H=32 d=f=d_v=128, window 64",
             "us_per_call": round(ms_c * 1e3, 2), "tokens_per_s": round(pw.L / (ms_c * 1e-3), 1),
             "same_call_from_position_0_us": round(ms_w * 1e3, 2)}
    return {"output_gate": gate, "continuation": contd}


def bench_wide_window(G, torch, windows=(256, 1024), reps=10):
    """hybrid_layer_fwd at the 32K layer shape with windows wider than one chunk
    (the gated part in the chunked kernels, then the window part with an online
    softmax over 64-key chunks, added to o), median of ``reps`` calls."""
    from gated_linear_attention_hybrid_amd.inputs import WORKLOADS, make_prefill
    dev = torch.device("cuda")
    wl = WORKLOADS["prefill_32k"]
    x = make_prefill(wl, dev)
    o = torch.empty((wl.B, wl.H, wl.L, wl.dv), dtype=wl.torch_dtype, device=dev)
    stream = torch.cuda.current_stream()
    out = []
    for w in windows:
        desc = G.make_desc(wl.B, wl.H, wl.L, wl.d, wl.dv, wl.f, window=w, n_meta=wl.n_meta, dtype=G.GLAH_BF16)
        ws = torch.empty(max(1, G.workspace_bytes(desc)), dtype=torch.uint8, device=dev)

        def call():
            G.hybrid_layer_fwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"], window=w, o=o,
                               ws=ws, stream=stream)

        for _ in range(3):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
        out.append({"window": w, "us_per_call": round(ms * 1e3, 1), "tokens_per_s": round(wl.L / (ms * 1e-3), 1),
                    "nonfinite_outputs": int((~torch.isfinite(o.float())).sum().item())})
        del ws
    del x, o
    return {"workload": "prefill_32k layer with a window wider than one chunk, B=1 H=32 L=32768", "calls": out}


def measured_ceilings(torch):
    """What this GPU reaches on plain library work: a 1 GiB device copy (HBM) and
    a large bf16 GEMM (hipBLASLt through torch), best of 3 each."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    a = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best_copy = best_gemm = float("inf")
    for _ in range(4):
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best_copy = min(best_copy, e0.elapsed_time(e1))
        e0.record()
        torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        best_gemm = min(best_gemm, e0.elapsed_time(e1))
    del src, dst, a, b
    return {"copy_GBps": round(2 * 4 * n / (best_copy * 1e-3) / 1e9, 1),
            "bf16_gemm_TFLOPs": round(2 * 8192 ** 3 / (best_gemm * 1e-3) / 1e12, 1),
            "note": "1 GiB device copy (read + write bytes) and an 8192^3 bf16 torch.matmul, best of 4"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, torch, target_s=12.0):
    """fp64 oracle on the host cores: all heads, the first L_s tokens, with L_s
    sized from a short calibration run so the sample takes roughly target_s; then
    a short sample on one core."""
    import oracle
    from gated_linear_attention_hybrid_amd.inputs import make_prefill, to_f64
    dev = torch.device("cuda")
    x = make_prefill(wl, dev)

    def sample(Ls):
        h = {k: (to_f64(v[:, :, :Ls]) if v.dim() == 4 else to_f64(v)) for k, v in x.items()}
        t0 = time.perf_counter()
        oracle.layer_fwd(h["q"], h["k"], h["v"], h["gate"], h["wq"], h["wk"], h["meta"],
                         window=wl.window)
        return time.perf_counter() - t0

    calib = 256
    tc = sample(calib)
    Ls = int(min(wl.L, max(calib, calib * target_s / max(tc, 1e-3))))
    Ls = max(64, (Ls // 64) * 64)
    t = sample(Ls)
    threads = min(oracle.num_threads(), wl.B * wl.H)
    all_threads = oracle.num_threads()
    oracle.set_num_threads(1)  # one core: a sample of about a second
    try:
        t1c = sample(calib)
        L1 = max(64, min(wl.L, int(calib * 1.0 / max(t1c, 1e-3))) // 64 * 64)
        t1 = sample(L1)
    finally:
        oracle.set_num_threads(all_threads)
    return {"value": round(wl.B * Ls / t, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "all %d heads of the first %d of %d tokens (fp64 oracle, OpenMP over heads), %.1f s"
                      % (wl.B * wl.H, Ls, wl.L, t),
            "one_core": {"value": round(wl.B * L1 / t1, 1), "unit": "tokens/s",
                         "sample": "all heads, first %d tokens, %.1f s" % (L1, t1)},
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-delta", action="store_true")
    ap.add_argument("--no-serving", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 2K-token and batch-8 strong-decay prefill legs")
    ap.add_argument("--delta-only", action="store_true",
                    help="run only the gated delta rule leg (for profiling) and print its JSON")
    ap.add_argument("--backward-only", action="store_true",
                    help="run only the backward leg (for profiling) and print its JSON")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a reference kernel "
                         "of known traffic for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer shards by heads or by sequence segments "
              "across GPUs, but this build runs and reports a single MI355X only", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from gated_linear_attention_hybrid_amd import binding as G
    if not os.path.exists(G.LIBRARY):
        from gated_linear_attention_hybrid_amd import build_lib
        build_lib.build(verbose=False)
    from gated_linear_attention_hybrid_amd.inputs import WORKLOADS

    wl = WORKLOADS["prefill_32k"]
    torch.cuda.set_device(0)
    if args.backward_only:
        print(json.dumps({"backward": [bench_backward(G, torch, WORKLOADS["prefill_2k"]),
                                       bench_backward(G, torch, wl)]}), flush=True)
        return
    if args.delta_only:
        print(json.dumps({"gated_delta": bench_delta(G, torch), "serving": bench_serving(G, torch)}), flush=True)
        return
    # The other legs run first: the headline call is then timed at the clocks the
    # GPU settles to under sustained work (its per-call spread is reported).
    legs = {}
    if args.copy_calibration_mib > 0:
        nel = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        legs["copy_calibration_bytes"] = {"read": nel * 4, "written": nel * 4}
        del src, dst
    legs["measured_ceilings"] = measured_ceilings(torch)
    if not args.no_decode:
        legs["decode"] = bench_decode(G, torch)
        # the step does not depend on the prefix length (constant-size state)
        short = bench_decode(G, torch, prefix=4096)
        legs["decode"]["flatness"] = {"prefix_4096_us_per_step": short["us_per_step"],
                                      "prefix_32768_us_per_step": legs["decode"]["us_per_step"]}
    if not args.no_configs:
        legs["prefill_configs"] = [bench_prefill_config(G, torch, WORKLOADS["prefill_2k"], flush=True),
                                   bench_prefill_config(G, torch, WORKLOADS["strong_decay_8k"], reps=10)]
    if not args.no_backward:
        legs["backward"] = [bench_backward(G, torch, WORKLOADS["prefill_2k"]), bench_backward(G, torch, wl)]
    if not args.no_delta:
        legs["gated_delta"] = bench_delta(G, torch)
    if not args.no_serving:
        legs["serving"] = bench_serving(G, torch)
        legs["wide_window"] = bench_wide_window(G, torch)

    ms_step, calls, bad = bench_prefill(G, wl, args.steps, args.warmup, torch)
    per_call_ms = sum(calls) / len(calls)
    token_heads = wl.B * wl.H * wl.L
    nbytes = PREFILL_BYTES_PER_TOKEN_HEAD * token_heads
    nflops = PREFILL_FLOPS_PER_TOKEN_HEAD * token_heads
    achieved = nbytes / (per_call_ms * 1e-3) / 1e9
    traffic = load_traffic("hybrid_layer_fwd/prefill_32k")
    out = {
        "metric": "hybrid GLA+SWA layer prefill tokens/s @L=32K",
        "value": round(wl.B * wl.L / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k,v~N(0,1/128), gate logits~N(3,1), meta~N(0,1))",
        "config": {"workload": "prefill_32k", "B": wl.B, "H": wl.H, "L": wl.L, "d": wl.d,
                   "f": wl.f, "d_v": wl.dv, "chunk": wl.chunk, "window": wl.window,
                   "n_meta": wl.n_meta, "seed": wl.seed},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "hybrid_layer_fwd call (state pass + segment scan + fused output pass)",
                     "us_per_launch": round(per_call_ms * 1e3, 2),
                     "us_per_launch_spread": spread_us(calls),
                     "timed_after": [k for k in legs if k != "copy_calibration_bytes"],
                     "algorithmic_bytes_per_launch": nbytes,
                     "mfma_frac": round(nflops / (per_call_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "algorithmic_flops_per_token_head": PREFILL_FLOPS_PER_TOKEN_HEAD,
                     "executed_flops_per_token_head": PREFILL_EXECUTED_FLOPS_PER_TOKEN_HEAD,
                     "transpose_flops_per_token_head": PREFILL_TRANSPOSE_FLOPS_PER_TOKEN_HEAD},
        "nonfinite_outputs": bad,
    }
    out.update(legs)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
