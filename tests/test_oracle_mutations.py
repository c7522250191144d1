"""Mutation check of the oracle pins.

Each case plants one plausible mistake in a copy of the oracle source (on the CPU,
in a temporary directory; the n-th occurrence of an anchor when it repeats, the
first by default), builds it, and runs every pin of ``test_oracle.py``
against it: at least one pin must fail, or the pins would not protect the oracle
from that mistake.  The committed oracle is never modified.  Every planted
mistake keeps all memory accesses in bounds (the pins run in this process).
"""
import inspect
import os

import pytest

import oracle
import test_oracle as pins

MUTATIONS = {
    "decay after the outer product": (
        "S[(size_t)r * dv + c] = gam * S[(size_t)r * dv + c] + phk[r] * vt[c];",
        "S[(size_t)r * dv + c] = gam * (S[(size_t)r * dv + c] + phk[r] * vt[c]);"),
    "negative Hedgehog half uses +u": (
        "phi[f2 + j] = exp(-u[j] + mn);", "phi[f2 + j] = exp(u[j] - mx);"),
    "Hedgehog projection transposed": (
        "acc += x[i] * W[(size_t)i * f2 + j];", "acc += x[i] * W[(size_t)j * d + i];"),
    "decode: decay after the outer product": (
        "S[(size_t)r * dv + c] = gam * S[(size_t)r * dv + c] + phk[r] * vt[c];",
        "S[(size_t)r * dv + c] = gam * (S[(size_t)r * dv + c] + phk[r] * vt[c]);", 1),
    "Hedgehog halves not normalised": ("phi[j] /= zp;", "phi[j] /= 1.0;"),
    "sigmoid sign flipped": ("return 1.0 / (1.0 + exp(-g));", "return 1.0 / (1.0 + exp(g));"),
    "window one key too narrow": ("const int j0 = t - window + 1 > 0 ? t - window + 1 : 0;",
                                  "const int j0 = t - window + 2 > 0 ? t - window + 2 : 0;"),
    "window excludes the query token": ("for (int j = j0; j <= t; ++j, ++n) {",
                                        "for (int j = j0; j < t; ++j, ++n) {"),
    "sink logit added without exp": ("den += exp(meta[mm] - m);", "den += meta[mm];"),
    "sinks dropped": ("for (int mm = 0; mm < n_meta; ++mm) den += exp(meta[mm] - m);", ""),
    "score scale ignored": ("s[j] = scale * acc;", "s[j] = acc;"),
    "readout with phi(k)": ("for (int r = 0; r < f; ++r) acc += phq[r] * S[(size_t)r * dv + c];",
                            "for (int r = 0; r < f; ++r) acc += phk[r] * S[(size_t)r * dv + c];"),
    "decode: readout with phi(k)": (
        "for (int r = 0; r < f; ++r) acc += phq[r] * S[(size_t)r * dv + c];",
        "for (int r = 0; r < f; ++r) acc += phk[r] * S[(size_t)r * dv + c];", 1),
    "state_in ignored": ("if (state_in) memcpy(", "if (0) memcpy("),
    "decode ring slot shifted": ("const int slot = (int)(p % window);",
                                 "const int slot = (int)((p + 1) % window);"),
    "decode window one key too narrow": (
        "const long long j0 = p - window + 1 > 0 ? p - window + 1 : 0;",
        "const long long j0 = p - window + 2 > 0 ? p - window + 2 : 0;"),
    "decode gate read as log-gate": ("const double gam = gate_value(gt[r], gate_is_log);",
                                     "const double gam = gate_value(gt[r], !gate_is_log);"),
}


def _pin_calls():
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        # the golden fixture is the oracle's own output: it would catch every
        # mutation trivially, so only the independent pins count here
        if not name.startswith("test_") or name == "test_golden_regression_fixture":
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            calls.append((name, fn, {}))
            continue
        argnames, values = params[0].args[0], params[0].args[1]
        argnames = [a.strip() for a in argnames.split(",")]
        for val in values:
            val = val if isinstance(val, tuple) else (val,)
            calls.append(("%s%s" % (name, val), fn, dict(zip(argnames, val))))
    return calls


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, tmp_path, monkeypatch):
    old, new, *nth = MUTATIONS[mutation]
    nth = nth[0] if nth else 0
    src = open(oracle.oracle.SOURCE).read()
    assert src.count(old) > nth, "mutation anchor not found: " + old
    at = -1
    for _ in range(nth + 1):
        at = src.index(old, at + 1)
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as fh:
        fh.write(src[:at] + new + src[at + len(old):])
    lib = oracle.compile_source(path, os.path.join(tmp_path, "libmutant.so"))
    variant = oracle.Oracle(lib)
    monkeypatch.setattr(oracle, "layer_fwd", variant.layer_fwd)
    monkeypatch.setattr(oracle, "decode_step", variant.decode_step)
    caught = []
    for name, fn, kw in _pin_calls():
        try:
            fn(**kw)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(name)
    assert caught, "no pin detects: " + mutation
