"""fp64 CPU oracle of the output-gate epilogue.

TEST INFRASTRUCTURE ONLY: the test suite uses this module to compute expected
values.  The GPU library never imports it, and it never imports the GPU library.

The "LT2" technical summary (2605.20670, contributions) adds a gate on the
attention output to keep activations from growing across loop iterations; it
gives no formula.  The reading taken: an elementwise sigmoid gate of logits
g = W_o x (computed by the caller), o <- o * sigmoid(g).
"""
from __future__ import annotations

import numpy as np


def output_gate(o, g):
    """o * sigmoid(g) elementwise, in float64 (sigmoid written as 1 / (1 + e^-g))."""
    o = np.asarray(o, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return o / (1.0 + np.exp(-g))
