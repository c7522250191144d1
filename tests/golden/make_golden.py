"""Writes tests/golden/tiny_hybrid.json: a regression fixture of the fp64 oracle.

The pages print no worked numeric example of the layer, so this fixture is not a
page value: it records the oracle's own output on a tiny fixed input so that any
later change to the oracle's arithmetic shows up.  It calls only ``oracle/``.
Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def fixed_inputs():
    # small rational-valued inputs built from index arithmetic (no RNG)
    B, H, L, d, f, dv, M = 1, 2, 6, 4, 6, 3, 2
    i = np.arange(B * H * L * d, dtype=np.float64).reshape(B, H, L, d)
    q = np.sin(0.7 * i + 0.1)
    k = np.cos(0.3 * i - 0.2)
    v = np.sin(0.11 * np.arange(B * H * L * dv, dtype=np.float64).reshape(B, H, L, dv) + 1.0)
    g = 1.5 * np.cos(0.5 * np.arange(B * H * L * f, dtype=np.float64).reshape(B, H, L, f))
    wq = 0.5 * np.sin(np.arange(H * d * (f // 2), dtype=np.float64).reshape(H, d, f // 2))
    wk = 0.5 * np.cos(np.arange(H * d * (f // 2), dtype=np.float64).reshape(H, d, f // 2))
    meta = np.array([[0.25, -1.0], [1.5, 0.0]])
    return dict(q=q, k=k, v=v, g=g, wq=wq, wk=wk, meta=meta, window=3, scale=0.5)


def main():
    c = fixed_inputs()
    o, st = oracle.layer_fwd(c["q"], c["k"], c["v"], c["g"], c["wq"], c["wk"], c["meta"],
                             window=c["window"], scale=c["scale"], return_state=True)
    out = {
        "what": "fp64 oracle regression fixture (not a page value; the pages print none)",
        "window": c["window"], "scale": c["scale"],
        "o": o.tolist(), "state": st.tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_hybrid.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
