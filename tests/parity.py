"""Helpers of the GPU parity tests: error metric and oracle plumbing."""
import numpy as np
import torch

from gated_linear_attention_hybrid_amd.inputs import to_f64

# max row-normwise relative error allowed: bf16 inputs / fp32 accumulation, and
# the fp32 mode
TOL_BF16 = 2e-2
TOL_F32 = 1e-4


def row_rel_err(out, ref, floor_frac=1e-6):
    """max over rows (all leading axes) of ||out - ref||_inf / ||ref||_inf.

    A row whose reference norm is below ``floor_frac`` of the largest row norm is
    measured against that floor instead (such rows carry no signal at this
    precision)."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    if out.size == 0:
        return 0.0
    err = np.max(np.abs(out - ref), axis=-1)
    nrm = np.max(np.abs(ref), axis=-1)
    den = np.maximum(nrm, max(float(np.max(nrm)) * floor_frac, 1e-30))
    return float(np.max(err / den))


def gpu_f64(t: torch.Tensor):
    torch.cuda.synchronize()
    return to_f64(t)


def oracle_inputs(x: dict):
    """Widen the (bf16 or fp32) device inputs exactly to float64 numpy arrays."""
    return {k: to_f64(v) for k, v in x.items()}


def assert_finite(t: torch.Tensor, what: str):
    bad = (~torch.isfinite(t.float())).sum().item()
    assert bad == 0, "%s has %d non-finite values" % (what, bad)


def seeded_randn(shape, seed, device="cuda"):
    """Standard normal draws from their own seeded CPU generator, on ``device``
    (test inputs never come from the process-global RNG, whose state depends on
    which tests ran before)."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    return torch.randn(shape, generator=gen).to(device)
