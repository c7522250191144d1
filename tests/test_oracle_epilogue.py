"""Pins of the output-gate oracle (oracle/epilogue.py): a library sigmoid,
the symmetry sigmoid(g) + sigmoid(-g) = 1, g = 0 halving, and the saturated
limits."""
import numpy as np
import scipy.special
import torch

from oracle import epilogue


def test_matches_library_sigmoid():
    rng = np.random.default_rng(0)
    o, g = rng.normal(size=(2, 3, 7, 5)), rng.normal(0, 4, size=(2, 3, 7, 5))
    np.testing.assert_allclose(epilogue.output_gate(o, g), o * scipy.special.expit(g), rtol=1e-14, atol=0)
    t = torch.sigmoid(torch.as_tensor(g)).numpy()
    np.testing.assert_allclose(epilogue.output_gate(o, g), o * t, rtol=1e-14, atol=0)


def test_symmetry_and_limits():
    rng = np.random.default_rng(1)
    o, g = rng.normal(size=100), rng.normal(0, 3, size=100)
    np.testing.assert_allclose(epilogue.output_gate(o, g) + epilogue.output_gate(o, -g), o, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(epilogue.output_gate(o, np.zeros_like(g)), o / 2)
    np.testing.assert_allclose(epilogue.output_gate(o, np.full_like(g, 50.0)), o, rtol=1e-15)
    assert np.all(np.abs(epilogue.output_gate(o, np.full_like(g, -800.0))) == 0.0)
