"""Pins of the row RMSNorm oracle against a worked example, closed forms,
invariants, an independent library routine and brute force.

Each pin is chosen so that a plausible slip fails it: the sum of squares not
divided by d, the square root dropped, eps added outside the root, the gain
applied twice or not at all, the weight bias ignored or subtracted, the
reduction over the wrong axis."""
import numpy as np
import pytest
import torch

from oracle import rms_norm_oracle as N


def test_worked_example():
    # x = (3, 4), g = (1, 2), eps = 0: mean square (9 + 16) / 2 = 12.5,
    # root 3.5355339..., so y = (3, 8) / sqrt(12.5)
    got = N.rms_norm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0)
    want = np.array([3.0 / np.sqrt(12.5), 8.0 / np.sqrt(12.5)])
    np.testing.assert_allclose(got, want, rtol=1e-15)
    np.testing.assert_allclose(got, [0.848528137423857, 2.262741699796952], rtol=1e-14)


@pytest.mark.parametrize("d", [1, 7, 2048, 7168])
@pytest.mark.parametrize("c,eps", [(3.0, 0.0), (-0.5, 1e-6), (2.0, 0.25)])
def test_constant_row_closed_form(d, c, eps):
    g = np.linspace(0.5, 1.5, d)
    got = N.rms_norm(np.full((3, d), c), g, eps, weight_bias=0.25)
    want = c / np.sqrt(c * c + eps) * (g + 0.25)
    np.testing.assert_allclose(got, np.broadcast_to(want, got.shape), rtol=1e-14, atol=0)


@pytest.mark.parametrize("d", [16, 4096])
def test_one_hot_row_closed_form(d):
    a, j, eps = 5.0, 3, 1e-2
    g = np.linspace(-1.0, 1.0, d)
    x = np.zeros(d)
    x[j] = a
    want = np.zeros(d)
    want[j] = a / np.sqrt(a * a / d + eps) * g[j]
    np.testing.assert_allclose(N.rms_norm(x, g, eps), want, rtol=1e-14, atol=0)


def test_unit_gain_gives_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.normal(0, 4.0, (6, 2048))
    y = N.rms_norm(x, np.ones(2048), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(N.rms_norm(-25.0 * x, np.ones(2048), 0.0), -y, rtol=1e-13)


def test_rows_are_independent():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 1.0, (4, 64))
    g = rng.normal(1, 0.1, 64)
    y = N.rms_norm(x, g, 1e-6)
    x2 = x.copy()
    x2[2] *= 1000.0
    y2 = N.rms_norm(x2, g, 1e-6)
    np.testing.assert_array_equal(np.delete(y2, 2, axis=0), np.delete(y, 2, axis=0))


def test_weight_bias_adds_to_gain():
    rng = np.random.default_rng(2)
    x = rng.normal(0, 1.0, (3, 256))
    g = rng.normal(0.0, 0.5, 256)
    np.testing.assert_allclose(N.rms_norm(x, g, 1e-5, 1.0), N.rms_norm(x, g + 1.0, 1e-5),
                               rtol=1e-15)


@pytest.mark.parametrize("d,eps", [(2048, 1e-6), (7168, 1e-5), (96, 0.5)])
def test_matches_torch_rms_norm(d, eps):
    # torch's own RMSNorm, in float64, as an independent implementation
    rng = np.random.default_rng(d)
    x = rng.normal(0, 2.0, (5, d))
    g = rng.normal(1.0, 0.2, d)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (d,), torch.from_numpy(g), eps)
    np.testing.assert_allclose(N.rms_norm(x, g, eps), ref.numpy(), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("d", [8, 33])
def test_matches_bruteforce_loops(d):
    rng = np.random.default_rng(d + 3)
    x = rng.normal(0, 1.5, (2, 3, d))
    g = rng.normal(1, 0.3, d)
    np.testing.assert_allclose(N.rms_norm(x, g, 1e-4, 0.5), N.rms_norm_bruteforce(x, g, 1e-4, 0.5),
                               rtol=1e-13)
