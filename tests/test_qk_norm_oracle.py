"""Pins of the QK-norm oracle against closed forms, invariants and brute force.

Each pin is chosen so that a plausible slip in the oracle fails it: the sum of
squares used without dividing by head_dim, the reciprocal square root dropped
(as in the section's one-line formula), eps added outside the root, the weight
bias ignored or subtracted, a wrong reduction axis."""
import numpy as np
import pytest

from oracle import qk_norm_oracle as Q


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("c,eps", [(3.0, 0.0), (0.5, 1e-6), (-2.0, 0.25)])
def test_constant_head_closed_form(hd, c, eps):
    # x = c * 1: mean of squares is c^2, so r_i = (w_i + b) * c / sqrt(c^2 + eps)
    rng = np.random.default_rng(hd)
    w = rng.normal(1.0, 0.1, hd)
    b = 0.5
    x = np.full((2, 3, hd), c)
    got = Q.qk_norm(x, w, b, eps)
    want = (w + b) * c / np.sqrt(c * c + eps)
    np.testing.assert_allclose(got, np.broadcast_to(want, got.shape), rtol=1e-15, atol=0)


@pytest.mark.parametrize("hd", [64, 256])
def test_one_hot_head_closed_form(hd):
    a, j, eps = 7.0, 5, 1e-3
    w = np.linspace(0.5, 1.5, hd)
    x = np.zeros(hd)
    x[j] = a
    got = Q.qk_norm(x, w, 0.0, eps)
    want = np.zeros(hd)
    want[j] = w[j] * a / np.sqrt(a * a / hd + eps)
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=0)


def test_unit_weight_gives_unit_rms():
    # w = 1, bias 0, eps 0: every normalised head has root-mean-square 1
    rng = np.random.default_rng(1)
    x = rng.normal(0, 3.0, (5, 4, 128))
    y = Q.qk_norm(x, np.ones(128), 0.0, 0.0)
    rms = np.sqrt(np.mean(y * y, axis=-1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-14)


def test_scale_invariance_and_odd_symmetry():
    rng = np.random.default_rng(2)
    x = rng.normal(0, 1.0, (3, 2, 64))
    w = rng.normal(1.0, 0.2, 64)
    y = Q.qk_norm(x, w, 0.0, 0.0)
    np.testing.assert_allclose(Q.qk_norm(37.0 * x, w, 0.0, 0.0), y, rtol=1e-14)
    np.testing.assert_allclose(Q.qk_norm(-x, w, 0.0, 0.0), -y, rtol=0, atol=0)
    # with eps > 0 a tiny head is damped, a huge one is not
    small = Q.qk_norm(1e-6 * x, w, 0.0, 1.0)
    assert np.max(np.abs(small)) < 1e-5
    np.testing.assert_allclose(Q.qk_norm(1e6 * x, w, 0.0, 1.0), y, rtol=1e-9)


def test_weight_bias_adds_to_weight():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 1.0, (4, 128))
    w = rng.normal(0.0, 0.3, 128)
    np.testing.assert_allclose(Q.qk_norm(x, w, 1.0, 1e-6), Q.qk_norm(x, w + 1.0, 0.0, 1e-6),
                               rtol=1e-15)


def test_each_head_normalised_on_its_own():
    # heads are independent: changing one head leaves the others untouched
    rng = np.random.default_rng(4)
    x = rng.normal(0, 1.0, (2, 3, 64))
    w = np.ones(64)
    y = Q.qk_norm(x, w, 0.0, 1e-6)
    x2 = x.copy()
    x2[1, 2] *= 100.0
    y2 = Q.qk_norm(x2, w, 0.0, 1e-6)
    mask = np.ones((2, 3), dtype=bool)
    mask[1, 2] = False
    np.testing.assert_array_equal(y2[mask], y[mask])


@pytest.mark.parametrize("hd", [64, 128])
def test_matches_bruteforce_loops(hd):
    rng = np.random.default_rng(hd + 9)
    x = rng.normal(0, 2.0, (3, 2, hd))
    w = rng.normal(1.0, 0.1, hd)
    np.testing.assert_allclose(Q.qk_norm(x, w, 0.25, 1e-5), Q.qk_norm_bruteforce(x, w, 0.25, 1e-5),
                               rtol=1e-13)


def test_pair_uses_each_tensors_own_weight():
    rng = np.random.default_rng(5)
    q = rng.normal(0, 1, (2, 4, 64))
    k = rng.normal(0, 1, (2, 1, 64))
    wq = rng.normal(1, 0.1, 64)
    wk = rng.normal(2, 0.1, 64)
    rq, rk = Q.qk_norm_pair(q, k, wq, wk, 0.0, 1e-6)
    np.testing.assert_array_equal(rq, Q.qk_norm(q, wq, 0.0, 1e-6))
    np.testing.assert_array_equal(rk, Q.qk_norm(k, wk, 0.0, 1e-6))
