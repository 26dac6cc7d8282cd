"""Pins of oracle/transforms.py against scipy's Hadamard matrix and the rotation identities."""
import numpy as np
import scipy.linalg

from oracle import transforms as T


def test_fwht_equals_hadamard_exactly_on_integers():
    rng = np.random.default_rng(7)
    for n in (16, 128, 512):
        u = rng.integers(-1000, 1000, (50, n)).astype(np.float32)
        H = scipy.linalg.hadamard(n).astype(np.float64)
        assert np.array_equal(T.fwht_f32(u).astype(np.float64), u.astype(np.float64) @ H)


def test_fwht_error_bound_random():
    rng = np.random.default_rng(8)
    for n in (128, 512):
        u = rng.standard_normal((200, n)).astype(np.float32) * 10
        H = scipy.linalg.hadamard(n).astype(np.float64)
        ref = u.astype(np.float64) @ H
        got = T.fwht_f32(u).astype(np.float64)
        bound = np.log2(n) * 2.0 ** -24 * np.sum(np.abs(u), -1, keepdims=True) * 1.01
        assert np.all(np.abs(got - ref) <= bound)


def test_fwht_involution():
    rng = np.random.default_rng(9)
    u = rng.integers(-50, 50, (10, 128)).astype(np.float32)
    assert np.array_equal(T.fwht_f32(T.fwht_f32(u)), 128 * u)


def test_smoothing_rotation_preserve_logits():
    rng = np.random.default_rng(10)
    d = 128
    q = rng.standard_normal((4, d))
    k = rng.standard_normal((64, d))
    lam = np.exp2(rng.integers(-3, 4, d)).astype(np.float64)
    H = scipy.linalg.hadamard(d).astype(np.float64)
    lhs = ((q * lam) @ H) @ ((k / lam) @ H).T / d
    assert np.allclose(lhs, q @ k.T, rtol=1e-12, atol=1e-12)
    # the float32 helpers compute the same transform as the matrix form
    x = T.rotate_keys(k.astype(np.float32), (1 / lam).astype(np.float32))
    assert np.allclose(x, (k.astype(np.float32) / lam) @ H, rtol=1e-5, atol=1e-4)
