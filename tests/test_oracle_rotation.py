"""Pins for the oracle's rotation R = (1/sqrt 32) H32 D and its sign source (CPU only)."""

import math

import numpy as np

from oracle import tq4_1s as tq


def _popcount(v):
    return bin(v).count("1")


def test_splitmix64_published_vector():
    # First outputs of splitmix64 seeded with 0 (Vigna's reference implementation).
    assert tq.splitmix64(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert tq.DEFAULT_SIGN_MASK == 0x7B1DCDAF


def test_sign_vector_bit_order():
    d = tq.sign_vector(0b101)
    assert d[0] == -1 and d[1] == 1 and d[2] == -1 and np.all(d[3:] == 1)
    assert np.all(tq.sign_vector(0xFFFFFFFF) == -1)


def test_hadamard_definition():
    h = tq.hadamard(32)
    ref = np.array([[(-1) ** _popcount(i & j) for j in range(32)] for i in range(32)], dtype=float)
    np.testing.assert_array_equal(h, ref)
    np.testing.assert_array_equal(h @ h, 32 * np.eye(32))
    np.testing.assert_array_equal(h, h.T)


def test_rotation_is_orthogonal_and_inverts():
    rng = np.random.default_rng(0)
    for mask in (0, tq.DEFAULT_SIGN_MASK, 0xFFFFFFFF, 0x80000001):
        r = tq.rotate_f64(np.eye(32), mask)           # row j = R e_j
        np.testing.assert_allclose(r @ r.T, np.eye(32), atol=1e-15)
        w = rng.normal(size=(7, 32))
        back = tq.inverse_rotate_f64(tq.rotate_f64(w, mask), mask)
        np.testing.assert_allclose(back, w, rtol=0, atol=1e-15 * np.abs(w).max() * 32)


def test_spike_closed_forms_fix_where_d_sits():
    """R e_j = D_j H[:, j]/sqrt32 while R^-1 e_j = D * H[:, j]/sqrt32 (D applied elementwise)."""
    mask = tq.DEFAULT_SIGN_MASK
    h = tq.hadamard()
    d = tq.sign_vector(mask)
    for j in (0, 5, 31):
        e = np.zeros(32)
        e[j] = 1.0
        np.testing.assert_allclose(tq.rotate_f64(e, mask), d[j] * h[:, j] / math.sqrt(32), atol=1e-16)
        np.testing.assert_allclose(tq.inverse_rotate_f64(e, mask), d * h[:, j] / math.sqrt(32), atol=1e-16)


def test_dot_product_identity():
    """w . x = (R w) . (R x): the rotation can move from the weights to the activation."""
    rng = np.random.default_rng(1)
    w = rng.normal(size=(50, 32))
    x = rng.normal(size=(50, 32))
    lhs = np.sum(w * x, axis=1)
    rhs = np.sum(tq.rotate_f64(w, tq.DEFAULT_SIGN_MASK) * tq.rotate_f64(x, tq.DEFAULT_SIGN_MASK), axis=1)
    np.testing.assert_allclose(rhs, lhs, rtol=1e-12, atol=1e-12)


def test_fwht_f32_against_matrix():
    rng = np.random.default_rng(2)
    v = rng.normal(size=(100, 32)).astype(np.float32)
    got = tq.fwht32_f32(v).astype(np.float64)
    ref = v.astype(np.float64) @ tq.hadamard().T
    bound = 5 * np.finfo(np.float32).eps * np.abs(v).sum(axis=1, keepdims=True)
    assert np.all(np.abs(got - ref) <= bound)
    # small integers are exact at every stage
    iv = rng.integers(-100, 100, size=(20, 32)).astype(np.float32)
    np.testing.assert_array_equal(tq.fwht32_f32(iv).astype(np.float64), iv.astype(np.float64) @ tq.hadamard().T)


def test_rotate_f32_close_to_f64():
    rng = np.random.default_rng(3)
    w = rng.normal(size=(64, 32)).astype(np.float32)
    got = tq.rotate_f32(w, tq.DEFAULT_SIGN_MASK).astype(np.float64)
    ref = tq.rotate_f64(w.astype(np.float64), tq.DEFAULT_SIGN_MASK)
    assert np.max(np.abs(got - ref)) < 1e-5 * np.abs(w).max() * 4
