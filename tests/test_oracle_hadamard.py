"""Pins for the oracle's Walsh-Hadamard rotation."""
import numpy as np
import pytest
import scipy.linalg

from oracle.hadamard import fwht, inverse_rotate, rotate, rotate_unnormalised, sylvester
from synth import sign_vector


def test_sylvester_matches_scipy():
    np.testing.assert_array_equal(sylvester(128), scipy.linalg.hadamard(128))


def test_sylvester_closed_form_entries():
    h = sylvester(128)
    i, j = np.meshgrid(np.arange(128), np.arange(128), indexing="ij")
    pop = np.vectorize(lambda v: bin(v).count("1"))(i & j)
    np.testing.assert_array_equal(h, (-1) ** pop)


def test_hadamard_orthogonality_exact():
    h = sylvester(128)
    np.testing.assert_array_equal(h @ h, 128 * np.eye(128, dtype=np.int64))
    np.testing.assert_array_equal(h, h.T)


def test_butterfly_equals_dense_on_integers():
    rng = np.random.default_rng(0)
    x = rng.integers(-1000, 1000, size=(17, 128))
    np.testing.assert_array_equal(fwht(x), x @ sylvester(128))


def test_first_column_is_flat():
    e0 = np.zeros(128)
    e0[0] = 1.0
    np.testing.assert_allclose(rotate(e0, np.ones(128)), np.full(128, 1 / np.sqrt(128)), rtol=0, atol=1e-16)


def test_signs_are_applied_before_h():
    s = sign_vector(0, "k")
    h = sylvester(128)
    for j in (0, 5, 127):
        e = np.zeros(128)
        e[j] = 1.0
        np.testing.assert_allclose(rotate(e, s), s[j] * h[:, j] / np.sqrt(128), atol=1e-16, rtol=0)
        np.testing.assert_allclose(inverse_rotate(e, s), s * h[:, j] / np.sqrt(128), atol=1e-16, rtol=0)


def test_round_trip_and_parseval():
    rng = np.random.default_rng(1)
    s = sign_vector(3, "v")
    x = rng.standard_normal((50, 128))
    y = rotate(x, s)
    np.testing.assert_allclose(inverse_rotate(y, s), x, atol=1e-14, rtol=0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-15)


def test_unnormalised_rotation_is_exact_for_fp16():
    """H (s * x) of fp16 inputs equals the exact integer transform scaled by 2**-24."""
    rng = np.random.default_rng(2)
    x = np.clip(rng.standard_t(3, size=(40, 128)) * 50, -65504, 65504).astype(np.float16)
    x[0, :] = np.float16(65504.0)
    x[1, :] = np.float16(2.0 ** -24)
    s = sign_vector(1, "k")
    m = (x.astype(np.float64) * 2.0 ** 24).astype(np.int64) * s.astype(np.int64)
    exact = fwht(m)
    np.testing.assert_array_equal(rotate_unnormalised(x, s) * 2.0 ** 24, exact.astype(np.float64))
    assert np.all(np.abs(exact) < 2 ** 53)


def test_sign_vectors_are_rademacher_and_distinct():
    for seed in range(4):
        sk, sv = sign_vector(seed, "k"), sign_vector(seed, "v")
        assert set(np.unique(sk)) <= {-1.0, 1.0} and set(np.unique(sv)) <= {-1.0, 1.0}
        assert not np.array_equal(sk, sv)
    np.testing.assert_array_equal(sign_vector(0, "k"), sign_vector(0, "k"))
