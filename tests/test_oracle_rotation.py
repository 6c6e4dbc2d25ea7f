"""Pins of the oracle's rotation H = B diag(signs) against scipy's Sylvester
Hadamard matrix (a library routine) and against orthogonality."""
import numpy as np
import pytest
import scipy.linalg

import oracle as O


def _signs(d, seed):
    rng = np.random.default_rng(seed)
    return (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128])
def test_power_of_two_matches_scipy(d):
    s = _signs(d, d)
    H = O.rotation_matrix(d, s)
    ref = scipy.linalg.hadamard(d).astype(np.float64) / np.sqrt(d) * s[None, :]
    assert np.allclose(H, ref, atol=1e-15, rtol=0)


@pytest.mark.parametrize("d", [2, 16, 64, 96, 128])
def test_orthogonal(d):
    H = O.rotation_matrix(d, _signs(d, 7 + d))
    assert np.abs(H @ H.T - np.eye(d)).max() < 1e-12
    assert np.abs(H.T @ H - np.eye(d)).max() < 1e-12


def test_d96_is_block_diagonal_64_then_32():
    s = _signs(96, 5)
    H = O.rotation_matrix(96, s)
    B = scipy.linalg.block_diag(scipy.linalg.hadamard(64) / 8.0,
                                scipy.linalg.hadamard(32) / np.sqrt(32.0))
    assert np.allclose(H, B * s[None, :], atol=1e-15, rtol=0)
    assert np.all(H[:64, 64:] == 0) and np.all(H[64:, :64] == 0)


def test_d2_closed_form():
    s = np.array([1, -1], np.int8)
    H = O.rotation_matrix(2, s)
    r = 1 / np.sqrt(2)
    assert np.allclose(H, [[r, -r], [r, r]], atol=1e-16, rtol=0)


def test_columns_are_signed_hadamard_columns():
    d = 32
    s = _signs(d, 3)
    H = O.rotation_matrix(d, s)
    W = scipy.linalg.hadamard(d)
    for j in range(d):
        e = np.zeros(d)
        e[j] = 1
        assert np.allclose(H @ e, s[j] * W[:, j] / np.sqrt(d), atol=1e-15, rtol=0)


@pytest.mark.parametrize("d", [2, 16, 64, 96, 128])
def test_rotate_applies_H_and_its_transpose(d):
    s = _signs(d, 40 + d)
    H = O.rotation_matrix(d, s)
    rng = np.random.default_rng(d)
    for _ in range(5):
        r = rng.standard_normal(d)
        assert np.allclose(O.rotate(d, s, r), H @ r, rtol=0, atol=1e-14)
        assert np.allclose(O.rotate_t(d, s, r), H.T @ r, rtol=0, atol=1e-14)
        assert np.allclose(O.rotate_t(d, s, O.rotate(d, s, r)), r, rtol=0, atol=1e-14)


def test_rotate_keeps_exact_cancellation_exact():
    """Signed inputs whose Walsh-Hadamard sum cancels give an exact zero (the
    +-1 sums are exact for short dyadic inputs; only the final scale rounds)."""
    d = 128
    s = np.ones(d, np.int8)
    r = np.zeros(d)
    r[0], r[1] = 0.375, -0.375          # row i of S sums to r0 + (-1)^{i&1} r1
    y = O.rotate(d, s, r)
    assert np.all(y[0::2] == 0.0)
    assert np.all(np.abs(y[1::2]) == np.float64(0.75) * (1 / np.sqrt(128.0)))
