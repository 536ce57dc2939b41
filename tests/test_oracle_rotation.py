"""Pins for the oracle's normalized Walsh-Hadamard transform.

The rotation is applied to q and k so that q.k is preserved ("Read What Matters",
Dual-QK abstract: the same orthogonal transform on queries preserves query-key
dot products; "The Asymmetric Key-Value Cache Compression Framework", Method).
"""
import math

import numpy as np
import pytest
import scipy.linalg

from oracle import wht128_fp32


def test_matches_library_hadamard():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    ref = x.astype(np.float64) @ scipy.linalg.hadamard(128).astype(np.float64).T / math.sqrt(128)
    got = wht128_fp32(x).astype(np.float64)
    assert np.allclose(got, ref, rtol=0, atol=2e-6 * np.abs(x).sum(axis=1, keepdims=True).max())


@pytest.mark.parametrize("j", [0, 1, 5, 64, 127])
def test_basis_vectors_give_sylvester_columns(j):
    # Closed form of the natural-order (Sylvester) Hadamard matrix:
    # H[i, j] = (-1)^popcount(i & j).
    e = np.zeros(128, dtype=np.float32)
    e[j] = 1.0
    got = wht128_fp32(e)
    signs = np.array([(-1) ** bin(i & j).count("1") for i in range(128)], dtype=np.float64)
    expect = (signs * np.float32(1.0 / math.sqrt(128.0))).astype(np.float32)
    assert np.array_equal(got, expect)


def test_e0_is_flat():
    e = np.zeros(128, dtype=np.float32)
    e[0] = 1.0
    assert np.all(wht128_fp32(e) == np.float32(1.0 / math.sqrt(128.0)))


def test_involution_and_norm():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    y = wht128_fp32(x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)
    assert np.allclose(wht128_fp32(y), x, atol=1e-5)


def test_dot_products_preserved():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 128)).astype(np.float32)
    k = rng.standard_normal((64, 128)).astype(np.float32) * 10
    a = q.astype(np.float64) @ k.astype(np.float64).T
    b = wht128_fp32(q).astype(np.float64) @ wht128_fp32(k).astype(np.float64).T
    assert np.allclose(a, b, atol=1e-3)


def test_rejects_other_lengths():
    with pytest.raises(ValueError):
        wht128_fp32(np.zeros(64, dtype=np.float32))
