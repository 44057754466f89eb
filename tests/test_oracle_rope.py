"""Pins of the oracle's partial RoPE and inverse RoPE.

The pages fix which channels rotate (the last 64, [cdjax] §1.1) and that the
core-attention output is rotated by the negative query position. The pair
layout and base are readings; these tests pin the oracle to the rotation it
claims (complex-exponential form) and to the relative-position property the
inverse rotation exists for.
"""

import numpy as np

import oracle as O


def test_matches_complex_exponential_form():
    rng = np.random.default_rng(0)
    D, R, base = 16, 8, 10000.0
    x = rng.standard_normal(D)
    pos = 37
    y = O.rope_rotate(x, pos, base, R)
    np.testing.assert_array_equal(y[:D - R], x[:D - R])
    z = x[D - R::2] + 1j * x[D - R + 1::2]
    freqs = base ** (-np.arange(0, R, 2) / R)
    zr = z * np.exp(1j * pos * freqs)
    np.testing.assert_allclose(y[D - R::2], zr.real, atol=1e-13)
    np.testing.assert_allclose(y[D - R + 1::2], zr.imag, atol=1e-13)


def test_inverse_and_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 32))
    y = O.rope_rotate(x, 1048576, 10000.0, 16)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    np.testing.assert_allclose(O.rope_rotate(y, -1048576, 10000.0, 16), x, atol=1e-12)


def test_relative_position_of_dot_products():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(24), rng.standard_normal(24)
    d1 = O.rope_rotate(q, 100, 10000.0, 16) @ O.rope_rotate(k, 40, 10000.0, 16)
    d2 = O.rope_rotate(q, 1060, 10000.0, 16) @ O.rope_rotate(k, 1000, 10000.0, 16)
    d3 = O.rope_rotate(q, 60, 10000.0, 16) @ k
    assert abs(d1 - d2) < 1e-12 and abs(d1 - d3) < 1e-12


def test_first_pair_rotates_at_unit_frequency():
    x = np.zeros(8)
    x[4] = 1.0
    y = O.rope_rotate(x, 0.5, 10000.0, 4)
    assert abs(y[4] - np.cos(0.5)) < 1e-15 and abs(y[5] - np.sin(0.5)) < 1e-15
