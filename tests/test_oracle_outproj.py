"""Pins of the oracle's grouped output projection: each check computes the
same quantity by a different route than the oracle (plain products, an
explicit block-diagonal matrix, scalar loops) or states a symmetry it must
have."""

import numpy as np
import pytest

import oracle as O


def _case(rng, T, n_h, c, g, d_g, d_model):
    o = rng.standard_normal((T, n_h, c))
    w_g = rng.standard_normal((g, d_g, (n_h // g) * c)) / np.sqrt((n_h // g) * c)
    w_o = rng.standard_normal((d_model, g * d_g)) / np.sqrt(g * d_g)
    return o, w_g, w_o


def test_one_group_is_the_plain_product():
    rng = np.random.default_rng(1)
    o, w_g, w_o = _case(rng, 5, 4, 6, 1, 7, 9)
    ref = (o.reshape(5, 24) @ w_g[0].T) @ w_o.T
    np.testing.assert_allclose(O.grouped_output_projection(o, w_g, w_o, round_mid=False), ref, rtol=1e-12)


@pytest.mark.parametrize("g", [2, 4, 8])
def test_grouped_equals_block_diagonal_product(g):
    rng = np.random.default_rng(2 + g)
    T, n_h, c, d_g, d_model = 3, 8, 5, 6, 11
    o, w_g, w_o = _case(rng, T, n_h, c, g, d_g, d_model)
    kg = (n_h // g) * c
    bd = np.zeros((n_h * c, g * d_g))
    for gi in range(g):
        bd[gi * kg:(gi + 1) * kg, gi * d_g:(gi + 1) * d_g] = w_g[gi].T
    ref = o.reshape(T, n_h * c) @ bd @ w_o.T
    np.testing.assert_allclose(O.grouped_output_projection(o, w_g, w_o, round_mid=False), ref, rtol=1e-12,
                               atol=1e-12)


def test_heads_permuted_inside_a_group_change_nothing():
    rng = np.random.default_rng(9)
    T, n_h, c, g, d_g, d_model = 4, 8, 3, 2, 5, 7
    o, w_g, w_o = _case(rng, T, n_h, c, g, d_g, d_model)
    perm = np.array([2, 0, 3, 1])                   # heads of group 0, reordered
    o2 = o.copy()
    o2[:, :4] = o[:, perm]
    w2 = w_g.copy()
    cols = w_g[0].reshape(d_g, 4, c)
    w2[0] = cols[:, perm].reshape(d_g, 4 * c)
    np.testing.assert_allclose(O.grouped_output_projection(o2, w2, w_o, round_mid=False),
                               O.grouped_output_projection(o, w_g, w_o, round_mid=False), rtol=1e-12)


def test_scalar_loops_tiny():
    rng = np.random.default_rng(10)
    T, n_h, c, g, d_g, d_model = 2, 4, 2, 2, 3, 2
    o, w_g, w_o = _case(rng, T, n_h, c, g, d_g, d_model)
    got = O.grouped_output_projection(o, w_g, w_o, round_mid=False)
    for t in range(T):
        mid = []
        for gi in range(g):
            for j in range(d_g):
                acc = 0.0
                for hh in range(n_h // g):
                    for ch in range(c):
                        acc += o[t, gi * (n_h // g) + hh, ch] * w_g[gi, j, hh * c + ch]
                mid.append(acc)
        for n in range(d_model):
            ref = sum(mid[i] * w_o[n, i] for i in range(g * d_g))
            assert abs(got[t, n] - ref) < 1e-12


def test_rounded_intermediate_is_bf16_exact():
    rng = np.random.default_rng(11)
    o, w_g, w_o = _case(rng, 3, 8, 4, 4, 6, 5)
    full = O.grouped_output_projection(o, w_g, w_o, round_mid=False)
    rnd = O.grouped_output_projection(o, w_g, w_o, round_mid=True)
    # bf16 rounding of the intermediate: relative change within 2^-8 of the row scale
    assert np.max(np.abs(full - rnd)) <= 2 ** -8 * np.max(np.abs(full)) * 4
    assert not np.allclose(full, rnd, rtol=0, atol=0)
