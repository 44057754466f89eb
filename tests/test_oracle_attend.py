"""Pins of the oracle's core attention (selected entries + window + sink)."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O


def test_sink_matches_sdpa_with_extra_column():
    # A sink logit with no value equals one more key whose logit is exactly the
    # sink and whose value row is zero: torch float64 SDPA with an additive mask.
    rng = np.random.default_rng(0)
    n, D = 37, 16
    X = rng.standard_normal((n, D))
    q = rng.standard_normal(D) * 3
    sink = 0.8
    scale = 1 / math.sqrt(D)
    o, lse, _ = O.sink_attention(q, X, sink, scale)
    K = np.vstack([X, np.zeros((1, D))])
    mask = np.zeros((1, n + 1))
    mask[0, n] = sink
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(K)[None, None],
        torch.from_numpy(K)[None, None], attn_mask=torch.from_numpy(mask)[None, None],
        scale=scale)[0, 0, 0].numpy()
    np.testing.assert_allclose(o, ref, atol=1e-13)
    logits = scale * (X @ q)
    assert abs(lse - np.logaddexp.reduce(np.append(logits, sink))) < 1e-12


def test_weights_sum_to_sigmoid_and_sink_scales_output():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((50, 8))
    q = rng.standard_normal(8) * 4
    sink = 1.3
    o, lse, wts = O.sink_attention(q, X, sink, 0.5)
    lse_x = np.logaddexp.reduce(0.5 * (X @ q))
    sig = 1 / (1 + math.exp(-(lse_x - sink)))
    assert abs(wts.sum() - sig) < 1e-13 and wts.sum() <= 1.0
    o0, _, _ = O.sink_attention(q, X, -1e300, 0.5)
    np.testing.assert_allclose(o, o0 * sig, atol=1e-13)


def test_no_rows_gives_zero_output():
    o, lse, w = O.sink_attention(np.ones(4), np.zeros((0, 4)), 0.25, 1.0)
    assert np.all(o == 0) and lse == 0.25


def test_brute_force_tiny():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((5, 3))
    q = rng.standard_normal(3)
    o, lse, _ = O.sink_attention(q, X, -0.4, 0.7)
    ex = [math.exp(0.7 * sum(q[d] * X[i, d] for d in range(3))) for i in range(5)]
    Z = sum(ex) + math.exp(-0.4)
    for d in range(3):
        assert abs(o[d] - sum(ex[i] * X[i, d] for i in range(5)) / Z) < 1e-13
    assert abs(lse - math.log(Z)) < 1e-13


def _small_case(rng, m=4, Tq=6, q_pos0=40, N=None, H=3, D=8, W=8):
    N = N or (q_pos0 + Tq) // m
    E = rng.standard_normal((N, D))
    win = rng.standard_normal((W - 1 + Tq, D))
    q = rng.standard_normal((Tq, H, D)) * 2
    sink = rng.standard_normal(H)
    return E, win, q, sink


def test_csa_with_all_entries_equals_hca():
    rng = np.random.default_rng(3)
    m, Tq, q_pos0, W = 4, 6, 40, 8
    E, win, q, sink = _small_case(rng, m, Tq, q_pos0, W=W)
    idx = np.full((Tq, 64), -1)
    for t in range(Tq):
        nv = O.n_visible(q_pos0 + t, m)
        idx[t, :nv] = np.arange(nv)
    a, la = O.csa_attend(q, E, idx, win, sink, 0.3, q_pos0, W)
    b, lb = O.hca_attend(q, E, m, win, sink, 0.3, q_pos0, W)
    np.testing.assert_allclose(a, b, atol=1e-13)
    np.testing.assert_allclose(la, lb, atol=1e-13)


def test_index_order_is_irrelevant():
    rng = np.random.default_rng(4)
    E, win, q, sink = _small_case(rng)
    sel = np.array([3, 7, 1, 9, -1, 0])
    a, _ = O.csa_attend_query(q[0], E, sel, win, sink, 0.3, 40, 40, 8)
    b, _ = O.csa_attend_query(q[0], E, sel[::-1], win, sink, 0.3, 40, 40, 8)
    np.testing.assert_allclose(a, b, atol=1e-13)


def test_window_only_is_textbook_sliding_window_softmax():
    # With no compressed entries and the sink at -inf, every query attends
    # exactly the raw tokens [max(0, p-W+1), p]: torch SDPA with a band mask.
    rng = np.random.default_rng(5)
    Tq, H, D, W = 20, 2, 8, 8
    win = rng.standard_normal((W - 1 + Tq, D))
    q = rng.standard_normal((Tq, H, D))
    idx = np.full((Tq, 4), -1)
    out, _ = O.csa_attend(q, np.zeros((1, D)), idx, win, np.full(H, -1e300), 0.4, 0, W)
    kv = win[W - 1:]                                     # positions 0..Tq-1
    pos = np.arange(Tq)
    allowed = (pos[None, :] <= pos[:, None]) & (pos[None, :] > pos[:, None] - W)
    mask = torch.from_numpy(np.where(allowed, 0.0, -np.inf))
    for h in range(H):
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q[:, h])[None], torch.from_numpy(kv)[None],
            torch.from_numpy(kv)[None], attn_mask=mask[None], scale=0.4)[0].numpy()
        np.testing.assert_allclose(out[:, h], ref, atol=1e-13)


def test_inverse_rope_makes_output_shift_invariant():
    # Rows carry RoPE at their own positions and queries at theirs; after the
    # output is rotated by -p the result depends only on relative positions,
    # so moving every position by the same offset leaves it unchanged.
    rng = np.random.default_rng(6)
    m, D, R, H, W, base = 4, 16, 8, 2, 8, 10000.0
    N, Tq = 12, 3
    E0 = rng.standard_normal((N, D))
    win0 = rng.standard_normal((W - 1 + Tq, D))
    q0 = rng.standard_normal((Tq, H, D))
    sink = rng.standard_normal(H)
    results = []
    for q_pos0 in (48, 48 + 4 * 1000):
        shift = q_pos0 - 48
        E = np.stack([O.rope_rotate(E0[j], j * m + shift, base, R) for j in range(N)])
        win = np.stack([O.rope_rotate(win0[r], q_pos0 - (W - 1) + r, base, R)
                        for r in range(W - 1 + Tq)])
        q = np.stack([O.rope_rotate(q0[t], q_pos0 + t, base, R) for t in range(Tq)])
        idx = np.tile(np.arange(N), (Tq, 1))
        # entries beyond the unshifted horizon are masked the same way
        out, _ = O.csa_attend(q, E, idx, win, sink, 0.25, q_pos0, W, inv_rope=True,
                              rope_base=base, rope_dims=R)
        results.append(out)
    np.testing.assert_allclose(results[0], results[1], atol=1e-10)


def test_window_clipped_at_sequence_start():
    assert O.window_positions(3, 128).tolist() == [0, 1, 2, 3]
    assert O.window_positions(200, 128)[0] == 73
