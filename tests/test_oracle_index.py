"""Pins of the oracle's Lightning Indexer scores and top-k selection."""

import json
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_scores_brute_force_loops():
    rng = np.random.default_rng(0)
    H_I, d_I, N = 3, 5, 11
    q, w, k = rng.standard_normal((H_I, d_I)), rng.standard_normal(H_I), rng.standard_normal((N, d_I))
    s = O.index_scores(q, w, k, 9)
    assert s.shape == (9,)
    for j in range(9):
        tot = 0.0
        for h in range(H_I):
            dot = sum(q[h, d] * k[j, d] for d in range(d_I))
            tot += w[h] * (dot if dot > 0 else 0.0)
        assert abs(s[j] - tot) < 1e-13


def test_single_head_positive_dots_are_inner_products():
    rng = np.random.default_rng(1)
    q = np.abs(rng.standard_normal((1, 16)))
    k = np.abs(rng.standard_normal((40, 16)))
    s = O.index_scores(q, np.ones(1), k, 40)
    ref = (torch.from_numpy(k) @ torch.from_numpy(q[0])).numpy()
    np.testing.assert_allclose(s, ref, rtol=1e-14)


def test_relu_drops_negative_dots():
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    k = np.array([[-2.0, 3.0], [4.0, -5.0], [-1.0, -1.0]])
    s = O.index_scores(q, np.array([2.0, 10.0]), k, 3)
    np.testing.assert_allclose(s, [30.0, 8.0, 0.0])


def test_topk_against_stable_sort_with_ties():
    rng = np.random.default_rng(2)
    for trial in range(50):
        n = int(rng.integers(1, 60))
        s = rng.integers(-3, 4, size=n).astype(np.float64)   # many ties
        k = int(rng.integers(1, 70))
        got = O.topk_select(s, k).tolist()
        want = sorted(range(n), key=lambda j: (-s[j], j))[:min(k, n)]
        assert got == want


def test_topk_matches_torch_on_tie_free_data():
    rng = np.random.default_rng(3)
    s = rng.standard_normal(5000)
    got = set(O.topk_select(s, 300).tolist())
    want = set(torch.topk(torch.from_numpy(s), 300).indices.tolist())
    assert got == want


def test_topk_classes_consistency():
    rng = np.random.default_rng(4)
    s = rng.standard_normal(2000)
    s[10] = s[11] = s[12] = 1.5                       # ties near the boundary
    k = 100
    cin, cout, amb = O.topk_classes(s, k)
    exact = np.zeros(2000, bool)
    exact[O.topk_select(s, k)] = True
    assert np.all(exact[cin]) and not np.any(exact[cout])
    assert np.all(cin | cout | amb) and not np.any(cin & cout)
    assert cin.sum() <= k <= cin.sum() + amb.sum()


def test_topk_classes_bf16_mode():
    rng = np.random.default_rng(5)
    s = rng.standard_normal(3000)
    k = 200
    cin, cout, amb = O.topk_classes(s, k, bf16_scores=True)
    sb = O.bf16_round(s)
    kth = sb[O.topk_select(sb, k)[-1]]
    assert np.all(amb[sb == kth])
    assert np.all(sb[cin] > kth) and np.all(sb[cout] < kth)


def test_short_list_keeps_everything():
    s = np.array([0.1, 0.3, 0.2])
    assert O.topk_select(s, 512).tolist() == [1, 2, 0]


def test_visible_entry_counts_at_page_shapes():
    hp = json.load(open(os.path.join(GOLD, "page_hparams.json")))
    m = hp["csa_compress_ratio"]["value"]
    m2 = hp["hca_compress_ratio"]["value"]
    assert O.n_visible(131072, m) == 32768
    assert O.n_visible(1048576, m2) == 8192
    assert O.n_visible(1048576, m) == 262144
    assert O.n_visible(1048576 + 4095, m) == 262144 + 1024
    assert O.n_visible(2, m) == 0 and O.n_visible(3, m) == 1
