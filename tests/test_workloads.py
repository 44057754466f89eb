"""Seeded input generators: shapes, storage exactness, per-sequence regeneration."""

import json
import os

import numpy as np
import torch

import workloads as WL

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_exact_matches_torch_storage_cast():
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(WL.bf16_exact(x), ref)


def test_sequences_regenerate_alone():
    full = WL.make_csa_decode(B=3, ctx=4096)
    one = WL.make_csa_decode(B=3, ctx=4096, seqs=[2])
    for k in ("E", "kI", "q", "qI", "w", "win"):
        np.testing.assert_array_equal(full[k][2], one[k][0])
    np.testing.assert_array_equal(full["sink"], one["sink"])


def test_decode_shapes_follow_page_hparams():
    hp = json.load(open(os.path.join(GOLD, "page_hparams.json")))
    d = WL.make_csa_decode(B=1, ctx=4096)
    assert d["m"] == hp["csa_compress_ratio"]["value"]
    assert d["W"] == hp["sliding_window"]["value"]
    assert d["k"] == hp["index_topk_flash"]["value"]
    assert d["H"] == hp["query_heads_flash"]["value"]
    assert d["D"] == hp["head_dim"]["value"] and d["d_I"] == hp["indexer_head_dim"]["value"]
    h = WL.make_hca_decode(B=1, ctx=1048576 // 64)
    assert h["m"] == hp["hca_compress_ratio"]["value"] and h["H"] == hp["query_heads_pro"]["value"]
    assert d["E"].shape == (1, 1024, 512) and d["win"].shape == (1, 128, 512)
    # values are exact bf16
    np.testing.assert_array_equal(WL.bf16_exact(d["E"]), d["E"])


def test_spikes_present():
    d = WL.make_csa_decode(B=1, ctx=40000)
    norms = np.linalg.norm(d["kI"][0], axis=1)
    assert np.sum(norms > 2.5) >= int(0.01 * 10000) * 0.9
