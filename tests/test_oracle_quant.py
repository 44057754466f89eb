"""Pins of the oracle's storage-precision quantisers and the storage layout."""

import json
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    # exact ties: values halfway between two bf16 neighbours
    ties = (np.float32(1.0) + np.float32(2.0 ** -8) * np.arange(1, 40, 2, dtype=np.float32))
    x = np.concatenate([x, ties, -ties, np.float32([0.0, 1e-40, -3e-39])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_round(x.astype(np.float64)), ref)
    assert O.bf16_round(np.array([1 + 2.0 ** -8]))[0] == 1.0          # tie to even


def test_e4m3fn_matches_torch_after_clamp():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-12, 7, 20000))).astype(np.float32)
    x = np.concatenate([x, np.float32([448, -448, 464, 500, 2.0 ** -9, 2.0 ** -10, 0.0])])
    xc = np.clip(x, -448, 448)
    ref = torch.from_numpy(xc).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3fn_decode(O.e4m3fn_encode(x.astype(np.float64)))
    np.testing.assert_array_equal(got, ref)


def test_e4m3fn_exhaustive_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = O.e4m3fn_decode(codes)
    back = O.e4m3fn_encode(vals)
    # -0 encodes as 0x80 and 0 as 0x00: both round-trip
    np.testing.assert_array_equal(back, codes)
    assert O.e4m3fn_decode(np.uint8(0x7E)) == 448.0
    assert O.e4m3fn_decode(np.uint8(0x01)) == 2.0 ** -9
    assert O.e4m3fn_decode(np.uint8(0x08)) == 2.0 ** -6


def test_e2m1_table_and_ties_from_ocp_spec():
    g = json.load(open(os.path.join(GOLD, "e2m1_ocp_mx.json")))
    table = {int(k): v for k, v in g["code_to_magnitude"].items()}
    for c in range(16):
        v = (-1 if c & 8 else 1) * table[c & 7]
        assert O.e2m1_decode(c) == v
        if c != 8:
            assert O.e2m1_encode(v) == c
    # halfway cases go to the code with mantissa bit 0; beyond 6 saturates
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 7.0: 7, 100.0: 7}
    for v, c in ties.items():
        assert O.e2m1_encode(v) == c, v
        assert O.e2m1_encode(-v) == c | 8, v


def test_mxfp4_scale_and_values():
    g = json.load(open(os.path.join(GOLD, "e2m1_ocp_mx.json")))
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64)).astype(np.float32) * 3
    codes, sc = O.mxfp4_quantize(x)
    for r in range(5):
        for b in range(2):
            amax = np.max(np.abs(x[r, 32 * b:32 * b + 32]))
            E = int(np.floor(np.log2(amax))) - g["emax_elem"]
            assert sc[r, b] == E + g["e8m0_bias"]
    dec = O.mxfp4_decode(codes, sc)
    # each decoded value is the nearest grid point of x / 2**E (within half a step)
    X = np.repeat(np.ldexp(1.0, sc.astype(int) - 127), 32, axis=1)
    y = np.abs(x) / X                           # in [0, 8)
    err = np.abs(dec - x) / X
    inside = y <= 6
    # inside the grid: at most half the largest gap (4 -> 6); above 6: saturate
    assert np.all(err[inside] <= 1.0 + 1e-12)
    np.testing.assert_array_equal(np.abs(dec[~inside]), 6 * X[~inside])
    assert np.all(np.abs(dec) <= 6 * X)


def test_mxfp4_zero_block():
    codes, sc = O.mxfp4_quantize(np.zeros((1, 32)))
    assert sc[0, 0] == 0 and np.all(codes == 0)


def test_kv_mixed_row_scale_and_roundtrip():
    rng = np.random.default_rng(3)
    rows = (rng.standard_normal((7, 512)) * 0.05).astype(np.float32)
    codes, rope, s = O.kv_mixed_quantize(rows)
    assert codes.shape == (7, 448) and rope.shape == (7, 64)
    amax = np.max(np.abs(rows[:, :448]), axis=1)
    np.testing.assert_array_equal(s, (amax / np.float32(448)).astype(np.float32))
    dec = O.kv_mixed_decode(codes, rope, s)
    rel = np.abs(dec[:, :448] - rows[:, :448]) / amax[:, None]
    assert rel.max() <= 2.0 ** -4 + 1e-7             # 3 mantissa bits: half-ulp 1/16 of binade
    np.testing.assert_array_equal(dec[:, 448:], O.bf16_round(rows[:, 448:].astype(np.float64)))


def test_storage_layout_matches_two_percent_figure():
    # The pages put the V4 KV cache at about 2% of a BF16 GQA8 (head dim 128)
    # cache at 1M context. With the mixed row (448 fp8 + 64 bf16 + fp32 scale)
    # and MXFP4 indexer keys (128 e2m1 + 4 e8m0), one CSA layer (m = 4) and
    # one HCA layer (m' = 128) average to about 2.0%.
    hp = json.load(open(os.path.join(GOLD, "page_hparams.json")))
    D, R, dI = hp["head_dim"]["value"], hp["rope_dims"]["value"], hp["indexer_head_dim"]["value"]
    m, m2 = hp["csa_compress_ratio"]["value"], hp["hca_compress_ratio"]["value"]
    kv_row = (D - R) * 1 + R * 2 + 4
    idx_row = dI // 2 + dI // 32
    assert kv_row == 580 and idx_row == 68
    csa = (kv_row + idx_row) / m
    hca = kv_row / m2
    gqa8 = 2 * 8 * 128 * 2                      # K and V, 8 heads, dim 128, bf16
    pct = 100 * (csa + hca) / 2 / gqa8
    assert abs(pct - hp["kv_cache_vs_bf16_gqa8_hd128_percent"]["value"]) < 0.1
    # an all-bf16 layout would be twice as large: the fp8/fp4 formats matter
    pct_bf16 = 100 * ((D * 2 + dI * 2) / m + D * 2 / m2) / 2 / gqa8
    assert pct_bf16 > 3.5


@pytest.mark.parametrize("v", [1.0, 2.0, 0.5, 2.0 ** -100, 3.0, 0.99609375, -1.0, -6.0, 2.0 ** -126])
def test_bf16_neighbours_match_torch_nextafter(v):
    # The bf16 ambiguity band of the top-k classes is built on the neighbours
    # of the k-th score. At a power of two the step below is half the step
    # above; torch's nextafter on bfloat16 fixes both independently.
    t = torch.tensor([v], dtype=torch.bfloat16)
    up = torch.nextafter(t, torch.tensor([1e30], dtype=torch.bfloat16)).double().item()
    dn = torch.nextafter(t, torch.tensor([-1e30], dtype=torch.bfloat16)).double().item()
    assert O.bf16_next(v, +1) == up
    assert O.bf16_next(v, -1) == dn


def test_kv_mixed_hand_built_rows():
    # Rows whose codes follow from the e4m3fn table by hand: an amax of
    # exactly 448 gives scale 1 and stores the channels themselves; a zero
    # row takes scale 1 and all-zero codes; the channel that holds the amax
    # always stores +-448 (code 0x7E / 0xFE), whatever the scale.
    rows = np.zeros((3, 512), np.float32)
    rows[0, :4] = [448.0, -1.0, 0.5, 2.0 ** -9]
    rows[0, 448:] = 1.0 + 2.0 ** -8                      # a bf16 tie: rounds to 1.0
    rows[2, :448] = np.linspace(-0.01, 0.02, 448, dtype=np.float32)
    codes, rope, s = O.kv_mixed_quantize(rows)
    assert s[0] == 1.0 and s[1] == 1.0
    assert list(codes[0, :4]) == [0x7E, 0xB8, 0x30, 0x01]
    assert np.all(codes[1] == 0) and np.all(rope[1] == 0)
    np.testing.assert_array_equal(rope[0], 1.0)
    assert codes[2, 447] == 0x7E and s[2] == np.float32(np.float32(0.02) / np.float32(448))
