"""Parity of each HIP entry point against the float64 oracle, at sizes the
oracle finishes in seconds: several tiles, ragged tails, degenerate cases."""

import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import (DEV, check_topk_set, dev_bf16, dev_f32, host, need_gpu, row_tol_check, say)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# quantise-on-write: codes must equal the oracle's bit for bit
# ---------------------------------------------------------------------------

def _special_rows(rng, n, D):
    x = (rng.standard_normal((n, D)) * np.exp(rng.uniform(-6, 3, (n, 1)))).astype(np.float32)
    x[0] = 0.0                                   # all-zero row
    x[1, :] = 1.0                                # constant row
    x[2, :8] = np.float32([448, -448, 1e-6, -1e-6, 2.0 ** -9, 3.0, -0.0, 7.0])
    return x


def test_quantize_kv_mixed_bit_exact():
    L = need_gpu()
    rng = np.random.default_rng(11)
    n, D, R = 333, 512, 64
    x = _special_rows(rng, n, D)
    out = torch.empty((n, D - R + 2 * R), dtype=torch.uint8, device=DEV)
    sc = torch.empty(n, dtype=torch.float32, device=DEV)
    L.lca_quantize_rows(L.KV_MIXED, dev_f32(x), out, sc, rope_dims=R)
    torch.cuda.synchronize()
    codes, rope, s = O.kv_mixed_quantize(x, R)
    o = out.cpu().numpy()
    np.testing.assert_array_equal(sc.cpu().numpy(), s)
    np.testing.assert_array_equal(o[:, :D - R], codes)
    tail = o[:, D - R:].copy().view(np.uint16).astype(np.uint32) << 16
    np.testing.assert_array_equal(tail.view(np.float32).astype(np.float64), rope)


def test_quantize_mxfp4_bit_exact():
    L = need_gpu()
    rng = np.random.default_rng(12)
    n, D = 257, 128
    x = _special_rows(rng, n, D)
    x[3, :32] = np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.9] * 4) * 0.5   # exact ties
    out = torch.empty((n, D // 2), dtype=torch.uint8, device=DEV)
    sc = torch.empty((n, D // 32), dtype=torch.uint8, device=DEV)
    L.lca_quantize_rows(L.MXFP4, dev_f32(x), out, sc)
    torch.cuda.synchronize()
    codes, scales = O.mxfp4_quantize(x)
    o = out.cpu().numpy()
    np.testing.assert_array_equal(sc.cpu().numpy(), scales)
    np.testing.assert_array_equal(o & 0xF, codes[:, 0::2])
    np.testing.assert_array_equal(o >> 4, codes[:, 1::2])


# ---------------------------------------------------------------------------
# compressor
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["csa", "csa_prev", "csa_norm_rope", "hca"])
def test_compress_matches_oracle(dt, mode):
    L = need_gpu()
    rng = np.random.default_rng(13)
    B, D = 2, 128
    m = 128 if mode == "hca" else 4
    T = 3 * m + 3 if mode != "hca" else 2 * m + 5        # ragged tail
    pos0 = 8 * m
    cast = (lambda a: WL.bf16_exact(a)) if dt == "bf16" else (lambda a: a.astype(np.float32))
    ca = cast(rng.standard_normal((B, T, D)).astype(np.float32))
    cb = cast(rng.standard_normal((B, T, D)).astype(np.float32))
    za = (rng.standard_normal((B, T)) * 2).astype(np.float32)
    zb = (rng.standard_normal((B, T)) * 2).astype(np.float32)
    pca = cast(rng.standard_normal((B, m, D)).astype(np.float32))
    pza = rng.standard_normal((B, m)).astype(np.float32)
    nw = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    overlap = mode != "hca"
    use_prev = mode in ("csa_prev", "csa_norm_rope")
    flags = (L.NORM | L.ROPE) if mode == "csa_norm_rope" else 0
    R = 64 if flags else 0
    up = dev_bf16 if dt == "bf16" else dev_f32
    dti = L.BF16 if dt == "bf16" else L.F32
    n_out = T // m
    out = torch.empty((B, n_out, D), dtype=torch.float32, device=DEV)
    L.csa_compress(dti, L.F32, up(cb), dev_f32(zb), m, ca=up(ca) if overlap else None,
                   za=dev_f32(za) if overlap else None,
                   prev_ca=up(pca) if use_prev else None, prev_za=dev_f32(pza) if use_prev else None,
                   overlap=overlap, pos0=pos0, flags=flags, norm_w=dev_f32(nw) if flags else None,
                   eps=1e-6, rope_base=10000.0, rope_dims=R, out=out)
    torch.cuda.synchronize()
    got = host(out)
    for b in range(B):
        ref = O.compress_sequence(cb[b], zb[b], m, ca[b] if overlap else None, za[b] if overlap else None,
                                  pca[b] if use_prev else None, pza[b] if use_prev else None, overlap)
        if flags:
            ref = O.compress_epilogue(ref, pos0, m, nw, 1e-6, 10000.0, R)
        row_tol_check(got[b], ref, 1e-5, f"compress {mode} {dt}")


def test_compress_chunked_equals_one_shot_bitwise():
    L = need_gpu()
    rng = np.random.default_rng(14)
    B, T, D, m = 2, 64, 256, 4
    ca, cb = (WL.bf16_exact(rng.standard_normal((B, T, D)).astype(np.float32)) for _ in range(2))
    za, zb = (rng.standard_normal((B, T)).astype(np.float32) for _ in range(2))
    full = torch.empty((B, T // m, D), dtype=torch.bfloat16, device=DEV)
    L.csa_compress(L.BF16, L.BF16, dev_bf16(cb), dev_f32(zb), m, ca=dev_bf16(ca), za=dev_f32(za), out=full)
    T1 = 24
    part = torch.empty((B, T // m, D), dtype=torch.bfloat16, device=DEV)
    L.csa_compress(L.BF16, L.BF16, dev_bf16(cb[:, :T1]), dev_f32(zb[:, :T1]), m, ca=dev_bf16(ca[:, :T1]),
                   za=dev_f32(za[:, :T1]), out=part, out_rows=T // m)
    L.csa_compress(L.BF16, L.BF16, dev_bf16(cb[:, T1:]), dev_f32(zb[:, T1:]), m, ca=dev_bf16(ca[:, T1:]),
                   za=dev_f32(za[:, T1:]), prev_ca=dev_bf16(ca[:, T1 - m:T1]),
                   prev_za=dev_f32(za[:, T1 - m:T1]), pos0=T1, out=part[:, T1 // m:], out_rows=T // m)
    torch.cuda.synchronize()
    assert torch.equal(full, part)


def test_compress_constant_sequence_quantised_outputs():
    # constant rows compress to themselves; then the quantised outputs equal
    # the oracle's quantisation of that row
    L = need_gpu()
    rng = np.random.default_rng(15)
    B, T, D, m = 1, 16, 512, 4
    c = rng.standard_normal(D).astype(np.float32)
    rows = np.tile(c, (B, T, 1))
    z = rng.standard_normal((B, T)).astype(np.float32)
    out = torch.empty((B, T // m, D + 64), dtype=torch.uint8, device=DEV)
    sc = torch.empty((B, T // m), dtype=torch.float32, device=DEV)
    L.csa_compress(L.F32, L.KV_MIXED, dev_f32(rows), dev_f32(z), m, ca=dev_f32(rows), za=dev_f32(z),
                   rope_dims=64, out=out, out_scale=sc)
    torch.cuda.synchronize()
    codes, rope, s = O.kv_mixed_quantize(c[None], 64)
    got = out.cpu().numpy()[0]
    # fp32 softmax weights sum to 1 within rounding: allow one code step
    dec_got = O.kv_mixed_decode(got[:, :448], (got[:, 448:].copy().view(np.uint16).astype(np.uint32) << 16)
                                .view(np.float32).astype(np.float64), sc.cpu().numpy()[0])
    dec_ref = O.kv_mixed_decode(codes, rope, s)[0]
    assert np.max(np.abs(dec_got - dec_ref)) <= 2 * np.max(np.abs(c)) / 16


# ---------------------------------------------------------------------------
# indexer scores + top-k
# ---------------------------------------------------------------------------

def _index_case(rng, B, Tq, H_I, d_I, N_cap, spikes=True, ties=False):
    qI = WL.bf16_exact(rng.standard_normal((B, Tq, H_I, d_I)).astype(np.float32) / np.sqrt(d_I))
    kI = rng.standard_normal((B, N_cap, d_I)).astype(np.float32) / np.sqrt(d_I)
    if spikes:
        kI[:, ::97] *= 4
    if ties:
        kI[:, 1::3] = kI[:, 0::3][:, :kI[:, 1::3].shape[1]]       # duplicated keys -> tied scores
    kI = WL.bf16_exact(kI)
    w = (rng.standard_normal((B, Tq, H_I)) / np.sqrt(H_I)).astype(np.float32)
    return qI, w, kI


@pytest.mark.parametrize("H_I", [1, 2, 4, 8, 16, 32, 64])
def test_index_topk_decode_bf16(H_I):
    L = need_gpu()
    rng = np.random.default_rng(20 + H_I)
    B, Tq, d_I, m, k = 3, 1, 128, 4, 256
    q_pos0 = 4 * 5000 + 2                    # n_vis = 5000: not a multiple of any tile
    N_cap = 5003
    qI, w, kI = _index_case(rng, B, Tq, H_I, d_I, N_cap)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    sco = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=q_pos0,
                     score_out=sco)
    torch.cuda.synchronize()
    idx_h, sco_h = idx.cpu().numpy(), sco.cpu().numpy()
    for b in range(B):
        nv = O.n_visible(q_pos0, m)
        s = O.index_scores(qI[b, 0], w[b, 0], kI[b], nv)
        check_topk_set(idx_h[b, 0], s, k)
        assert np.all(np.diff(idx_h[b, 0]) > 0), "indices not increasing"
        np.testing.assert_allclose(sco_h[b, 0], s[idx_h[b, 0]], rtol=1e-4, atol=1e-6)


@pytest.mark.parametrize("bf16_scores", [False, True])
def test_index_topk_prefill_causal_bf16(bf16_scores):
    L = need_gpu()
    rng = np.random.default_rng(30)
    B, Tq, H_I, d_I, m, k = 2, 37, 4, 64, 4, 50
    q_pos0 = 180
    N_cap = (q_pos0 + Tq) // m
    qI, w, kI = _index_case(rng, B, Tq, H_I, d_I, N_cap, ties=True)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=q_pos0,
                     flags=L.SCORE_BF16 if bf16_scores else 0)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    for b in range(B):
        for t in range(Tq):
            nv = O.n_visible(q_pos0 + t, m)
            s = O.index_scores(qI[b, t], w[b, t], kI[b], nv)
            check_topk_set(idx_h[b, t], s, k, bf16_scores=bf16_scores)


@pytest.mark.parametrize("H_I", [1, 4, 16])
@pytest.mark.parametrize("bf16_scores", [False, True])
def test_index_topk_many_queries_tiled(H_I, bf16_scores):
    # >= 64 queries with d_I = 128 take the key-tiled path: ragged query tiles,
    # ragged key tiles and key ranges, causal limits inside a tile
    L = need_gpu()
    rng = np.random.default_rng(60 + H_I)
    B, Tq, d_I, m, k = 2, 150, 128, 4, 100
    q_pos0 = 4 * 1700 + 1
    N_cap = (q_pos0 + Tq) // m + 5
    qI, w, kI = _index_case(rng, B, Tq, H_I, d_I, N_cap, ties=True)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    sco = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    say(f"tiled index H_I={H_I} bf16={bf16_scores}")
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=q_pos0,
                     flags=L.SCORE_BF16 if bf16_scores else 0, score_out=sco)
    torch.cuda.synchronize()
    idx_h, sco_h = idx.cpu().numpy(), sco.cpu().numpy()
    for b in range(B):
        for t in range(Tq):
            nv = O.n_visible(q_pos0 + t, m)
            s = O.index_scores(qI[b, t], w[b, t], kI[b], nv)
            check_topk_set(idx_h[b, t], s, k, bf16_scores=bf16_scores)
            sel = idx_h[b, t][idx_h[b, t] >= 0]
            ref = O.bf16_round(s[sel]) if bf16_scores else s[sel]
            tol = np.abs(ref) * (2.0 ** -7 if bf16_scores else 1e-4) + 1e-6 * np.max(np.abs(s))
            assert np.all(np.abs(sco_h[b, t][:len(sel)] - ref) <= tol), (b, t)


@pytest.mark.parametrize("H_I,bf16_scores", [(32, False), (64, True)])
def test_index_topk_wide_heads_many_queries(H_I, bf16_scores):
    # The pages' 64 indexer heads (and 32): one query's heads span several
    # MFMA tiles. 70 queries over lists longer than one register round: the
    # scores and group maxima of the wide kernel feed the chunked select.
    L = need_gpu()
    rng = np.random.default_rng(62 + H_I)
    B, Tq, d_I, m, k = 1, 70, 128, 4, 300
    q_pos0 = 4 * 40000 + 3
    N_cap = (q_pos0 + Tq) // m + 2
    qI, w, kI = _index_case(rng, B, Tq, H_I, d_I, N_cap)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    sco = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    say(f"wide-head index H_I={H_I} bf16={bf16_scores}")
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=q_pos0,
                     flags=L.SCORE_BF16 if bf16_scores else 0, score_out=sco)
    torch.cuda.synchronize()
    idx_h, sco_h = idx.cpu().numpy(), sco.cpu().numpy()
    for t in list(range(0, Tq, 7)) + [Tq - 1]:
        nv = O.n_visible(q_pos0 + t, m)
        s = O.index_scores(qI[0, t], w[0, t], kI[0], nv)
        check_topk_set(idx_h[0, t], s, k, bf16_scores=bf16_scores)
        sel = idx_h[0, t][idx_h[0, t] >= 0]
        ref = O.bf16_round(s[sel]) if bf16_scores else s[sel]
        tol = np.abs(ref) * (2.0 ** -7 if bf16_scores else 1e-4) + 1e-6 * np.max(np.abs(s))
        assert np.all(np.abs(sco_h[0, t][:len(sel)] - ref) <= tol), t


def test_index_topk_many_queries_from_sequence_start():
    # tiled path with queries from position 0: the first ones see no entry
    L = need_gpu()
    rng = np.random.default_rng(61)
    B, Tq, H_I, d_I, m, k = 1, 300, 4, 128, 4, 16
    N_cap = Tq // m
    qI, w, kI = _index_case(rng, B, Tq, H_I, d_I, N_cap)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=0)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    assert np.all(idx_h[0, :3] == -1)
    for t in range(Tq):
        s = O.index_scores(qI[0, t], w[0, t], kI[0], O.n_visible(t, m))
        check_topk_set(idx_h[0, t], s, k)


@pytest.mark.parametrize("bf16_scores", [False, True])
@pytest.mark.parametrize("distinct", [None, 40, 6])
def test_index_topk_long_lists(bf16_scores, distinct):
    # lists longer than one register round (32768) take the two-read select:
    # first-digit histogram, then the boundary bin's entries as candidates in
    # LDS. 40 distinct keys: ~2500 tied candidates, resolved in LDS. 6 distinct
    # keys: ~16700 in the boundary bin, more than LDS holds -> full passes.
    L = need_gpu()
    crowded = distinct is not None
    rng = np.random.default_rng(70 + 2 * (distinct or 0) + bf16_scores)
    B, Tq, H_I, d_I, m, k = 2, 1, 4, 128, 4, 1024
    N_cap = 100003
    q_pos0 = 4 * 100000 + 1                   # n_vis = 100000: four rounds, ragged
    qI, w, kI = _index_case(rng, B, Tq, H_I, d_I, N_cap)
    if crowded:
        kI = WL.bf16_exact(kI[:, rng.integers(0, distinct, size=N_cap)])
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    sco = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    say(f"long list bf16={bf16_scores} distinct={distinct}")
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=q_pos0,
                     flags=L.SCORE_BF16 if bf16_scores else 0, score_out=sco)
    torch.cuda.synchronize()
    idx_h, sco_h = idx.cpu().numpy(), sco.cpu().numpy()
    for b in range(B):
        nv = O.n_visible(q_pos0, m)
        s = O.index_scores(qI[b, 0], w[b, 0], kI[b], nv)
        check_topk_set(idx_h[b, 0], s, k, bf16_scores=bf16_scores)
        assert np.all(np.diff(idx_h[b, 0]) > 0), "indices not increasing"
        sel = idx_h[b, 0]
        ref = O.bf16_round(s[sel]) if bf16_scores else s[sel]
        tol = np.abs(ref) * (2.0 ** -7 if bf16_scores else 1e-4) + 1e-6 * np.max(np.abs(s))
        assert np.all(np.abs(sco_h[b, 0] - ref) <= tol)


def test_index_topk_f32_from_sequence_start():
    # queries from position 0: the first ones see no entry (all padding)
    L = need_gpu()
    rng = np.random.default_rng(31)
    B, Tq, H_I, d_I, m, k = 1, 80, 4, 64, 4, 8
    N_cap = Tq // m
    qI = rng.standard_normal((B, Tq, H_I, d_I)).astype(np.float32)
    kI = rng.standard_normal((B, N_cap, d_I)).astype(np.float32)
    w = rng.standard_normal((B, Tq, H_I)).astype(np.float32)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    sco = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    L.csa_index_topk(L.F32, dev_f32(qI), dev_f32(w), dev_f32(kI), idx, m=m, k=k, q_pos0=0, score_out=sco)
    torch.cuda.synchronize()
    idx_h, sco_h = idx.cpu().numpy(), sco.cpu().numpy()
    assert np.all(idx_h[0, :3] == -1)
    for t in range(Tq):
        nv = O.n_visible(t, m)
        s = O.index_scores(qI[0, t], w[0, t], kI[0], nv)
        check_topk_set(idx_h[0, t], s, k)
        sel = idx_h[0, t][idx_h[0, t] >= 0]
        # fp32 accumulation with cancellation: absolute error scales with |score| overall
        np.testing.assert_allclose(sco_h[0, t][:len(sel)], s[sel], rtol=1e-5,
                                   atol=1e-6 * max(1.0, float(np.max(np.abs(s))) if nv else 1.0))


def _mxfp4_on_gpu(L, x):
    """Quantise float32 rows [..., 128] to MXFP4 on the GPU (codes checked bit-exact elsewhere)."""
    flat = x.reshape(-1, x.shape[-1])
    codes = torch.empty((flat.shape[0], flat.shape[1] // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((flat.shape[0], flat.shape[1] // 32), dtype=torch.uint8, device=DEV)
    L.lca_quantize_rows(L.MXFP4, dev_f32(flat), codes, scales)
    return codes.reshape(x.shape[:-1] + (x.shape[-1] // 2,)), scales.reshape(x.shape[:-1] + (x.shape[-1] // 32,))


@pytest.mark.parametrize("H_I", [1, 4, 16, 32, 64])
@pytest.mark.parametrize("bf16_scores", [True, False])
def test_index_topk_mxfp4(H_I, bf16_scores):
    # MXFP4 indexer operands (queries and keys), heavy-tailed query norms; the
    # oracle quantises the same float32 sources itself and scores the decoded values
    L = need_gpu()
    rng = np.random.default_rng(50 + H_I)
    B, Tq, d_I, m, k = 2, 2, 128, 4, 300
    q_pos0 = 4 * 5000 + 2
    N_cap = 5003
    g = rng.standard_normal((B, Tq, H_I, d_I)).astype(np.float32)
    tau = rng.standard_t(3, size=(B, Tq, H_I, 1)).astype(np.float32)
    qI = g / np.linalg.norm(g, axis=-1, keepdims=True) * np.abs(tau)
    kI = (rng.standard_normal((B, N_cap, d_I)) / np.sqrt(d_I)).astype(np.float32)
    kI[:, ::97] *= 4
    w = (rng.standard_normal((B, Tq, H_I)) / np.sqrt(H_I)).astype(np.float32)
    qc, qs = _mxfp4_on_gpu(L, qI)
    kc, ks = _mxfp4_on_gpu(L, kI)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    sco = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    say(f"mxfp4 index H_I={H_I} bf16={bf16_scores}")
    L.csa_index_topk(L.MXFP4, qc, dev_f32(w), kc, idx, m=m, k=k, q_pos0=q_pos0, d_I=d_I, qI_scale=qs,
                     kI_scale=ks, flags=L.SCORE_BF16 if bf16_scores else 0, score_out=sco)
    torch.cuda.synchronize()
    idx_h, sco_h = idx.cpu().numpy(), sco.cpu().numpy()
    qd = O.mxfp4_decode(*O.mxfp4_quantize(qI))
    kd = O.mxfp4_decode(*O.mxfp4_quantize(kI))
    for b in range(B):
        for t in range(Tq):
            nv = O.n_visible(q_pos0 + t, m)
            s = O.index_scores(qd[b, t], w[b, t], kd[b], nv)
            check_topk_set(idx_h[b, t], s, k, bf16_scores=bf16_scores)
            sel = idx_h[b, t][idx_h[b, t] >= 0]
            ref = O.bf16_round(s[sel]) if bf16_scores else s[sel]
            # bf16 mode: equal unless the fp32 sum sat on a rounding midpoint (one bf16 step)
            tol = np.abs(ref) * (2.0 ** -7 if bf16_scores else 1e-5) + 1e-6 * np.max(np.abs(s))
            assert np.all(np.abs(sco_h[b, t][:len(sel)] - ref) <= tol)
            if bf16_scores:
                assert np.mean(sco_h[b, t][:len(sel)] == ref) > 0.99


@pytest.mark.parametrize("bf16_scores", [False, True])
def test_index_topk_chunked_ties_exact(bf16_scores):
    # 20000 entries with 5 distinct keys, k = 700: thousands of entries tie at
    # the threshold, spread over the whole list. The result must be exactly the
    # oracle order (score descending, index ascending) cut at k.
    L = need_gpu()
    rng = np.random.default_rng(71 + bf16_scores)
    B, Tq, H_I, d_I, m, k = 2, 1, 4, 128, 4, 700
    N_cap = 20000
    base = WL.bf16_exact(rng.standard_normal((5, d_I)).astype(np.float32))
    kI = np.stack([base[rng.integers(0, 5, size=N_cap)] for _ in range(B)])
    qI = WL.bf16_exact(rng.standard_normal((B, Tq, H_I, d_I)).astype(np.float32))
    w = np.abs(rng.standard_normal((B, Tq, H_I))).astype(np.float32)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    q_pos0 = 4 * N_cap - 1
    say(f"chunked ties bf16={bf16_scores}")
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=q_pos0,
                     flags=L.SCORE_BF16 if bf16_scores else 0)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for b in range(B):
        sc = O.index_scores(qI[b, 0], w[b, 0], kI[b], N_cap)
        if bf16_scores:
            sc = O.bf16_round(sc)
        vals = np.unique(sc)
        assert len(vals) == 5 and np.min(np.diff(vals)) > 1e-4 * np.max(np.abs(vals)), "keys must be apart"
        order = np.lexsort((np.arange(N_cap), -sc))          # score descending, then index ascending
        np.testing.assert_array_equal(got[b, 0], np.sort(order[:k]))


def test_index_topk_all_ties_take_lowest_indices():
    L = need_gpu()
    B, Tq, H_I, d_I, m, k = 1, 1, 4, 128, 4, 100
    N_cap = 3000
    kI = np.zeros((B, N_cap, d_I), np.float32)
    kI[0, :, 0] = 1.0                          # every key identical
    qI = np.zeros((B, Tq, H_I, d_I), np.float32)
    qI[0, 0, :, 0] = 0.5
    w = np.ones((B, Tq, H_I), np.float32)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=4 * N_cap - 1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy()[0, 0], np.arange(k))


@pytest.mark.parametrize("case", ["spread", "spikes", "ragged", "small_k", "ties5", "zeros", "same",
                                  "fine", "fine_spikes", "fine_ties5"])
@pytest.mark.parametrize("bf16_scores", [False, True])
def test_index_topk_select_exact_order(case, bf16_scores):
    # Integer indexer vectors and power-of-two head weights make every score
    # exact in fp32, so the expected result is exact: score descending, index
    # ascending, cut at k, returned in index order. Lists of 20000 - 32768
    # entries with k far below n / 64 take the select that filters candidates
    # by the threads' maxima (spread, spikes, ragged, small_k; zeros, the exact
    # zeros of all-negative head weights, as a candidate range one key wide);
    # 5 distinct keys and one key for every entry crowd the candidates past
    # their cap and take the full passes. The fine cases (12000 - 20001 entries,
    # k = 512: fewer than 2k threads hold a score) bound the k-th score by the
    # maxima of runs of 8 scores. With integer scores the boundary bin is often
    # a crowd of equal keys, ranked directly when it holds at most 64.
    L = need_gpu()
    rng = np.random.default_rng(400 + len(case) + 7 * bf16_scores)
    B, Tq, H_I, d_I, m = 2, 1, 4, 128, 4
    N_cap, k = 32768, 512
    if case == "ragged":
        N_cap, k = 30001, 256
    if case == "small_k":
        k = 16
    if case.startswith("fine"):
        N_cap = 12000 if case == "fine" else 20001
    qI = rng.integers(-8, 9, size=(B, Tq, H_I, d_I)).astype(np.float32)
    kI = rng.integers(-8, 9, size=(B, N_cap, d_I)).astype(np.float32)
    w = np.tile(np.array([1.0, 0.5, 0.25, 0.125], np.float32), (B, Tq, 1))
    if case in ("spikes", "fine_spikes"):
        for b in range(B):
            kI[b, rng.choice(N_cap, size=N_cap // 100, replace=False)] *= 4
    elif case in ("ties5", "fine_ties5"):
        base = rng.integers(-8, 9, size=(5, d_I)).astype(np.float32)
        kI = np.stack([base[rng.integers(0, 5, size=N_cap)] for _ in range(B)])
    elif case == "zeros":
        w = -w
    elif case == "same":
        kI[:] = kI[:, :1]
    q_pos0 = m * N_cap - 1                 # every entry visible
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    say(f"select exact order {case} bf16={bf16_scores}")
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=q_pos0,
                     flags=L.SCORE_BF16 if bf16_scores else 0)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for b in range(B):
        nv = min(N_cap, O.n_visible(q_pos0, m))
        sc = O.index_scores(qI[b, 0], w[b, 0], kI[b], nv)
        assert np.all(np.abs(sc) < 2.0 ** 23), "scores must stay exact in fp32"
        if bf16_scores:
            sc = O.bf16_round(sc)
        order = np.lexsort((np.arange(nv), -sc))
        np.testing.assert_array_equal(got[b, 0], np.sort(order[:k]), err_msg=f"{case} b={b}")


@pytest.mark.parametrize("case", ["spread", "spikes", "zeros", "same", "ties5", "cluster"])
@pytest.mark.parametrize("bf16_scores", [False, True])
def test_index_topk_long_exact_order(case, bf16_scores):
    # Lists longer than one register round take the chunked select: the bound
    # from group maxima (here from the bound kernel, with groups merged in
    # pairs past 8192 of them), candidates per 4096-entry chunk (512 slots
    # above 131072 entries), then one workgroup per row. Integer vectors and
    # power-of-two weights make every score exact, so the expected result is
    # exact. zeros: all-negative head weights, the k-th score is 0 and a crowd
    # of ties at the bound decides (the winners are the lowest indices); same:
    # every entry equal; ties5: five distinct scores; cluster: the highest
    # scores crowd one chunk past its slots (the full passes resolve the row).
    L = need_gpu()
    rng = np.random.default_rng(500 + len(case) + 7 * bf16_scores)
    B, Tq, H_I, d_I, m, k = 1, 1, 4, 128, 4, 1024
    N_cap = 140000
    qI = rng.integers(-8, 9, size=(B, Tq, H_I, d_I)).astype(np.float32)
    kI = rng.integers(-8, 9, size=(B, N_cap, d_I)).astype(np.float32)
    w = np.tile(np.array([1.0, 0.5, 0.25, 0.125], np.float32), (B, Tq, 1))
    if case == "spikes":
        kI[0, rng.choice(N_cap, size=N_cap // 100, replace=False)] *= 4
    elif case == "zeros":
        w = -w
    elif case == "same":
        kI[:] = kI[:, :1]
    elif case == "ties5":
        base = rng.integers(-8, 9, size=(5, d_I)).astype(np.float32)
        kI = base[rng.integers(0, 5, size=N_cap)][None]
    elif case == "cluster":
        kI[0, 50000:54096] *= 3
    q_pos0 = m * N_cap - 1
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    sco = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    say(f"long exact order {case} bf16={bf16_scores}")
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=q_pos0,
                     flags=L.SCORE_BF16 if bf16_scores else 0, score_out=sco)
    torch.cuda.synchronize()
    got, gs = idx.cpu().numpy(), sco.cpu().numpy()
    sc = O.index_scores(qI[0, 0], w[0, 0], kI[0], N_cap)
    assert np.all(np.abs(sc) < 2.0 ** 23), "scores must stay exact in fp32"
    if bf16_scores:
        sc = O.bf16_round(sc)
    want = np.sort(np.lexsort((np.arange(N_cap), -sc))[:k])
    np.testing.assert_array_equal(got[0, 0], want, err_msg=case)
    np.testing.assert_array_equal(gs[0, 0], sc[want].astype(np.float32))


@pytest.mark.parametrize("case,H_I,k", [("mixed_w", 4, 1024), ("cluster", 4, 1024), ("mixed_w", 2, 1024),
                                        ("mixed_w", 8, 1024), ("mixed_w", 4, 256), ("cluster", 16, 256)])
@pytest.mark.parametrize("bf16_scores", [False, True])
def test_index_topk_prefill_without_stored_scores(case, H_I, k, bf16_scores):
    # Many queries over long lists take the prefill path that stores no
    # scores: tiled scoring writes group maxima, the bound kernel bounds each
    # row, tiled scoring runs again and writes only the candidates, the final
    # kernel selects (output scores rebuilt from the candidates' keys). Exact
    # integer scores; per-query head weights, one query in four with all of
    # them negative (the k-th score is 0, a crowd of ties at the bound);
    # cluster: the highest scores of every query crowd 3 key ranges, more
    # candidates than the final workgroup holds in registers. H_I = 2 puts
    # two queries in each lane's accumulators, H_I = 8 one query in two lane
    # groups. The maxima pass takes every second 64-key tile (140000
    # entries: 4375 such groups, at least 3 k), so the bound comes from a
    # sample of the maxima.
    L = need_gpu()
    rng = np.random.default_rng(540 + 3 * bf16_scores + len(case) + H_I + k)
    B, Tq, d_I, m = 1, 70, 128, 4
    q_pos0 = 4 * 140000
    N_cap = (q_pos0 + Tq) // m + 3
    qI = rng.integers(-8, 9, size=(B, Tq, H_I, d_I)).astype(np.float32)
    kI = rng.integers(-8, 9, size=(B, N_cap, d_I)).astype(np.float32)
    w = np.tile((0.5 ** np.arange(H_I)).astype(np.float32), (B, Tq, 1))
    w[:, ::4] *= -1
    if case == "cluster":
        w = np.abs(w)
        kI[0, 60000:63072] *= 3
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    sco = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    say(f"prefill without stored scores {case} H_I={H_I} k={k} bf16={bf16_scores}")
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=q_pos0,
                     flags=L.SCORE_BF16 if bf16_scores else 0, score_out=sco)
    torch.cuda.synchronize()
    got, gs = idx.cpu().numpy(), sco.cpu().numpy()
    for t in range(Tq):
        nv = O.n_visible(q_pos0 + t, m)
        sc = O.index_scores(qI[0, t], w[0, t], kI[0], nv)
        assert np.all(np.abs(sc) < 2.0 ** 23), "scores must stay exact in fp32"
        if bf16_scores:
            sc = O.bf16_round(sc)
        want = np.sort(np.lexsort((np.arange(nv), -sc))[:k])
        np.testing.assert_array_equal(got[0, t], want, err_msg=f"{case} t={t}")
        np.testing.assert_array_equal(gs[0, t], sc[want].astype(np.float32), err_msg=f"{case} t={t}")


def test_index_topk_prefill_without_stored_scores_ragged_query_tiles():
    # 130 queries: two whole 64-query tiles and a 2-query tail, over lists
    # between 2^15 and 2^18 entries, real-valued scores (oracle set check with
    # the near-tie classes) on the path that stores no scores
    L = need_gpu()
    rng = np.random.default_rng(560)
    B, Tq, H_I, d_I, m, k = 1, 130, 4, 128, 4, 512
    q_pos0 = 4 * 70000
    N_cap = (q_pos0 + Tq) // m + 5
    qI = WL.bf16_exact(rng.standard_normal((B, Tq, H_I, d_I)).astype(np.float32) / np.sqrt(d_I))
    kI = rng.standard_normal((B, N_cap, d_I)).astype(np.float32) / np.sqrt(d_I)
    kI[:, ::89] *= 4
    kI = WL.bf16_exact(kI)
    w = (rng.standard_normal((B, Tq, H_I)) / np.sqrt(H_I)).astype(np.float32)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    say("prefill without stored scores, ragged query tiles")
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=q_pos0)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for t in list(range(0, Tq, 9)) + [Tq - 2, Tq - 1]:
        nv = O.n_visible(q_pos0 + t, m)
        s = O.index_scores(qI[0, t], w[0, t], kI[0], nv)
        check_topk_set(got[0, t], s, k)
        sel = got[0, t][got[0, t] >= 0]
        assert np.all(np.diff(sel) > 0), "indices not increasing"


@pytest.mark.parametrize("k", [1024, 256, 128])
def test_index_topk_prefill_without_stored_scores_all_ties(k):
    # Every key identical, so every score of a row ties: the bound equals the
    # row's largest key, the bound kernel limits the candidates to the groups
    # up to the k-th one, and the answer is the k lowest indices. Odd queries
    # take negative head weights (their ties sit below zero or at zero). The
    # maxima pass takes every tile at k = 1024 and every second one at
    # k = 256 and 128 (40000 entries); the limit is then the end of the tile
    # of the k-th sampled group.
    L = need_gpu()
    rng = np.random.default_rng(570 + k)
    B, Tq, H_I, d_I, m = 1, 66, 4, 128, 4
    q_pos0 = 4 * 40000 + 2
    N_cap = (q_pos0 + Tq) // m + 1
    kI = np.tile(rng.integers(-4, 5, size=(1, 1, d_I)), (B, N_cap, 1)).astype(np.float32)
    qI = rng.integers(-4, 5, size=(B, Tq, H_I, d_I)).astype(np.float32)
    w = np.tile(np.array([0.5, 0.25, 1.0, 0.125], np.float32), (B, Tq, 1))
    w[:, 1::2] *= -1
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    say(f"prefill without stored scores, every score tied, k={k}")
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=q_pos0)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for t in range(Tq):
        nv = O.n_visible(q_pos0 + t, m)
        sc = O.index_scores(qI[0, t], w[0, t], kI[0], nv)
        assert np.all(sc == sc[0])
        np.testing.assert_array_equal(got[0, t], np.arange(k), err_msg=f"t={t}")


def test_index_topk_long_ragged_rows():
    # A ragged batch bounded at 140000 entries: the long rows take the chunked
    # select with a bound, the short ones (5000, 300 entries) have too few
    # groups for one, every score is a candidate, their chunks overflow and
    # the full passes resolve them; the empty row is all padding.
    L = need_gpu()
    rng = np.random.default_rng(520)
    B, Tq, H_I, d_I, m, k = 5, 1, 4, 128, 4, 1024
    N_cap = 140000
    bound = m * N_cap - 1
    pos = [bound, 0, 4 * 5000, 4 * 70000 + 3, 4 * 300]
    qI = rng.integers(-8, 9, size=(B, Tq, H_I, d_I)).astype(np.float32)
    kI = rng.integers(-8, 9, size=(B, N_cap, d_I)).astype(np.float32)
    w = np.tile(np.array([1.0, -0.5, 0.25, 0.125], np.float32), (B, Tq, 1))
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    qp = torch.tensor(pos, dtype=torch.int64, device=DEV)
    say("long ragged rows")
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=bound, q_pos=qp)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for b in range(B):
        nv = O.n_visible(pos[b], m)
        sc = O.index_scores(qI[b, 0], w[b, 0], kI[b], nv)
        want = np.sort(np.lexsort((np.arange(nv), -sc))[:k])
        np.testing.assert_array_equal(got[b, 0][:len(want)], want, err_msg=f"b={b}")
        assert np.all(got[b, 0][len(want):] == -1)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _attend_case(rng, B, Tq, H, D, N_cap, W, sharp, cast):
    q = cast((rng.standard_normal((B, Tq, H, D)) * sharp / np.sqrt(D)).astype(np.float32))
    E = cast((rng.standard_normal((B, N_cap, D)) / np.sqrt(D)).astype(np.float32))
    win = cast((rng.standard_normal((B, W - 1 + Tq, D)) / np.sqrt(D)).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    return q, E, win, sink


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["csa", "hca"])
@pytest.mark.parametrize("sharp", [1.0, 30.0])
def test_attend_matches_oracle(dt, kind, sharp):
    L = need_gpu()
    rng = np.random.default_rng(40)
    H, D = (8, 128) if dt == "f32" else (64, 256)
    B, Tq, W, m = 2, 5, 128, (4 if kind == "csa" else 128)
    q_pos0 = 3000 if kind == "csa" else 20000
    N_cap = (q_pos0 + Tq) // m + 3
    k = 300
    cast = WL.bf16_exact if dt == "bf16" else (lambda a: a)
    q, E, win, sink = _attend_case(rng, B, Tq, H, D, N_cap, W, sharp, cast)
    up = dev_bf16 if dt == "bf16" else dev_f32
    dtc = L.BF16 if dt == "bf16" else L.F32
    scale = 1 / math.sqrt(D)
    out = torch.empty((B, Tq, H, D), dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device=DEV)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=DEV)
    if kind == "csa":
        idx = np.full((B, Tq, k), -1, np.int32)
        for b in range(B):
            for t in range(Tq):
                nv = O.n_visible(q_pos0 + t, m)
                sel = rng.choice(nv, size=min(k - 7, nv), replace=False)
                idx[b, t, :len(sel)] = np.sort(sel)
        L.csa_attend(dtc, dtc, up(q), up(E), torch.from_numpy(idx).to(DEV), up(win), dev_f32(sink), out,
                     m=m, W=W, q_pos0=q_pos0, scale=scale, flags=L.INV_ROPE, rope_dims=64, lse_out=lse)
    else:
        L.hca_attend(dtc, dtc, up(q), up(E), up(win), dev_f32(sink), out, m=m, W=W, q_pos0=q_pos0,
                     scale=scale, flags=L.INV_ROPE, rope_dims=64, lse_out=lse)
    torch.cuda.synchronize()
    got, got_lse = host(out), lse.cpu().numpy()
    tol = 1e-4 if dt == "f32" else 2e-2
    for b in range(B):
        if kind == "csa":
            ref, rl = O.csa_attend(q[b], E[b], idx[b], win[b], sink, scale, q_pos0, W, True, 10000.0, 64)
        else:
            ref, rl = O.hca_attend(q[b], E[b], m, win[b], sink, scale, q_pos0, W, True, 10000.0, 64)
        row_tol_check(got[b], ref, tol, f"{kind} {dt} sharp={sharp}")
        np.testing.assert_allclose(got_lse[b], rl, atol=1e-4 if dt == "f32" else 2e-2)


def test_attend_window_clipped_and_no_entries():
    # queries at positions 0..9: fewer window rows than W, no visible entries
    L = need_gpu()
    rng = np.random.default_rng(41)
    B, Tq, H, D, W, m = 1, 10, 16, 128, 128, 4
    q, E, win, sink = _attend_case(rng, B, Tq, H, D, 4, W, 20.0, WL.bf16_exact)
    out = torch.empty((B, Tq, H, D), dtype=torch.bfloat16, device=DEV)
    idx = np.full((B, Tq, 8), -1, np.int32)
    idx[0, 3:, 0] = 0                          # entry 0 visible from position 3 on
    idx[0, 7:, 1] = 1
    L.csa_attend(L.BF16, L.BF16, dev_bf16(q), dev_bf16(E), torch.from_numpy(idx).to(DEV), dev_bf16(win),
                 dev_f32(sink), out, m=m, W=W, q_pos0=0, scale=1 / math.sqrt(D))
    torch.cuda.synchronize()
    ref, _ = O.csa_attend(q[0], E[0], idx[0], win[0], sink, 1 / math.sqrt(D), 0, W)
    row_tol_check(host(out)[0], ref, 2e-2, "clipped window")


@pytest.mark.parametrize("kind", ["csa", "hca"])
@pytest.mark.parametrize("Tq,H", [(1, 64), (4, 16), (4, 64)])
@pytest.mark.parametrize("q_pos0", [45, 60001])
def test_attend_512_short_ragged_lists(kind, Tq, H, q_pos0):
    # bf16 rows of 512 channels, few queries and a few hundred rows each (the
    # decode shapes): row counts that are not multiples of the 32-row tile,
    # q_pos0 = 45 clips the window and leaves few visible entries, CSA lists
    # carry absent (-1) entries in any order, 16 heads leave 3 of 4 waves idle.
    L = need_gpu()
    rng = np.random.default_rng(44 + Tq + H + (q_pos0 > 100))
    B, D, W = 3, 512, 128
    m = 4 if kind == "csa" else 128
    N_cap = (q_pos0 + Tq) // m + 2
    k = 517
    q, E, win, sink = _attend_case(rng, B, Tq, H, D, N_cap, W, 4.0, WL.bf16_exact)
    scale = 1 / math.sqrt(D)
    out = torch.empty((B, Tq, H, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=DEV)
    say(f"short ragged lists {kind} Tq={Tq} H={H} q_pos0={q_pos0}")
    if kind == "csa":
        idx = np.full((B, Tq, k), -1, np.int32)
        for b in range(B):
            for t in range(Tq):
                nv = O.n_visible(q_pos0 + t, m)
                sel = rng.choice(nv, size=min(k - 5, nv), replace=False)
                idx[b, t, :len(sel)] = sel                      # any order; -1 tail
        L.csa_attend(L.BF16, L.BF16, dev_bf16(q), dev_bf16(E), torch.from_numpy(idx).to(DEV), dev_bf16(win),
                     dev_f32(sink), out, m=m, W=W, q_pos0=q_pos0, scale=scale, flags=L.INV_ROPE, rope_dims=64,
                     lse_out=lse)
    else:
        L.hca_attend(L.BF16, L.BF16, dev_bf16(q), dev_bf16(E), dev_bf16(win), dev_f32(sink), out, m=m, W=W,
                     q_pos0=q_pos0, scale=scale, flags=L.INV_ROPE, rope_dims=64, lse_out=lse)
    torch.cuda.synchronize()
    got, got_lse = host(out), lse.cpu().numpy()
    for b in range(B):
        if kind == "csa":
            ref, rl = O.csa_attend(q[b], E[b], idx[b], win[b], sink, scale, q_pos0, W, True, 10000.0, 64)
        else:
            ref, rl = O.hca_attend(q[b], E[b], m, win[b], sink, scale, q_pos0, W, True, 10000.0, 64)
        row_tol_check(got[b], ref, 2e-2, f"short lists {kind} Tq={Tq} H={H} q_pos0={q_pos0} b={b}")
        np.testing.assert_allclose(got_lse[b], rl, atol=2e-2)


@pytest.mark.parametrize("Tq", [1, 16])
def test_attend_mixed_kv_matches_oracle(Tq):
    # 16 queries x 128 heads: one split per query (output written by the kernel)
    L = need_gpu()
    rng = np.random.default_rng(42)
    B, H, D, W, m, k = 2, 128, 512, 128, 4, 200
    q_pos0 = 4 * 3000
    N_cap = (q_pos0 + Tq) // m + 1
    q = WL.bf16_exact((rng.standard_normal((B, Tq, H, D)) * 10 / np.sqrt(D)).astype(np.float32))
    Esrc = (rng.standard_normal((B, N_cap, D)) / np.sqrt(D)).astype(np.float32)
    wsrc = (rng.standard_normal((B, W - 1 + Tq, D)) / np.sqrt(D)).astype(np.float32)
    sink = rng.standard_normal(H).astype(np.float32)
    Eq = torch.empty((B, N_cap, D + 64), dtype=torch.uint8, device=DEV)
    Es = torch.empty((B, N_cap), dtype=torch.float32, device=DEV)
    Wq = torch.empty((B, W - 1 + Tq, D + 64), dtype=torch.uint8, device=DEV)
    Ws = torch.empty((B, W - 1 + Tq), dtype=torch.float32, device=DEV)
    L.lca_quantize_rows(L.KV_MIXED, dev_f32(Esrc), Eq, Es)
    L.lca_quantize_rows(L.KV_MIXED, dev_f32(wsrc), Wq, Ws)
    idx = np.stack([np.stack([np.sort(rng.choice(3000, size=k, replace=False)) for _ in range(Tq)])
                    for _ in range(B)]).astype(np.int32)
    out = torch.empty((B, Tq, H, D), dtype=torch.bfloat16, device=DEV)
    L.csa_attend(L.BF16, L.KV_MIXED, dev_bf16(q), Eq, torch.from_numpy(idx).to(DEV), Wq, dev_f32(sink), out,
                 m=m, W=W, q_pos0=q_pos0, scale=1 / math.sqrt(D), kv_scale=Es, win_scale=Ws,
                 flags=L.INV_ROPE, rope_dims=64)
    torch.cuda.synchronize()
    for b in range(B):
        Ed = O.kv_mixed_decode(*O.kv_mixed_quantize(Esrc[b], 64))
        Wd = O.kv_mixed_decode(*O.kv_mixed_quantize(wsrc[b], 64))
        ref, _ = O.csa_attend(q[b], Ed, idx[b], Wd, sink, 1 / math.sqrt(D), q_pos0, W, True, 10000.0, 64)
        row_tol_check(host(out)[b], ref, 2e-2, "mixed kv")


@pytest.mark.parametrize("Tq", [1, 32])
def test_attend_mixed_logit_ramp_exact_recompute(Tq):
    # KV_MIXED rows, 128 heads (32 per wave): logits that climb by hundreds
    # along the entries overflow the in-kernel headroom, so flagged splits are
    # recomputed exactly from the stored fp8 / bf16 rows (1 query: 2 splits of
    # 512 rows, merged by the combine; 32 queries: one split, fixed up after).
    L = need_gpu()
    rng = np.random.default_rng(45 + Tq)
    B, H, D, W, m = 1, 128, 512, 128, 128
    q_pos0 = m * 600
    N_cap = (q_pos0 + Tq) // m + 1
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    ramp = np.linspace(-1.0, 1.0, N_cap)
    Esrc = (ramp[:, None] * u[None, :] + 0.05 * rng.standard_normal((N_cap, D)) / np.sqrt(D)).astype(np.float32)
    wsrc = (rng.standard_normal((W - 1 + Tq, D)) / np.sqrt(D)).astype(np.float32)
    sharp = np.geomspace(1.0, 4000.0, H)
    q = (sharp[None, :, None] * (u[None, None, :] + 0.1 * rng.standard_normal((Tq, H, D)) / np.sqrt(D)))
    q = WL.bf16_exact((q * np.sqrt(D)).astype(np.float32))[None]
    sink = rng.standard_normal(H).astype(np.float32)
    Eq = torch.empty((1, N_cap, D + 64), dtype=torch.uint8, device=DEV)
    Es = torch.empty((1, N_cap), dtype=torch.float32, device=DEV)
    Wq = torch.empty((1, W - 1 + Tq, D + 64), dtype=torch.uint8, device=DEV)
    Ws = torch.empty((1, W - 1 + Tq), dtype=torch.float32, device=DEV)
    L.lca_quantize_rows(L.KV_MIXED, dev_f32(Esrc[None]), Eq, Es)
    L.lca_quantize_rows(L.KV_MIXED, dev_f32(wsrc[None]), Wq, Ws)
    out = torch.empty((B, Tq, H, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=DEV)
    say(f"ramp mixed hca Tq={Tq} entries={O.n_visible(q_pos0, m)}")
    L.hca_attend(L.BF16, L.KV_MIXED, dev_bf16(q), Eq, Wq, dev_f32(sink), out, m=m, W=W, q_pos0=q_pos0,
                 scale=1 / math.sqrt(D), kv_scale=Es, win_scale=Ws, flags=L.INV_ROPE, rope_dims=64, lse_out=lse)
    torch.cuda.synchronize()
    Ed = O.kv_mixed_decode(*O.kv_mixed_quantize(Esrc, 64))
    Wd = O.kv_mixed_decode(*O.kv_mixed_quantize(wsrc, 64))
    ref, rl = O.hca_attend(q[0], Ed, m, Wd, sink, 1 / math.sqrt(D), q_pos0, W, True, 10000.0, 64)
    assert np.ptp(rl) > 100.0, "the case must span a wide logit range"
    row_tol_check(host(out)[0], ref, 2e-2, f"mixed ramp Tq={Tq}")
    lse_err = np.abs(lse.cpu().numpy()[0] - rl) / np.maximum(1.0, np.abs(rl))
    assert lse_err.max() <= 2e-2, f"lse relative error {lse_err.max()}"


@pytest.mark.parametrize("kind,D,Tq,H", [("hca", 512, 1, 64), ("csa", 512, 1, 64), ("csa", 256, 1, 64),
                                          ("hca", 512, 16, 128), ("csa", 256, 16, 128)])
def test_attend_logit_ramp_exact_recompute(kind, D, Tq, H):
    # Logits that climb by hundreds along the entries: inside one split, later
    # tiles exceed the first tile's max by far more than the in-kernel headroom,
    # so those splits must be recomputed exactly when the partials are merged.
    # Heads get different sharpness, so flagged and unflagged splits mix. With
    # 16 queries and 128 heads the plan has one split per query: outputs are
    # written by the attention kernel itself and flagged heads fixed up after.
    L = need_gpu()
    rng = np.random.default_rng(43)
    B, W = 1, 128
    m = 4 if kind == "csa" else 128
    q_pos0 = 4 * 2500 if kind == "csa" else 128 * 600
    N_cap = (q_pos0 + Tq) // m + 1
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    ramp = np.linspace(-1.0, 1.0, N_cap)
    E = WL.bf16_exact((ramp[:, None] * u[None, :] + 0.05 * rng.standard_normal((N_cap, D)) / np.sqrt(D))
                      .astype(np.float32))[None]
    sharp = np.geomspace(1.0, 4000.0, H)
    q = (sharp[None, :, None] * (u[None, None, :] + 0.1 * rng.standard_normal((Tq, H, D)) / np.sqrt(D)))
    q = WL.bf16_exact((q * np.sqrt(D)).astype(np.float32))[None]
    win = WL.bf16_exact((rng.standard_normal((B, W - 1 + Tq, D)) / np.sqrt(D)).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    scale = 1 / math.sqrt(D)
    out = torch.empty((B, Tq, H, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=DEV)
    if kind == "csa":
        nv = O.n_visible(q_pos0, m)
        idx = np.stack([np.sort(rng.choice(nv, size=900, replace=False)) for _ in range(Tq)]).astype(np.int32)[None]
        say(f"ramp csa D={D} Tq={Tq} H={H} k=900 nv={nv}")
        L.csa_attend(L.BF16, L.BF16, dev_bf16(q), dev_bf16(E), torch.from_numpy(idx).to(DEV), dev_bf16(win),
                     dev_f32(sink), out, m=m, W=W, q_pos0=q_pos0, scale=scale, flags=L.INV_ROPE, rope_dims=64,
                     lse_out=lse)
        ref, rl = O.csa_attend(q[0], E[0], idx[0], win[0], sink, scale, q_pos0, W, True, 10000.0, 64)
    else:
        say(f"ramp hca D={D} Tq={Tq} H={H} entries={O.n_visible(q_pos0, m)}")
        L.hca_attend(L.BF16, L.BF16, dev_bf16(q), dev_bf16(E), dev_bf16(win), dev_f32(sink), out, m=m, W=W,
                     q_pos0=q_pos0, scale=scale, flags=L.INV_ROPE, rope_dims=64, lse_out=lse)
        ref, rl = O.hca_attend(q[0], E[0], m, win[0], sink, scale, q_pos0, W, True, 10000.0, 64)
    torch.cuda.synchronize()
    assert np.ptp(rl) > 100.0, "the case must span a wide logit range"
    row_tol_check(host(out)[0], ref, 2e-2, f"ramp {kind} D={D} Tq={Tq} H={H}")
    lse_err = np.abs(lse.cpu().numpy()[0] - rl) / np.maximum(1.0, np.abs(rl))
    assert lse_err.max() <= 2e-2, f"lse relative error {lse_err.max()}"
