"""End-to-end parity on the stated workloads, at their full sizes, in the
launch configuration the benchmark times. The oracle checks sampled sequences
(and sampled queries for prefill); batch invariance and run-to-run
determinism are checked bit for bit."""

import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import (DEV, check_topk_set, dev_bf16, dev_f32, host, need_gpu, row_tol_check, say)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# workload 1: one CSA layer forward in fp32 (1024 causal tokens from position 0)
# ---------------------------------------------------------------------------

def _csa_layer_gpu(L, d):
    B, T, D, m, dI, H_I, k = d["B"], d["T"], d["D"], d["m"], d["d_I"], d["H_I"], d["k"]
    E = torch.empty((B, T // m, D), dtype=torch.float32, device=DEV)
    KI = torch.empty((B, T // m, dI), dtype=torch.float32, device=DEV)
    L.csa_compress(L.F32, L.F32, dev_f32(d["cb"]), dev_f32(d["zb"]), m, ca=dev_f32(d["ca"]),
                   za=dev_f32(d["za"]), pos0=0, flags=L.NORM | L.ROPE, norm_w=dev_f32(d["norm_w"]),
                   eps=d["eps"], rope_base=d["rope_base"], rope_dims=d["rope_dims"], out=E)
    L.csa_compress(L.F32, L.F32, dev_f32(d["icb"]), dev_f32(d["izb"]), m, ca=dev_f32(d["ica"]),
                   za=dev_f32(d["iza"]), pos0=0, out=KI)
    idx = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    L.csa_index_topk(L.F32, dev_f32(d["qI"]), dev_f32(d["w"]), KI, idx, m=m, k=k, q_pos0=0)
    out = torch.empty((B, T, d["H"], D), dtype=torch.float32, device=DEV)
    L.csa_attend(L.F32, L.F32, dev_f32(d["q"]), E, idx, dev_f32(d["win"]), dev_f32(d["sink"]), out, m=m,
                 W=d["W"], q_pos0=0, scale=1 / math.sqrt(D), flags=L.INV_ROPE, rope_dims=d["rope_dims"])
    torch.cuda.synchronize()
    return E, KI, idx, out


@pytest.mark.parametrize("sharp", [1.0, 40.0])
def test_csa_layer_fp32_end_to_end(sharp):
    L = need_gpu()
    d = WL.make_csa_layer(sharp=sharp)
    say(f"csa layer fp32 sharp={sharp}")
    E, KI, idx, out = _csa_layer_gpu(L, d)
    m, R = d["m"], d["rope_dims"]
    Eo = O.compress_epilogue(O.compress_sequence(d["cb"][0], d["zb"][0], m, d["ca"][0], d["za"][0]),
                             0, m, d["norm_w"], d["eps"], d["rope_base"], R)
    Ko = O.compress_sequence(d["icb"][0], d["izb"][0], m, d["ica"][0], d["iza"][0])
    row_tol_check(host(E)[0], Eo, 1e-5, "entries")
    row_tol_check(host(KI)[0], Ko, 1e-5, "indexer keys")
    idx_h = idx.cpu().numpy()[0]
    amb = 0
    for t in range(d["T"]):
        s = O.index_scores(d["qI"][0, t], d["w"][0, t], Ko, O.n_visible(t, m))
        amb += check_topk_set(idx_h[t], s, d["k"])
    # conditional parity: oracle attention with the GPU's selection
    ref, _ = O.csa_attend(d["q"][0], Eo, idx_h, d["win"][0], d["sink"], 1 / math.sqrt(d["D"]), 0, d["W"],
                          True, d["rope_base"], R)
    w = row_tol_check(host(out)[0], ref, 1e-4, "csa layer out")
    say(f"  ambiguous top-k entries {amb}, worst row error {w:.2e}")


# ---------------------------------------------------------------------------
# workload 2: CSA decode, B = 16 at 131072 tokens (bf16)
# ---------------------------------------------------------------------------

def _csa_decode_gpu(L, d, reps=1):
    B, H, D, m, k = d["B"], d["H"], d["D"], d["m"], d["k"]
    t = {n: dev_bf16(d[n]) for n in ("E", "kI", "q", "qI", "win")}
    t["w"] = dev_f32(d["w"])
    t["sink"] = dev_f32(d["sink"])
    outs = []
    for _ in range(reps):
        idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
        out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=DEV)
        L.csa_index_topk(L.BF16, t["qI"], t["w"], t["kI"], idx, m=m, k=k, q_pos0=d["q_pos0"])
        L.csa_attend(L.BF16, L.BF16, t["q"], t["E"], idx, t["win"], t["sink"], out, m=m, W=d["W"],
                     q_pos0=d["q_pos0"], scale=1 / math.sqrt(D), flags=L.INV_ROPE, rope_dims=64)
        outs.append((idx, out))
    torch.cuda.synchronize()
    return outs


def _check_csa_decode_seq(d, b, idx_h, out_h):
    m, k, D = d["m"], d["k"], d["D"]
    nv = O.n_visible(d["q_pos0"], m)
    s = O.index_scores(d["qI"][b, 0], d["w"][b, 0], d["kI"][b], nv)
    amb = check_topk_set(idx_h, s, k)
    ref, _ = O.csa_attend_query(d["q"][b, 0], d["E"][b], idx_h, d["win"][b], d["sink"], 1 / math.sqrt(D),
                                d["q_pos0"], d["q_pos0"], d["W"], True, 10000.0, 64)
    w = row_tol_check(out_h, ref, 2e-2, f"csa decode seq {b}")
    return amb, w


@pytest.mark.parametrize("sharp", [1.0, 20.0])
def test_csa_decode_full_size(sharp):
    L = need_gpu()
    say(f"csa decode B=16 ctx=131072 sharp={sharp}: generating")
    d = WL.make_csa_decode(sharp=sharp)
    say("  running")
    (idx, out), = _csa_decode_gpu(L, d)
    idx_h, out_h = idx.cpu().numpy(), host(out)
    for b in (0, 9, 15):
        amb, w = _check_csa_decode_seq(d, b, idx_h[b, 0], out_h[b, 0])
        say(f"  seq {b}: ambiguous {amb}, worst row error {w:.2e}")


def test_csa_decode_batch_invariant_and_deterministic():
    L = need_gpu()
    say("csa decode batch invariance: B=16 vs B=1")
    d = WL.make_csa_decode(ctx=65536)
    (i1, o1), (i2, o2) = _csa_decode_gpu(L, d, reps=2)
    assert torch.equal(i1, i2) and torch.equal(o1, o2), "not deterministic"
    d1 = WL.make_csa_decode(ctx=65536, B=16, seqs=[11])
    d1["B"] = 1
    (i3, o3), = _csa_decode_gpu(L, d1)
    assert torch.equal(i1[11], i3[0]), "index set depends on the batch"
    assert torch.equal(o1[11], o3[0]), "output depends on the batch"


# ---------------------------------------------------------------------------
# workload 3: HCA decode, B = 8 at 1048576 tokens (8192 entries, 128 heads)
# ---------------------------------------------------------------------------

def _hca_decode_gpu(L, d, reps=1):
    B, H, D = d["B"], d["H"], d["D"]
    t = {n: dev_bf16(d[n]) for n in ("E", "q", "win")}
    sink = dev_f32(d["sink"])
    outs = []
    for _ in range(reps):
        out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((B, 1, H), dtype=torch.float32, device=DEV)
        L.hca_attend(L.BF16, L.BF16, t["q"], t["E"], t["win"], sink, out, m=d["m"], W=d["W"],
                     q_pos0=d["q_pos0"], scale=1 / math.sqrt(D), flags=L.INV_ROPE, rope_dims=64, lse_out=lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("sharp", [1.0, 20.0])
def test_hca_decode_full_size(sharp):
    L = need_gpu()
    say(f"hca decode B=8 ctx=1048576 sharp={sharp}")
    d = WL.make_hca_decode(sharp=sharp)
    (out, lse), = _hca_decode_gpu(L, d)
    out_h, lse_h = host(out), lse.cpu().numpy()
    for b in (0, 5):
        ref, rl = O.hca_attend(d["q"][b], d["E"][b], d["m"], d["win"][b], d["sink"], 1 / math.sqrt(d["D"]),
                               d["q_pos0"], d["W"], True, 10000.0, 64)
        w = row_tol_check(out_h[b], ref, 2e-2, f"hca seq {b}")
        np.testing.assert_allclose(lse_h[b], rl, atol=2e-2)
        say(f"  seq {b}: worst row error {w:.2e}")


def test_hca_decode_batch_invariant_and_deterministic():
    L = need_gpu()
    d = WL.make_hca_decode(ctx=1048576 // 4)
    (o1, l1), (o2, l2) = _hca_decode_gpu(L, d, reps=2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    d1 = WL.make_hca_decode(ctx=1048576 // 4, seqs=[6])
    d1["B"] = 1
    (o3, l3), = _hca_decode_gpu(L, d1)
    assert torch.equal(o1[6], o3[0]) and torch.equal(l1[6], l3[0])


# ---------------------------------------------------------------------------
# workload 5: mixed-precision CSA + HCA layer pair, decode at 1048576 tokens.
# fp32 sources are quantised by the path itself (KV_MIXED rows, MXFP4 indexer
# operands); index scores are rounded to bf16 before top-k. Two of the 64
# sequences are generated (each regenerates alone; kernels are batch-invariant).
# ---------------------------------------------------------------------------

def _quant(L, dt, x, D_out, n_scale):
    flat = x.reshape(-1, x.shape[-1])
    out = torch.empty((flat.shape[0], D_out), dtype=torch.uint8, device=DEV)
    if dt == L.KV_MIXED:
        sc = torch.empty((flat.shape[0],), dtype=torch.float32, device=DEV)
    else:
        sc = torch.empty((flat.shape[0], n_scale), dtype=torch.uint8, device=DEV)
    L.lca_quantize_rows(dt, dev_f32(flat), out, sc)
    return out.reshape(x.shape[:-1] + (D_out,)), sc.reshape(x.shape[:-1] + tuple(sc.shape[1:]))


def test_mixed_pair_full_context():
    L = need_gpu()
    seqs = [0, 63]
    say("mixed pair B=64 (sequences 0, 63) ctx=1048576: generating")
    d = WL.make_mixed_pair(seqs=seqs)
    B, H, D, m, m2, k, W = len(seqs), d["H"], d["D"], d["m"], d["m2"], d["k"], d["W"]
    q_pos0 = d["q_pos0"]
    say("  quantising on the GPU")
    Eq, Es = _quant(L, L.KV_MIXED, d["E"], D + 64, 0)
    Wq, Ws = _quant(L, L.KV_MIXED, d["win"], D + 64, 0)
    E2q, E2s = _quant(L, L.KV_MIXED, d["E2"], D + 64, 0)
    W2q, W2s = _quant(L, L.KV_MIXED, d["win2"], D + 64, 0)
    kc, ks = _quant(L, L.MXFP4, d["kI"], d["d_I"] // 2, d["d_I"] // 32)
    qc, qs = _quant(L, L.MXFP4, d["qI"], d["d_I"] // 2, d["d_I"] // 32)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=DEV)
    out2 = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=DEV)
    scale = 1 / math.sqrt(D)
    say("  running index_topk (MXFP4, bf16 scores), csa_attend and hca_attend (KV_MIXED)")
    L.csa_index_topk(L.MXFP4, qc, dev_f32(d["w"]), kc, idx, m=m, k=k, q_pos0=q_pos0, d_I=d["d_I"],
                     qI_scale=qs, kI_scale=ks, flags=L.SCORE_BF16)
    L.csa_attend(L.BF16, L.KV_MIXED, dev_bf16(d["q"]), Eq, idx, Wq, dev_f32(d["sink"]), out, m=m, W=W,
                 q_pos0=q_pos0, scale=scale, kv_scale=Es, win_scale=Ws, flags=L.INV_ROPE, rope_dims=64)
    L.hca_attend(L.BF16, L.KV_MIXED, dev_bf16(d["q2"]), E2q, W2q, dev_f32(d["sink2"]), out2, m=m2, W=W,
                 q_pos0=q_pos0, scale=scale, kv_scale=E2s, win_scale=W2s, flags=L.INV_ROPE, rope_dims=64)
    torch.cuda.synchronize()
    idx_h, o_h, o2_h = idx.cpu().numpy(), host(out), host(out2)
    nv = O.n_visible(q_pos0, m)
    for b in range(B):
        say(f"  oracle, sequence {seqs[b]}")
        qd = O.mxfp4_decode(*O.mxfp4_quantize(d["qI"][b, 0]))
        kd = O.mxfp4_decode(*O.mxfp4_quantize(d["kI"][b]))
        s = O.index_scores(qd, d["w"][b, 0], kd, nv)
        amb = check_topk_set(idx_h[b, 0], s, k, bf16_scores=True)
        sel = idx_h[b, 0][idx_h[b, 0] >= 0]
        Esel = O.kv_mixed_decode(*O.kv_mixed_quantize(d["E"][b][sel], 64))
        Wd = O.kv_mixed_decode(*O.kv_mixed_quantize(d["win"][b], 64))
        ref, _ = O.csa_attend_query(d["q"][b, 0], Esel, np.arange(len(sel)), Wd, d["sink"], scale, q_pos0,
                                    q_pos0, W, True, 10000.0, 64)
        w1 = row_tol_check(o_h[b, 0], ref, 2e-2, f"mixed csa seq {seqs[b]}")
        E2d = O.kv_mixed_decode(*O.kv_mixed_quantize(d["E2"][b], 64))
        W2d = O.kv_mixed_decode(*O.kv_mixed_quantize(d["win2"][b], 64))
        ref2, _ = O.hca_attend_query(d["q2"][b, 0], E2d, O.n_visible(q_pos0, m2), W2d, d["sink2"], scale,
                                     q_pos0, q_pos0, W, True, 10000.0, 64)
        w2 = row_tol_check(o2_h[b, 0], ref2, 2e-2, f"mixed hca seq {seqs[b]}")
        say(f"    ambiguous top-k entries {amb}, worst row error csa {w1:.2e} hca {w2:.2e}")


# ---------------------------------------------------------------------------
# workload 4: CSA chunked prefill, 4096 new tokens after 1048576 (B = 1,
# 262144 + 1024 entries, 128 heads, k = 1024). The GPU runs every query; the
# oracle checks sampled query rows (the others are left zero by the generator).
# ---------------------------------------------------------------------------

PREFILL_ROWS = [0, 1, 2, 3, 4, 5, 6, 7, 127, 128, 129, 511, 512, 1023, 1024, 2047, 2048, 3000,
                4088, 4091, 4092, 4093, 4094, 4095]


def _csa_prefill_gpu(L, d):
    m, D, dI, Tq, N0 = d["m"], d["D"], d["d_I"], d["Tq"], d["N0"]
    N_cap = d["N_cap"]
    E = torch.empty((1, N_cap, D), dtype=torch.bfloat16, device=DEV)
    KI = torch.empty((1, N_cap, dI), dtype=torch.bfloat16, device=DEV)
    E[:, :N0] = dev_bf16(d["E_prefix"])
    KI[:, :N0] = dev_bf16(d["kI_prefix"])
    # the new tokens' entries land after the prefix, inside the same cache
    L.csa_compress(L.BF16, L.BF16, dev_bf16(d["cb"]), dev_f32(d["zb"]), m, ca=dev_bf16(d["ca"]),
                   za=dev_f32(d["za"]), prev_ca=dev_bf16(d["prev_ca"]), prev_za=dev_f32(d["prev_za"]),
                   pos0=d["pos0"], flags=L.NORM | L.ROPE, norm_w=dev_f32(d["norm_w"]), eps=d["eps"],
                   rope_base=d["rope_base"], rope_dims=d["rope_dims"], out=E[:, N0:], out_rows=N_cap)
    L.csa_compress(L.BF16, L.BF16, dev_bf16(d["icb"]), dev_f32(d["izb"]), m, ca=dev_bf16(d["ica"]),
                   za=dev_f32(d["iza"]), prev_ca=dev_bf16(d["iprev_ca"]), prev_za=dev_f32(d["iprev_za"]),
                   pos0=d["pos0"], out=KI[:, N0:], out_rows=N_cap)
    idx = torch.empty((1, Tq, d["k"]), dtype=torch.int32, device=DEV)
    L.csa_index_topk(L.BF16, dev_bf16(d["qI"]), dev_f32(d["w"]), KI, idx, m=m, k=d["k"], q_pos0=d["q_pos0"])
    out = torch.empty((1, Tq, d["H"], D), dtype=torch.bfloat16, device=DEV)
    L.csa_attend(L.BF16, L.BF16, dev_bf16(d["q"]), E, idx, dev_bf16(d["win"]), dev_f32(d["sink"]), out, m=m,
                 W=d["W"], q_pos0=d["q_pos0"], scale=1 / math.sqrt(D), flags=L.INV_ROPE,
                 rope_dims=d["rope_dims"])
    torch.cuda.synchronize()
    return E, KI, idx, out


def test_csa_prefill_full_size_sampled_queries():
    L = need_gpu()
    say("csa prefill Tq=4096 ctx=1048576 H=128 k=1024: generating")
    d = WL.make_csa_prefill(q_rows=PREFILL_ROWS)
    m, D, N0, R = d["m"], d["D"], d["N0"], d["rope_dims"]
    say("  running compress, index_topk, attend")
    E, KI, idx, out = _csa_prefill_gpu(L, d)
    say("  oracle")
    E_new = O.compress_epilogue(O.compress_sequence(d["cb"][0], d["zb"][0], m, d["ca"][0], d["za"][0],
                                                    d["prev_ca"][0], d["prev_za"][0]),
                                d["pos0"], m, d["norm_w"], d["eps"], d["rope_base"], R)
    K_new = O.compress_sequence(d["icb"][0], d["izb"][0], m, d["ica"][0], d["iza"][0], d["iprev_ca"][0],
                                d["iprev_za"][0])
    row_tol_check(host(E)[0, N0:], E_new, 1e-2, "prefill entries")
    row_tol_check(host(KI)[0, N0:], K_new, 1e-2, "prefill indexer keys")
    # the cache as stored (bf16), from the oracle's own entries
    E_all = np.concatenate([d["E_prefix"][0], O.bf16_round(E_new)])
    K_all = np.concatenate([d["kI_prefix"][0], O.bf16_round(K_new)])
    idx_h, out_h = idx.cpu().numpy()[0], host(out)[0]
    worst, amb = 0.0, 0
    for t in PREFILL_ROWS:
        p = d["q_pos0"] + t
        s = O.index_scores(d["qI"][0, t], d["w"][0, t], K_all, O.n_visible(p, m))
        amb += check_topk_set(idx_h[t], s, d["k"])
        ref, _ = O.csa_attend_query(d["q"][0, t], E_all, idx_h[t], d["win"][0], d["sink"], 1 / math.sqrt(D), p,
                                    d["q_pos0"], d["W"], True, d["rope_base"], R)
        worst = max(worst, row_tol_check(out_h[t], ref, 2e-2, f"prefill query {t}"))
    say(f"  {len(PREFILL_ROWS)} sampled queries: ambiguous top-k entries {amb}, worst row error {worst:.2e}")
