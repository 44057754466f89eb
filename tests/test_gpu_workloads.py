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
