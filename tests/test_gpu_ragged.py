"""Ragged batches on the GPU: every sequence of a batch at its own position
(q_pos[b]), as a decode batch drawn from per-request KV caches ([kwkr] §4.4,
State Cache and Classical KV Cache). Each sequence is checked against the
oracle at its own position, and against calls that hold that sequence alone:
with the same bound the result is bitwise the same (batch invariance), and a
uniform call at the sequence's own position gives the same bits whenever its
split plan is the same one."""

import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, check_topk_set, dev_bf16, dev_f32, host, need_gpu, row_tol_check, say

pytestmark = pytest.mark.gpu


def _qp(vals):
    return torch.tensor(vals, dtype=torch.int64, device=DEV)


# ---------------------------------------------------------------------------
# indexer scores + top-k
# ---------------------------------------------------------------------------

_INDEX_CASES = {
    # B, Tq, H_I, k, bound, positions, N_cap
    # one query per sequence: an empty list (position 0), a list shorter than
    # k, a list at the bound and one between
    "decode": (4, 1, 4, 256, 4 * 5000 + 2, [4 * 5000 + 2, 0, 37, 4 * 2999 + 3], 5003),
    # 70 queries per sequence take the key-tiled scoring path
    "tiled": (3, 70, 4, 50, 700, [700, 3, 311], (700 + 70) // 4),
    # lists beyond one register round take the two-read select; the short one
    # (20000 entries) goes through the same kernel in one round
    "long": (2, 1, 4, 1024, 4 * 100000 + 1, [4 * 20000 + 3, 4 * 100000 + 1], 100003),
}


@pytest.mark.parametrize("case", list(_INDEX_CASES))
@pytest.mark.parametrize("bf16_scores", [False, True])
def test_index_topk_ragged(case, bf16_scores):
    L = need_gpu()
    B, Tq, H_I, k, bound, pos, N_cap = _INDEX_CASES[case]
    d_I, m = 128, 4
    rng = np.random.default_rng(90 + len(case) + bf16_scores)
    qI = WL.bf16_exact(rng.standard_normal((B, Tq, H_I, d_I)).astype(np.float32) / np.sqrt(d_I))
    kI = rng.standard_normal((B, N_cap, d_I)).astype(np.float32) / np.sqrt(d_I)
    kI[:, ::97] *= 4
    kI = WL.bf16_exact(kI)
    w = (rng.standard_normal((B, Tq, H_I)) / np.sqrt(H_I)).astype(np.float32)
    flags = L.SCORE_BF16 if bf16_scores else 0
    say(f"ragged index_topk {case} bf16_scores={bf16_scores} positions={pos} bound={bound}")
    q_d, w_d, k_d = dev_bf16(qI), dev_f32(w), dev_bf16(kI)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    sco = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    L.csa_index_topk(L.BF16, q_d, w_d, k_d, idx, m=m, k=k, q_pos0=bound, flags=flags, score_out=sco,
                     q_pos=_qp(pos))
    torch.cuda.synchronize()
    idx_h, sco_h = idx.cpu().numpy(), sco.cpu().numpy()
    for b in range(B):
        for t in range(Tq):
            nv = O.n_visible(pos[b] + t, m)
            s = O.index_scores(qI[b, t], w[b, t], kI[b], min(nv, N_cap))
            check_topk_set(idx_h[b, t], s, k, bf16_scores=bf16_scores)
            sel = idx_h[b, t][idx_h[b, t] >= 0]
            assert np.all(np.diff(sel) > 0), "indices not increasing"
        # the sequence alone, uniform call at its own position: same bits
        i1 = torch.empty((1, Tq, k), dtype=torch.int32, device=DEV)
        s1 = torch.empty((1, Tq, k), dtype=torch.float32, device=DEV)
        L.csa_index_topk(L.BF16, q_d[b:b + 1], w_d[b:b + 1], k_d[b:b + 1], i1, m=m, k=k, q_pos0=pos[b],
                         flags=flags, score_out=s1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(i1.cpu().numpy()[0], idx_h[b])
        valid = idx_h[b] >= 0
        np.testing.assert_array_equal(s1.cpu().numpy()[0][valid], sco_h[b][valid])


def test_index_topk_ragged_positions_clamped():
    # positions outside [0, bound] are clamped on the device: -5 reads as 0
    # (nothing visible) and bound + 1000 as the bound
    L = need_gpu()
    rng = np.random.default_rng(97)
    B, Tq, H_I, d_I, m, k, bound = 2, 1, 4, 128, 4, 64, 4 * 600
    N_cap = 601
    qI = WL.bf16_exact(rng.standard_normal((B, Tq, H_I, d_I)).astype(np.float32) / np.sqrt(d_I))
    kI = WL.bf16_exact(rng.standard_normal((B, N_cap, d_I)).astype(np.float32) / np.sqrt(d_I))
    w = (rng.standard_normal((B, Tq, H_I)) / np.sqrt(H_I)).astype(np.float32)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    say("ragged index_topk clamped positions")
    L.csa_index_topk(L.BF16, dev_bf16(qI), dev_f32(w), dev_bf16(kI), idx, m=m, k=k, q_pos0=bound,
                     q_pos=_qp([-5, bound + 1000]))
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    assert np.all(idx_h[0] == -1)
    s = O.index_scores(qI[1, 0], w[1, 0], kI[1], O.n_visible(bound, m))
    check_topk_set(idx_h[1, 0], s, k)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

_ATTEND_CASES = [
    # kind, kv type, H, D, Tq
    ("csa", "bf16", 64, 512, 1),
    ("hca", "bf16", 64, 512, 1),
    ("csa", "bf16", 128, 512, 2),
    ("hca", "bf16", 128, 512, 1),
    ("csa", "mixed", 128, 512, 1),
    ("hca", "mixed", 128, 512, 1),
    ("csa", "f32", 8, 128, 3),
    ("hca", "f32", 8, 128, 3),
]


@pytest.mark.parametrize("kind,kv,H,D,Tq", _ATTEND_CASES)
def test_attend_ragged(kind, kv, H, D, Tq):
    L = need_gpu()
    rng = np.random.default_rng(100 + H + D + Tq + (kind == "csa") + 3 * len(kv))
    B, W, k = 4, 128, 517
    m = 4 if kind == "csa" else 128
    bound = 4 * 3000 + 1 if kind == "csa" else 60001
    # the bound, the first position (window of one row, nothing visible), a
    # clipped window, and a position in between
    pos = [bound, 0, 45, bound // 3]
    N_cap = (bound + Tq) // m + 2
    cast = (lambda a: a) if kv == "f32" else WL.bf16_exact
    q = cast((rng.standard_normal((B, Tq, H, D)) * 4 / np.sqrt(D)).astype(np.float32))
    Esrc = (rng.standard_normal((B, N_cap, D)) / np.sqrt(D)).astype(np.float32)
    wsrc = (rng.standard_normal((B, W - 1 + Tq, D)) / np.sqrt(D)).astype(np.float32)
    sink = rng.standard_normal(H).astype(np.float32)
    scale = 1 / math.sqrt(D)
    if kv == "mixed":
        Eq = torch.empty((B, N_cap, D + 64), dtype=torch.uint8, device=DEV)
        Es = torch.empty((B, N_cap), dtype=torch.float32, device=DEV)
        Wq = torch.empty((B, W - 1 + Tq, D + 64), dtype=torch.uint8, device=DEV)
        Ws = torch.empty((B, W - 1 + Tq), dtype=torch.float32, device=DEV)
        L.lca_quantize_rows(L.KV_MIXED, dev_f32(Esrc), Eq, Es)
        L.lca_quantize_rows(L.KV_MIXED, dev_f32(wsrc), Wq, Ws)
        E_ref = [O.kv_mixed_decode(*O.kv_mixed_quantize(Esrc[b], 64)) for b in range(B)]
        W_ref = [O.kv_mixed_decode(*O.kv_mixed_quantize(wsrc[b], 64)) for b in range(B)]
        dt_q, dt_kv, q_d = L.BF16, L.KV_MIXED, dev_bf16(q)
        E_d, W_d, Es_d, Ws_d = Eq, Wq, Es, Ws
        odt = torch.bfloat16
    else:
        Esrc, wsrc = cast(Esrc), cast(wsrc)
        E_ref, W_ref = list(Esrc), list(wsrc)
        up = dev_f32 if kv == "f32" else dev_bf16
        dt_q = dt_kv = L.F32 if kv == "f32" else L.BF16
        q_d, E_d, W_d, Es_d, Ws_d = up(q), up(Esrc), up(wsrc), None, None
        odt = torch.float32 if kv == "f32" else torch.bfloat16
    idx = None
    if kind == "csa":
        idx = np.full((B, Tq, k), -1, np.int32)
        for b in range(B):
            for t in range(Tq):
                nv = O.n_visible(pos[b] + t, m)
                sel = rng.choice(nv, size=min(k - 5, nv), replace=False)
                idx[b, t, :len(sel)] = sel
        idx_d = torch.from_numpy(idx).to(DEV)
    sink_d = dev_f32(sink)

    def run(sl, q_pos0, q_pos):
        n = sl.stop - sl.start
        out = torch.empty((n, Tq, H, D), dtype=odt, device=DEV)
        lse = torch.empty((n, Tq, H), dtype=torch.float32, device=DEV)
        common = dict(m=m, W=W, q_pos0=q_pos0, scale=scale, N_cap=N_cap, flags=L.INV_ROPE, rope_dims=64,
                      lse_out=lse, q_pos=q_pos,
                      kv_scale=None if Es_d is None else Es_d[sl],
                      win_scale=None if Ws_d is None else Ws_d[sl])
        if kind == "csa":
            L.csa_attend(dt_q, dt_kv, q_d[sl], E_d[sl], idx_d[sl], W_d[sl], sink_d, out, **common)
        else:
            L.hca_attend(dt_q, dt_kv, q_d[sl], E_d[sl], W_d[sl], sink_d, out, **common)
        torch.cuda.synchronize()
        return out, lse

    say(f"ragged attend {kind} {kv} H={H} D={D} Tq={Tq} positions={pos} bound={bound}")
    out, lse = run(slice(0, B), bound, _qp(pos))
    got, got_lse = host(out), lse.cpu().numpy()
    tol = 1e-4 if kv == "f32" else 2e-2
    for b in range(B):
        if kind == "csa":
            ref, rl = O.csa_attend(q[b], E_ref[b], idx[b], W_ref[b], sink, scale, pos[b], W, True, 10000.0, 64)
        else:
            ref, rl = O.hca_attend(q[b], E_ref[b], m, W_ref[b], sink, scale, pos[b], W, True, 10000.0, 64)
        row_tol_check(got[b], ref, tol, f"ragged {kind} {kv} b={b} pos={pos[b]}")
        np.testing.assert_allclose(got_lse[b], rl, atol=1e-4 if kv == "f32" else 2e-2)
        # the sequence alone with the same bound: the same bits
        o1, l1 = run(slice(b, b + 1), bound, _qp([pos[b]]))
        assert torch.equal(o1[0], out[b]), f"batch invariance {kind} {kv} b={b}"
        assert torch.equal(l1[0], lse[b])
        # a uniform call at the sequence's own position plans the same splits
        # when the rows per query are the same: CSA once the window is full,
        # HCA at the bound
        same_plan = pos[b] >= W - 1 if kind == "csa" else pos[b] == bound
        if same_plan:
            o2, l2 = run(slice(b, b + 1), pos[b], None)
            assert torch.equal(o2[0], out[b]), f"uniform call {kind} {kv} b={b}"
            assert torch.equal(l2[0], lse[b])
