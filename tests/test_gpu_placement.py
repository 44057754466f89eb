"""Split placement on the GPU: one workgroup per split plus the combine kernel
(the latency placement), or one workgroup walking all of a query's splits and
folding them in registers (the throughput placement). [Qiaomu] 批不变 kernel and
[kwkr] §4.3 describe a pair of attention kernels of these two kinds whose
accumulation order is the same, so the result never depends on which one ran.
Here both placements merge splits with one shared fold; the tests force each
placement and require the same bits, with flagged (recomputed) splits
included, and check that the automatic choice, which follows the batch size,
leaves every sequence's output unchanged."""

import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, dev_bf16, dev_f32, host, need_gpu, row_tol_check, say

pytestmark = pytest.mark.gpu


def _case(rng, B, Tq, H, D, N_cap, W, sharp):
    q = WL.bf16_exact((rng.standard_normal((B, Tq, H, D)) * sharp / np.sqrt(D)).astype(np.float32))
    E = WL.bf16_exact((rng.standard_normal((B, N_cap, D)) / np.sqrt(D)).astype(np.float32))
    win = WL.bf16_exact((rng.standard_normal((B, W - 1 + Tq, D)) / np.sqrt(D)).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    return q, E, win, sink


def _run(L, kind, q_d, E_d, idx_d, win_d, sink_d, m, W, q_pos0, flags, q_pos=None):
    B, Tq, H, D = q_d.shape
    out = torch.empty((B, Tq, H, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=DEV)
    kw = dict(m=m, W=W, q_pos0=q_pos0, scale=1 / math.sqrt(D), flags=L.INV_ROPE | flags, rope_dims=64,
              lse_out=lse, q_pos=q_pos)
    if kind == "csa":
        L.csa_attend(L.BF16, L.BF16, q_d, E_d, idx_d, win_d, sink_d, out, **kw)
    else:
        L.hca_attend(L.BF16, L.BF16, q_d, E_d, win_d, sink_d, out, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("kind,Tq,H,q_pos0", [("csa", 1, 64, 12001), ("csa", 3, 64, 12001), ("hca", 1, 64, 60001),
                                              ("csa", 1, 32, 45), ("hca", 2, 16, 300001),
                                              # 128 heads, 16 queries: the 128-head split kernel
                                              # against the fold kernel as two 64-head groups
                                              ("csa", 16, 128, 12001), ("hca", 16, 128, 128 * 1000 + 5)])
def test_placements_give_the_same_bits(kind, Tq, H, q_pos0):
    L = need_gpu()
    rng = np.random.default_rng(160 + Tq + H)
    B, D, W, k = 3, 512, 128, 517
    m = 4 if kind == "csa" else 128
    N_cap = (q_pos0 + Tq) // m + 2
    q, E, win, sink = _case(rng, B, Tq, H, D, N_cap, W, 6.0)
    idx = None
    idx_d = None
    if kind == "csa":
        idx = np.full((B, Tq, k), -1, np.int32)
        for b in range(B):
            for t in range(Tq):
                nv = O.n_visible(q_pos0 + t, m)
                sel = rng.choice(nv, size=min(k - 4, nv), replace=False)
                idx[b, t, :len(sel)] = sel
        idx_d = torch.from_numpy(idx).to(DEV)
    args = (dev_bf16(q), dev_bf16(E), idx_d, dev_bf16(win), dev_f32(sink), m, W, q_pos0)
    say(f"placements {kind} Tq={Tq} H={H} q_pos0={q_pos0}")
    o1, l1 = _run(L, kind, *args, L.SPLITS_MANY_WG)
    o2, l2 = _run(L, kind, *args, L.SPLITS_ONE_WG)
    assert torch.equal(o1, o2), "the two placements differ"
    assert torch.equal(l1, l2)
    scale = 1 / math.sqrt(D)
    for b in range(B):
        if kind == "csa":
            ref, rl = O.csa_attend(q[b], E[b], idx[b], win[b], sink, scale, q_pos0, W, True, 10000.0, 64)
        else:
            ref, rl = O.hca_attend(q[b], E[b], m, win[b], sink, scale, q_pos0, W, True, 10000.0, 64)
        row_tol_check(host(o2)[b], ref, 2e-2, f"one-workgroup placement {kind} b={b}")
        np.testing.assert_allclose(l2.cpu().numpy()[b], rl, atol=2e-2)


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_placements_agree_on_recomputed_splits(kind):
    # Logits that climb by hundreds along the rows overflow the in-kernel
    # headroom; flagged splits are recomputed exactly, by the combine kernel in
    # one placement and inside the attention kernel in the other.
    L = need_gpu()
    rng = np.random.default_rng(170 + len(kind))
    B, Tq, H, D, W = 1, 1, 64, 512, 128
    m = 4 if kind == "csa" else 128
    q_pos0 = 4 * 2500 if kind == "csa" else 128 * 900
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
    idx = None
    idx_d = None
    if kind == "csa":
        nv = O.n_visible(q_pos0, m)
        idx = np.sort(rng.choice(nv, size=900, replace=False)).astype(np.int32)[None, None]
        idx_d = torch.from_numpy(idx).to(DEV)
    args = (dev_bf16(q), dev_bf16(E), idx_d, dev_bf16(win), dev_f32(sink), m, W, q_pos0)
    say(f"placements on a logit ramp {kind}")
    o1, l1 = _run(L, kind, *args, L.SPLITS_MANY_WG)
    o2, l2 = _run(L, kind, *args, L.SPLITS_ONE_WG)
    scale = 1 / math.sqrt(D)
    if kind == "csa":
        ref, rl = O.csa_attend(q[0], E[0], idx[0], win[0], sink, scale, q_pos0, W, True, 10000.0, 64)
    else:
        ref, rl = O.hca_attend(q[0], E[0], m, win[0], sink, scale, q_pos0, W, True, 10000.0, 64)
    assert np.ptp(rl) > 100.0, "the case must span a wide logit range"
    row_tol_check(host(o2)[0], ref, 2e-2, f"ramp one-workgroup placement {kind}")
    assert torch.equal(o1, o2), "the placements differ on recomputed splits"
    assert torch.equal(l1, l2)


def test_automatic_placement_follows_the_batch_not_the_bits():
    # 300 sequences give 300 (query, head group) items, enough for one
    # workgroup per query (automatic choice); a sequence alone takes the split
    # kernel. Each sequence's output is the same bits either way; a ragged
    # batch too.
    L = need_gpu()
    rng = np.random.default_rng(180)
    B, Tq, H, D, W, m, k = 300, 1, 64, 512, 128, 4, 300
    q_pos0 = 4 * 900 + 3
    N_cap = (q_pos0 + Tq) // m
    q, E, win, sink = _case(rng, B, Tq, H, D, N_cap, W, 5.0)
    nv = O.n_visible(q_pos0, m)
    idx = np.stack([np.sort(rng.choice(nv, size=k, replace=False)) for _ in range(B)]).astype(np.int32)[:, None]
    q_d, E_d, win_d, sink_d = dev_bf16(q), dev_bf16(E), dev_bf16(win), dev_f32(sink)
    idx_d = torch.from_numpy(idx).to(DEV)
    say("automatic placement: B = 300 against single sequences")
    o_all, l_all = _run(L, "csa", q_d, E_d, idx_d, win_d, sink_d, m, W, q_pos0, 0)
    for b in (0, 151, 299):
        o1, l1 = _run(L, "csa", q_d[b:b + 1], E_d[b:b + 1], idx_d[b:b + 1], win_d[b:b + 1], sink_d, m, W, q_pos0, 0)
        assert torch.equal(o1[0], o_all[b]), f"sequence {b}: batch of 300 differs from the sequence alone"
        assert torch.equal(l1[0], l_all[b])
        ref, _ = O.csa_attend(q[b], E[b], idx[b], win[b], sink, 1 / math.sqrt(D), q_pos0, W, True, 10000.0, 64)
        row_tol_check(host(o_all)[b], ref, 2e-2, f"batch of 300, sequence {b}")
    # ragged positions, same bound: a batch of 300 against the sequence alone
    pos = rng.integers(W, q_pos0 + 1, size=B).astype(np.int64)
    qp = torch.from_numpy(pos).to(DEV)
    for b in range(B):
        nvb = O.n_visible(int(pos[b]), m)
        idx[b, 0] = np.where(idx[b, 0] < nvb, idx[b, 0], -1)
    idx_d = torch.from_numpy(idx).to(DEV)
    o_r, _ = _run(L, "csa", q_d, E_d, idx_d, win_d, sink_d, m, W, q_pos0, 0, q_pos=qp)
    for b in (7, 200):
        o1, _ = _run(L, "csa", q_d[b:b + 1], E_d[b:b + 1], idx_d[b:b + 1], win_d[b:b + 1], sink_d, m, W, q_pos0, 0,
                     q_pos=qp[b:b + 1])
        assert torch.equal(o1[0], o_r[b]), f"ragged sequence {b} differs"


@pytest.mark.parametrize("kind,H,B,Tq", [("csa", 64, 16, 1), ("hca", 128, 8, 16), ("csa", 128, 16, 16),
                                         ("csa", 64, 2, 64), ("hca", 128, 2, 80)])
def test_sequence_major_grid_keeps_the_bits(kind, H, B, Tq):
    # 128-head workgroups (16+ queries per call) in batches of a multiple of 8
    # sequences run on one-dimensional grids that keep each sequence's
    # workgroups on one XCD; a single sequence with 64+ queries gives each XCD
    # a contiguous range of queries; other calls use the (units, 1, B) grid.
    # The mapping moves work, never arithmetic: a sequence gives the same bits
    # alone and in the batch.
    L = need_gpu()
    rng = np.random.default_rng(190 + H + Tq)
    D, W, k = 512, 128, 300
    m = 4 if kind == "csa" else 128
    q_pos0 = 4 * 2000 + 1 if kind == "csa" else 128 * 600 + 7
    N_cap = (q_pos0 + Tq) // m
    q, E, win, sink = _case(rng, B, Tq, H, D, N_cap, W, 5.0)
    idx_d = None
    idx = None
    if kind == "csa":
        nv = O.n_visible(q_pos0, m)
        idx = np.stack([np.stack([np.sort(rng.choice(nv, size=k, replace=False)) for _ in range(Tq)])
                        for _ in range(B)]).astype(np.int32)
        idx_d = torch.from_numpy(idx).to(DEV)
    q_d, E_d, win_d, sink_d = dev_bf16(q), dev_bf16(E), dev_bf16(win), dev_f32(sink)
    say(f"sequence-major grid {kind} H={H} B={B} Tq={Tq}: the batch against single sequences")
    o_all, l_all = _run(L, kind, q_d, E_d, idx_d, win_d, sink_d, m, W, q_pos0, 0)
    for b in sorted({0, min(5, B - 1), B - 1}):
        sl = slice(b, b + 1)
        o1, l1 = _run(L, kind, q_d[sl], E_d[sl], idx_d[sl] if idx_d is not None else None, win_d[sl], sink_d, m, W,
                      q_pos0, 0)
        assert torch.equal(o1[0], o_all[b]), f"sequence {b}: the batch differs from the sequence alone"
        assert torch.equal(l1[0], l_all[b])
    b = max(0, B - 2)
    if kind == "csa":
        ref, _ = O.csa_attend(q[b], E[b], idx[b], win[b], sink, 1 / math.sqrt(D), q_pos0, W, True, 10000.0, 64)
    else:
        ref, _ = O.hca_attend(q[b], E[b], m, win[b], sink, 1 / math.sqrt(D), q_pos0, W, True, 10000.0, 64)
    row_tol_check(host(o_all)[b], ref, 2e-2, f"batch of {B}, sequence {b}")


def _mixed(L, src):
    """KV_MIXED rows (448 e4m3fn + 64 bf16 channels, fp32 row scale) of fp32 rows."""
    B, N, D = src.shape
    rows = torch.empty((B, N, D + 64), dtype=torch.uint8, device=DEV)
    scale = torch.empty((B, N), dtype=torch.float32, device=DEV)
    L.lca_quantize_rows(L.KV_MIXED, dev_f32(src), rows, scale)
    return rows, scale


def _run_mixed(L, kind, q_d, E, idx_d, win, sink_d, m, W, q_pos0, flags):
    B, Tq, H, D = q_d.shape
    out = torch.empty((B, Tq, H, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=DEV)
    kw = dict(m=m, W=W, q_pos0=q_pos0, scale=1 / math.sqrt(D), flags=L.INV_ROPE | flags, rope_dims=64,
              lse_out=lse, kv_scale=E[1], win_scale=win[1])
    if kind == "csa":
        L.csa_attend(L.BF16, L.KV_MIXED, q_d, E[0], idx_d, win[0], sink_d, out, **kw)
    else:
        L.hca_attend(L.BF16, L.KV_MIXED, q_d, E[0], win[0], sink_d, out, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("kind,ramp", [("csa", False), ("hca", False), ("hca", True)])
def test_mixed_row_placements_give_the_same_bits(kind, ramp):
    # KV_MIXED rows, 128 heads, one query: 2 splits of 512 rows. The split
    # placement (128-head mixed kernel, bf16 partials, combine) against the
    # mixed fold kernel (two 64-head groups walking both splits); with the
    # logit ramp, splits are flagged and recomputed exactly in both.
    L = need_gpu()
    rng = np.random.default_rng(180 + len(kind) + ramp)
    B, Tq, H, D, W, k = 2, 1, 128, 512, 128, 517
    m = 4 if kind == "csa" else 128
    q_pos0 = 12001 if kind == "csa" else 128 * 700 + 9
    N_cap = (q_pos0 + Tq) // m + 2
    if ramp:
        u = rng.standard_normal(D)
        u /= np.linalg.norm(u)
        lin = np.linspace(-1.0, 1.0, N_cap)
        Esrc = np.stack([(lin[:, None] * u[None, :] + 0.05 * rng.standard_normal((N_cap, D)) / np.sqrt(D))
                         for _ in range(B)]).astype(np.float32)
        sharp = np.geomspace(1.0, 4000.0, H)
        q = sharp[None, None, :, None] * (u + 0.1 * rng.standard_normal((B, Tq, H, D)) / np.sqrt(D))
        q = WL.bf16_exact((q * np.sqrt(D)).astype(np.float32))
    else:
        Esrc = (rng.standard_normal((B, N_cap, D)) / np.sqrt(D)).astype(np.float32)
        q = WL.bf16_exact((rng.standard_normal((B, Tq, H, D)) * 6.0 / np.sqrt(D)).astype(np.float32))
    wsrc = (rng.standard_normal((B, W - 1 + Tq, D)) / np.sqrt(D)).astype(np.float32)
    sink = rng.standard_normal(H).astype(np.float32)
    idx = None
    idx_d = None
    if kind == "csa":
        idx = np.full((B, Tq, k), -1, np.int32)
        for b in range(B):
            nv = O.n_visible(q_pos0, m)
            sel = rng.choice(nv, size=k - 3, replace=False)
            idx[b, 0, :len(sel)] = sel
        idx_d = torch.from_numpy(idx).to(DEV)
    E, win = _mixed(L, Esrc), _mixed(L, wsrc)
    args = (dev_bf16(q), E, idx_d, win, dev_f32(sink), m, W, q_pos0)
    say(f"mixed-row placements {kind} ramp={ramp}")
    o1, l1 = _run_mixed(L, kind, *args, L.SPLITS_MANY_WG)
    o2, l2 = _run_mixed(L, kind, *args, L.SPLITS_ONE_WG)
    assert torch.equal(o1, o2), "the two placements differ"
    assert torch.equal(l1, l2)
    scale = 1 / math.sqrt(D)
    for b in range(B):
        Ed = O.kv_mixed_decode(*O.kv_mixed_quantize(Esrc[b], 64))
        Wd = O.kv_mixed_decode(*O.kv_mixed_quantize(wsrc[b], 64))
        if kind == "csa":
            ref, rl = O.csa_attend(q[b], Ed, idx[b], Wd, sink, scale, q_pos0, W, True, 10000.0, 64)
        else:
            ref, rl = O.hca_attend(q[b], Ed, m, Wd, sink, scale, q_pos0, W, True, 10000.0, 64)
        if ramp:
            assert np.ptp(rl) > 100.0, "the case must span a wide logit range"
        row_tol_check(host(o2)[b], ref, 2e-2, f"mixed one-workgroup placement {kind} b={b}")
        lse_err = np.abs(l2.cpu().numpy()[b] - rl) / np.maximum(1.0, np.abs(rl))
        assert lse_err.max() <= 2e-2, f"lse relative error {lse_err.max()}"
