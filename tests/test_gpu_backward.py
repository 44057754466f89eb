"""Attention backward on the GPU against the oracle's chain rule: dq, the
entries' and window rows' gradients (summed over every query that read
them), and the sink's; several accumulation slots with window rows shared
between them; and two runs that must agree bit for bit. The GPU forward
supplies out and lse to the GPU backward; the oracle recomputes everything
from the seeded inputs."""

import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, dev_bf16, dev_f32, host, need_gpu, row_tol_check, say

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _case(rng, B, Tq, H, N_cap, W, sharp, D=512):
    q = WL.bf16_exact((rng.standard_normal((B, Tq, H, D)) * sharp / np.sqrt(D)).astype(np.float32))
    E = WL.bf16_exact((rng.standard_normal((B, N_cap, D)) / np.sqrt(D)).astype(np.float32))
    win = WL.bf16_exact((rng.standard_normal((B, W - 1 + Tq, D)) / np.sqrt(D)).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    dout = WL.bf16_exact(rng.standard_normal((B, Tq, H, D)).astype(np.float32))
    return q, E, win, sink, dout


@pytest.mark.parametrize("kind,Tq,H,inv", [("csa", 5, 64, True), ("csa", 3, 64, False), ("hca", 4, 64, True),
                                           ("csa", 40, 64, True), ("csa", 2, 128, True), ("hca", 36, 128, False)])
def test_attend_backward_matches_oracle(kind, Tq, H, inv):
    L = need_gpu()
    rng = np.random.default_rng(300 + Tq + H + inv)
    B, D, W = 2, 512, 128
    m = 4 if kind == "csa" else 128
    q_pos0 = 200 if kind == "csa" else 128 * 40 + 5
    k = 24
    N_cap = (q_pos0 + Tq) // m + 3
    q, E, win, sink, dout = _case(rng, B, Tq, H, N_cap, W, 4.0)
    scale = 1 / math.sqrt(D)
    R = 64 if inv else 0
    flags = L.INV_ROPE if inv else 0
    idx = None
    idx_d = None
    if kind == "csa":
        idx = np.full((B, Tq, k), -1, np.int32)
        for b in range(B):
            for t in range(Tq):
                nv = O.n_visible(q_pos0 + t, m)
                sel = rng.choice(nv, size=min(k - 3, nv), replace=False)
                idx[b, t, :len(sel)] = sel
        idx_d = torch.from_numpy(idx).to(DEV)
    q_d, E_d, win_d, sink_d, dout_d = dev_bf16(q), dev_bf16(E), dev_bf16(win), dev_f32(sink), dev_bf16(dout)
    out = torch.empty((B, Tq, H, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=DEV)
    kw = dict(m=m, W=W, q_pos0=q_pos0, scale=scale, flags=flags, rope_dims=R)
    if kind == "csa":
        L.csa_attend(L.BF16, L.BF16, q_d, E_d, idx_d, win_d, sink_d, out, lse_out=lse, **kw)
    else:
        L.hca_attend(L.BF16, L.BF16, q_d, E_d, win_d, sink_d, out, lse_out=lse, **kw)
    say(f"backward {kind} Tq={Tq} H={H} inv_rope={inv}")
    g1 = L.attend_backward(kind, q_d, E_d, win_d, sink_d, out, lse, dout_d, idx=idx_d, **kw)
    g2 = L.attend_backward(kind, q_d, E_d, win_d, sink_d, out, lse, dout_d, idx=idx_d, **kw)
    torch.cuda.synchronize()
    for x, y in zip(g1, g2):
        assert torch.equal(x, y), "two runs differ"
    dq, dkv, dwin, dsink = (host(x) for x in g1)
    ds_ref = np.zeros(H)
    for b in range(B):
        if kind == "csa":
            rq, rE, rw, rs = O.csa_attend_backward(q[b], E[b], idx[b], win[b], sink, scale, q_pos0, dout[b], W, inv,
                                                   10000.0, R)
        else:
            rq, rE, rw, rs = O.hca_attend_backward(q[b], E[b], m, win[b], sink, scale, q_pos0, dout[b], W, inv,
                                                   10000.0, R)
        ds_ref += rs
        # the bf16 bar (2e-2) of the forward holds for the gradients too
        worst = [row_tol_check(dq[b], rq, TOL, f"dq b={b}")]
        touched = np.abs(rE).max(axis=1) > 0
        worst.append(row_tol_check(dkv[b][touched], rE[touched], TOL, f"dkv b={b}"))
        assert np.all(dkv[b][~touched] == 0), "rows no query read must be zero"
        wt = np.abs(rw).max(axis=1) > 0
        worst.append(row_tol_check(dwin[b][wt], rw[wt], TOL, f"dwin b={b}"))
        assert np.all(dwin[b][~wt] == 0)
        say(f"  b={b} worst row errors dq {worst[0]:.2e} dkv {worst[1]:.2e} dwin {worst[2]:.2e}")
    np.testing.assert_allclose(dsink, ds_ref, rtol=TOL, atol=TOL * np.abs(ds_ref).max())
