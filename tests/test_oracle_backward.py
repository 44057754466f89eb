"""Pins of the oracle's attention backward: central finite differences of
L = sum(dout * out) through the oracle's (separately pinned) forward, float64
torch autograd through an independently written forward, and closed forms."""

import math

import numpy as np
import pytest
import torch

import oracle as O


def _tiny(rng, Tq=3, H=2, D=8, N=7, k=3, W=4):
    q = rng.standard_normal((Tq, H, D))
    E = rng.standard_normal((N, D))
    win = rng.standard_normal((W - 1 + Tq, D))
    sink = rng.standard_normal(H)
    dout = rng.standard_normal((Tq, H, D))
    return q, E, win, sink, dout


def _loss(q, E, idx, win, sink, dout, scale, q_pos0, W, inv, m=None):
    if m is None:
        out, _ = O.csa_attend(q, E, idx, win, sink, scale, q_pos0, W, inv, 10000.0, 4 if inv else 0)
    else:
        out, _ = O.hca_attend(q, E, m, win, sink, scale, q_pos0, W, inv, 10000.0, 4 if inv else 0)
    return float(np.sum(dout * out))


@pytest.mark.parametrize("kind,inv", [("csa", False), ("csa", True), ("hca", True)])
def test_finite_differences(kind, inv):
    rng = np.random.default_rng(1 + inv + 2 * (kind == "hca"))
    Tq, H, D, W = 3, 2, 8, 4
    q, E, win, sink, dout = _tiny(rng, Tq=Tq, H=H, D=D, W=W)
    scale, q_pos0 = 0.7, 9 if kind == "csa" else 11     # HCA: (11 + 2 + 1) // 2 = 7 entries
    m = 4 if kind == "csa" else 2
    idx = None
    if kind == "csa":
        # entries visible at q_pos0 + t: (q_pos0 + t + 1) // 4 = 2, 2, 3; an absent slot
        idx = np.array([[1, 0, -1], [0, 1, -1], [2, 0, 1]])
        dq, dE, dwin, ds = O.csa_attend_backward(q, E, idx, win, sink, scale, q_pos0, dout, W, inv, 10000.0,
                                                 4 if inv else 0)
    else:
        dq, dE, dwin, ds = O.hca_attend_backward(q, E, m, win, sink, scale, q_pos0, dout, W, inv, 10000.0,
                                                 4 if inv else 0)
    eps = 1e-6

    def fd(arr, setter):
        g = np.zeros_like(arr)
        for ix in np.ndindex(arr.shape):
            a = arr.copy(); a[ix] += eps
            b = arr.copy(); b[ix] -= eps
            g[ix] = (setter(a) - setter(b)) / (2 * eps)
        return g
    mm = None if kind == "csa" else m
    np.testing.assert_allclose(dq, fd(q, lambda a: _loss(a, E, idx, win, sink, dout, scale, q_pos0, W, inv, mm)),
                               atol=1e-7)
    np.testing.assert_allclose(dE, fd(E, lambda a: _loss(q, a, idx, win, sink, dout, scale, q_pos0, W, inv, mm)),
                               atol=1e-7)
    np.testing.assert_allclose(dwin, fd(win, lambda a: _loss(q, E, idx, a, sink, dout, scale, q_pos0, W, inv, mm)),
                               atol=1e-7)
    np.testing.assert_allclose(ds, fd(sink, lambda a: _loss(q, E, idx, win, a, dout, scale, q_pos0, W, inv, mm)),
                               atol=1e-7)


def test_torch_autograd_through_an_independent_forward():
    # forward written with torch ops: logits of the rows and a sink column,
    # logsumexp-normalised; the output's last R channels turned by -p
    rng = np.random.default_rng(7)
    Tq, H, D, N, k, W, R = 4, 3, 16, 9, 4, 5, 8
    q, E, win, sink, dout = _tiny(rng, Tq=Tq, H=H, D=D, N=N, k=k, W=W)
    q_pos0, scale, m = 20, 0.3, 4
    idx = np.stack([rng.choice(O.n_visible(q_pos0 + t, m), size=k, replace=False) for t in range(Tq)])
    tq = torch.tensor(q, requires_grad=True)
    tE = torch.tensor(E, requires_grad=True)
    tw = torch.tensor(win, requires_grad=True)
    ts = torch.tensor(sink, requires_grad=True)
    loss = 0.0
    for t in range(Tq):
        p = q_pos0 + t
        wpos = [pp for pp in range(max(0, p - W + 1), p + 1)]
        X = torch.cat([tE[torch.tensor(idx[t])], tw[torch.tensor([pp - (q_pos0 - (W - 1)) for pp in wpos])]])
        lg = scale * (tq[t] @ X.T)                                  # [H, rows]
        full = torch.cat([lg, ts[:, None]], dim=1)
        wts = torch.softmax(full, dim=1)[:, :-1]
        o = wts @ X                                                  # [H, D]
        i = torch.arange(R // 2, dtype=torch.float64)
        ang = -p * 10000.0 ** (-2 * i / R)
        c, sn = torch.cos(ang), torch.sin(ang)
        u, v = o[:, D - R::2], o[:, D - R + 1::2]
        rot = torch.stack([u * c - v * sn, u * sn + v * c], dim=2).reshape(H, R)
        out = torch.cat([o[:, :D - R], rot], dim=1)
        loss = loss + (torch.tensor(dout[t]) * out).sum()
    loss.backward()
    dq, dE, dwin, ds = O.csa_attend_backward(q, E, idx, win, sink, scale, q_pos0, dout, W, True, 10000.0, R)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dE, tE.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dwin, tw.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(ds, ts.grad.numpy(), atol=1e-11)


def test_closed_forms():
    rng = np.random.default_rng(9)
    H, D = 2, 6
    q = rng.standard_normal((H, D))
    x = rng.standard_normal((1, D))
    dout = rng.standard_normal((H, D))
    # one row and no sink (sink -> -inf): the output is that row whatever q is,
    # so dq = 0, dx = sum_h dout_h, dsink = 0
    dq, dX, ds = O.attend_backward_query(q, x, np.full(H, -np.inf), 0.5, 0, dout)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dX[0], dout.sum(axis=0), atol=1e-14)
    np.testing.assert_allclose(ds, 0.0, atol=1e-15)
    # no rows: output 0, nothing flows anywhere
    dq, dX, ds = O.attend_backward_query(q, np.zeros((0, D)), np.zeros(H), 0.5, 0, dout)
    assert dX.shape == (0, D) and np.all(dq == 0) and np.all(ds == 0)
    # n equal rows, no sink: the output is x whatever q is, so dq = 0
    X = np.repeat(x, 4, axis=0)
    dq, dX, ds = O.attend_backward_query(q, X, np.full(H, -np.inf), 0.5, 0, dout)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)
    np.testing.assert_allclose(dX.sum(axis=0), dout.sum(axis=0), atol=1e-13)
    # n equal rows with a sink s: out = sigma(a) x with a = scale q.x + log n - s,
    # so dq = sigma' (dout . x) scale x and dsink = -sigma' (dout . x), sigma' = sigma (1 - sigma)
    sink = np.array([0.3, -1.0])
    dq, dX, ds = O.attend_backward_query(q, X, sink, 0.5, 0, dout)
    for h in range(H):
        a = 0.5 * float(q[h] @ x[0]) + math.log(4) - sink[h]
        sg = 1 / (1 + math.exp(-a))
        g = sg * (1 - sg) * float(dout[h] @ x[0])
        np.testing.assert_allclose(dq[h], g * 0.5 * x[0], atol=1e-13)
        np.testing.assert_allclose(ds[h], -g, atol=1e-13)
