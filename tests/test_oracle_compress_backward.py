"""Pins of the oracle's compressor backward against the forward itself:
central finite differences of L = sum(dout * entries) with respect to every
input, for CSA (overlap, carried rows, RMSNorm + RoPE epilogue) and HCA
shapes, and the closed form of equal gate logits."""

import numpy as np
import pytest

import oracle as O


def _forward(inp, m, overlap, pos0, eps, rope_base, R, use_norm, use_prev):
    ent = O.compress_sequence(inp["cb"], inp["zb"], m, inp.get("ca"), inp.get("za"),
                              inp.get("prev_ca") if use_prev else None,
                              inp.get("prev_za") if use_prev else None, overlap=overlap)
    return O.compress_epilogue(ent, pos0, m, inp["norm_w"] if use_norm else None, eps,
                               rope_base if R else None, R)


@pytest.mark.parametrize("overlap,use_norm,R,use_prev,T", [
    (True, True, 4, True, 14),      # CSA with the epilogue and carried rows, a trailing partial block
    (True, False, 0, False, 12),    # plain merge, block 0 without its stream-a half
    (True, True, 0, True, 8),       # RMSNorm only
    (False, True, 4, False, 13),    # HCA-style (stream b only)
])
def test_compress_backward_matches_finite_differences(overlap, use_norm, R, use_prev, T):
    rng = np.random.default_rng(7 + T + 3 * overlap + use_norm + R)
    D, m, pos0, eps, base = 8, 4, 20, 1e-3, 100.0
    inp = {"cb": rng.standard_normal((T, D)), "zb": rng.standard_normal(T),
           "norm_w": 1 + 0.3 * rng.standard_normal(D)}
    if overlap:
        inp["ca"] = rng.standard_normal((T, D))
        inp["za"] = rng.standard_normal(T)
        inp["prev_ca"] = rng.standard_normal((m, D))
        inp["prev_za"] = rng.standard_normal(m)
    n_out = T // m
    dout = rng.standard_normal((n_out, D))
    args = (m, overlap, pos0, eps, base, R, use_norm, use_prev)
    got = O.compress_backward(dout, inp["cb"], inp["zb"], m, inp.get("ca"), inp.get("za"),
                              inp.get("prev_ca") if use_prev else None, inp.get("prev_za") if use_prev else None,
                              overlap=overlap, pos0=pos0, norm_w=inp["norm_w"] if use_norm else None, eps=eps,
                              rope_base=base if R else None, rope_dims=R)
    names = {"cb": "dcb", "zb": "dzb", "norm_w": "dnorm_w"}
    if overlap:
        names.update({"ca": "dca", "za": "dza"})
        if use_prev:
            names.update({"prev_ca": "dprev_ca", "prev_za": "dprev_za"})
    if not use_norm:
        names.pop("norm_w")
    h = 1e-6
    for name, gname in names.items():
        x = inp[name]
        num = np.zeros_like(x)
        for ix in np.ndindex(x.shape):
            old = x[ix]
            x[ix] = old + h
            lp = float(np.sum(dout * _forward(inp, *args)))
            x[ix] = old - h
            lm = float(np.sum(dout * _forward(inp, *args)))
            x[ix] = old
            num[ix] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(got[gname], num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_compress_backward_equal_logits_closed_form():
    # every gate logit equal: the merge is the mean of the n rows, so
    # dx_i = de / n and dl_i = (x_i - mean) . de / n
    rng = np.random.default_rng(11)
    T, D, m = 8, 5, 4
    ca, cb = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    z = np.full(T, 0.7)
    dout = rng.standard_normal((T // m, D))
    got = O.compress_backward(dout, cb, z, m, ca, z)
    # block 1 reads ca[0:4] and cb[4:8] (n = 8)
    x = np.concatenate([ca[0:4], cb[4:8]])
    de = dout[1]
    np.testing.assert_allclose(got["dca"][0:4], np.tile(de / 8, (4, 1)), rtol=1e-12)
    np.testing.assert_allclose(got["dcb"][4:8], np.tile(de / 8, (4, 1)), rtol=1e-12)
    dl = (x - x.mean(axis=0)) @ de / 8
    np.testing.assert_allclose(got["dza"][0:4], dl[:4], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(got["dzb"][4:8], dl[4:], rtol=1e-12, atol=1e-15)
    # block 0 has no stream-a half (no carried rows): cb[0:4] only, n = 4
    np.testing.assert_allclose(got["dcb"][0:4], np.tile(dout[0] / 4, (4, 1)), rtol=1e-12)
    # stream a of the last block feeds no entry here
    assert np.all(got["dca"][4:8] == 0) and np.all(got["dza"][4:8] == 0)
