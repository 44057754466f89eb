"""Compressor backward on the GPU against the oracle's chain rule: the two
streams' row and gate-logit gradients, the carried rows', and the RMSNorm
gain's (summed over every entry of every sequence), for CSA (overlap, m = 4)
and HCA (m = 128) shapes, fp32 and bf16 inputs, with and without the
epilogue; rows that no entry reads come back as zeros; two runs agree bit
for bit."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, dev_bf16, dev_f32, need_gpu, say

pytestmark = pytest.mark.gpu


def _rel(got, ref):
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


@pytest.mark.parametrize("dt,m,overlap,flags,prev,T,D", [
    ("f32", 4, True, "norm+rope", True, 258, 512),     # CSA shape, trailing partial block
    ("bf16", 4, True, "norm+rope", False, 256, 512),   # bf16 rows, block 0 without its stream-a half
    ("f32", 4, True, "", True, 64, 128),               # plain merge
    ("f32", 128, False, "norm", False, 300, 512),      # HCA shape (stream b only)
    ("bf16", 128, False, "", False, 100, 256),         # fewer tokens than one block: all zeros
])
def test_compress_backward_matches_oracle(dt, m, overlap, flags, prev, T, D):
    L = need_gpu()
    rng = np.random.default_rng(900 + m + T + D + overlap)
    B, R, pos0, eps, base = 2, 64, 4 * m, 1e-6, 10000.0
    fl = (L.NORM if "norm" in flags else 0) | (L.ROPE if "rope" in flags else 0)
    cast = WL.bf16_exact if dt == "bf16" else (lambda x: x.astype(np.float32))
    dev = dev_bf16 if dt == "bf16" else dev_f32
    dtc = L.BF16 if dt == "bf16" else L.F32
    cb = cast((rng.standard_normal((B, T, D)) / np.sqrt(D)).astype(np.float32))
    zb = rng.standard_normal((B, T)).astype(np.float32)
    ca = cast((rng.standard_normal((B, T, D)) / np.sqrt(D)).astype(np.float32)) if overlap else None
    za = rng.standard_normal((B, T)).astype(np.float32) if overlap else None
    pca = cast((rng.standard_normal((B, m, D)) / np.sqrt(D)).astype(np.float32)) if prev else None
    pza = rng.standard_normal((B, m)).astype(np.float32) if prev else None
    g = (1 + 0.2 * rng.standard_normal(D)).astype(np.float32)
    n_out = T // m
    dout = rng.standard_normal((B, n_out, D)).astype(np.float32)
    f = lambda shape: torch.full(shape, np.nan, dtype=torch.float32, device=DEV)   # every cell must be written
    out = {"dcb": f((B, T, D)), "dzb": f((B, T))}
    kw = {}
    if overlap:
        out.update(dca=f((B, T, D)), dza=f((B, T)))
        kw.update(ca=dev(ca), za=dev_f32(za))
        if prev:
            out.update(dprev_ca=f((B, m, D)), dprev_za=f((B, m)))
            kw.update(prev_ca=dev(pca), prev_za=dev_f32(pza))
    if fl & L.NORM:
        out["dnorm_w"] = f((D,))
        kw["norm_w"] = dev_f32(g)
    say(f"compress backward {dt} m={m} overlap={overlap} flags={flags} prev={prev} T={T} D={D}")
    args = (dtc, dev(cb), dev_f32(zb), m, dev_f32(dout) if n_out else torch.zeros(0, device=DEV))
    runs = []
    for _ in range(2):
        L.csa_compress_backward(*args, out["dcb"], out["dzb"], overlap=overlap, pos0=pos0, flags=fl, eps=eps,
                                rope_base=base, rope_dims=R if fl & L.ROPE else 0,
                                **{k: v for k, v in out.items() if k not in ("dcb", "dzb")}, **kw)
        torch.cuda.synchronize()
        runs.append({k: v.cpu().numpy().copy() for k, v in out.items()})
    for k in runs[0]:
        assert np.array_equal(runs[0][k], runs[1][k]), f"{k} differs between runs"
        assert not np.isnan(runs[0][k]).any(), f"{k} has unwritten cells"
    got = runs[0]
    tol = 1e-4 if dt == "f32" else 2e-3
    dg_ref = np.zeros(D)
    for b in range(B):
        ref = O.compress_backward(dout[b], cb[b], zb[b], m, ca[b] if overlap else None, za[b] if overlap else None,
                                  pca[b] if prev else None, pza[b] if prev else None, overlap=overlap, pos0=pos0,
                                  norm_w=g if fl & L.NORM else None, eps=eps, rope_base=base if fl & L.ROPE else None,
                                  rope_dims=R if fl & L.ROPE else 0)
        for k, v in ref.items():
            if k == "dnorm_w":
                dg_ref += v
                continue
            e = _rel(got[k][b], v)
            assert e <= tol, f"{k} b={b}: relative error {e:.2e}"
    if fl & L.NORM:
        e = _rel(got["dnorm_w"], dg_ref)
        assert e <= tol, f"dnorm_w: relative error {e:.2e}"


def test_compress_backward_rejects_bad_arguments():
    L = need_gpu()
    B, T, D, m = 1, 8, 64, 4
    cb = torch.zeros((B, T, D), device=DEV)
    zb = torch.zeros((B, T), device=DEV)
    dout = torch.zeros((B, T // m, D), device=DEV)
    dcb, dzb = torch.zeros_like(cb), torch.zeros_like(zb)
    with pytest.raises(ValueError):
        # overlap without the stream-a gradients (caught by the binding)
        L.csa_compress_backward(L.F32, cb, zb, m, dout, dcb, dzb, ca=cb, za=zb, overlap=True)
    with pytest.raises(ValueError):
        # RMSNorm without dnorm_w (caught by the binding)
        L.csa_compress_backward(L.F32, cb, zb, m, dout, dcb, dzb, overlap=False, flags=L.NORM,
                                norm_w=torch.ones(D, device=DEV))
