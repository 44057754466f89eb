"""Helpers for the GPU parity tests: device upload, tolerance metric, and the
oracle-side composition of a CSA / HCA layer (oracle functions only)."""

from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle as O

DEV = "cuda"


def need_gpu():
    import long_context_attention_12_amd as L
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(L.lib_path):
        raise RuntimeError("liblca.so missing on a GPU machine: build before testing")
    return L


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(x):
    """Upload float32 values that are exact in bf16 as a bf16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def row_tol_check(got, ref, tol, what=""):
    """Per (t, h) row: max|got - ref| <= tol * max(max|ref_row|, 1e-3 * max|ref|)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    D = ref.shape[-1]
    g = got.reshape(-1, D)
    r = ref.reshape(-1, D)
    keep = ~np.isnan(r).any(axis=1)
    g, r = g[keep], r[keep]
    gmax = np.max(np.abs(r)) if r.size else 0.0
    err = np.max(np.abs(g - r), axis=1)
    den = np.maximum(np.max(np.abs(r), axis=1), 1e-3 * gmax)
    worst = np.max(err / np.maximum(den, 1e-300)) if err.size else 0.0
    assert worst <= tol, f"{what}: worst row error {worst:.3e} > {tol:.1e}"
    return worst


def check_topk_set(gpu_idx_row, scores, k, bf16_scores=False):
    """Spec acceptance of a top-k set against the oracle's classes."""
    n = scores.shape[0]
    k_eff = min(k, n)
    sel = [int(i) for i in gpu_idx_row if i >= 0]
    assert len(sel) == k_eff, (len(sel), k_eff)
    assert len(set(sel)) == k_eff, "duplicate indices"
    assert all(0 <= i < n for i in sel)
    # padding comes last
    assert all(i < 0 for i in gpu_idx_row[k_eff:])
    cin, cout, amb = O.topk_classes(scores, k, bf16_scores=bf16_scores)
    G = np.zeros(n, bool)
    G[sel] = True
    assert np.all(G[cin]), "a certain-in entry is missing"
    assert not np.any(G[cout]), "a certain-out entry was selected"
    return int(amb.sum())


def oracle_csa_rows(E, idx_row, win, q_t, sink, scale, p, q_pos0, W, rope_base, rope_dims, inv):
    return O.csa_attend_query(q_t, E, idx_row, win, sink, scale, p, q_pos0, W, inv, rope_base, rope_dims)
