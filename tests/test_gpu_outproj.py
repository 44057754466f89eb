"""Grouped output projection on the GPU against the oracle: ragged row counts
around the 16-row MFMA tiles, the Flash and Pro shapes in full, and rows that
keep their bits whatever the row count of the call."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, dev_bf16, host, need_gpu, row_tol_check, say

pytestmark = pytest.mark.gpu


def _case(rng, T, n_h, c, g, d_g, d_model):
    o = WL.bf16_exact(rng.standard_normal((T, n_h, c)).astype(np.float32))
    kg = (n_h // g) * c
    w_g = WL.bf16_exact((rng.standard_normal((g, d_g, kg)) / np.sqrt(kg)).astype(np.float32))
    w_o = WL.bf16_exact((rng.standard_normal((d_model, g * d_g)) / np.sqrt(g * d_g)).astype(np.float32))
    return o, w_g, w_o


def _check(L, o, w_g, w_o, what):
    T, n_h, c = o.shape
    g, d_g, _ = w_g.shape
    d_model = w_o.shape[0]
    out = torch.empty((T, d_model), dtype=torch.bfloat16, device=DEV)
    mid = L.lca_grouped_out_proj(dev_bf16(o), dev_bf16(w_g), dev_bf16(w_o), out)
    torch.cuda.synchronize()
    ref, mid_ref = O.grouped_output_projection(o, w_g, w_o, round_mid=True, return_mid=True)
    # stage 1 against the exact intermediate: bf16 rounding of fp32 sums
    err = np.abs(host(mid) - mid_ref)
    assert np.all(err <= 2 ** -8 * np.abs(mid_ref) + 1e-3 * np.max(np.abs(mid_ref))), f"{what}: intermediate"
    # stage 2 against the oracle, which rounds its own intermediate to bf16
    row_tol_check(host(out), ref, 1e-2, what)
    return mid, out


@pytest.mark.parametrize("T", [1, 7, 16, 33, 64, 100, 257])
def test_grouped_out_proj_ragged_rows(T):
    L = need_gpu()
    rng = np.random.default_rng(200 + T)
    o, w_g, w_o = _case(rng, T, 16, 64, 4, 128, 96)
    say(f"grouped out proj T={T}")
    _check(L, o, w_g, w_o, f"T={T}")


@pytest.mark.parametrize("shape", ["flash", "pro"])
def test_grouped_out_proj_model_shapes(shape):
    # Flash: 64 heads x 512 in 8 groups of 1024, width 4096 (decode batch 16);
    # Pro: 128 heads in 16 groups, width 7168 (batch 4)
    L = need_gpu()
    T, n_h, g, d_model = (16, 64, 8, 4096) if shape == "flash" else (4, 128, 16, 7168)
    rng = np.random.default_rng(210 + g)
    o, w_g, w_o = _case(rng, T, n_h, 512, g, 1024, d_model)
    say(f"grouped out proj {shape}: T={T} n_h={n_h} g={g} d_model={d_model}")
    _check(L, o, w_g, w_o, shape)


def test_grouped_out_proj_rows_keep_their_bits():
    # a row's result does not depend on how many rows the call holds
    L = need_gpu()
    rng = np.random.default_rng(220)
    o, w_g, w_o = _case(rng, 70, 16, 128, 2, 128, 128)
    od, wgd, wod = dev_bf16(o), dev_bf16(w_g), dev_bf16(w_o)
    full = torch.empty((70, 128), dtype=torch.bfloat16, device=DEV)
    L.lca_grouped_out_proj(od, wgd, wod, full)
    say("grouped out proj rows vs row counts")
    for lo, hi in ((0, 1), (5, 21), (17, 49), (3, 70)):
        part = torch.empty((hi - lo, 128), dtype=torch.bfloat16, device=DEV)
        L.lca_grouped_out_proj(od[lo:hi].contiguous(), wgd, wod, part)
        torch.cuda.synchronize()
        assert torch.equal(part, full[lo:hi]), f"rows {lo}:{hi}"


def test_grouped_out_proj_tiled_rows_keep_their_bits():
    # 300 rows take the tiled kernel in both stages (256-row blocks, a ragged
    # tail), a few rows the per-row-tile kernel: the same K slices summed in
    # the same order, so the same bits
    L = need_gpu()
    rng = np.random.default_rng(230)
    o, w_g, w_o = _case(rng, 300, 16, 128, 2, 128, 256)
    say("grouped out proj tiled: 300 rows vs row subsets")
    mid, full = _check(L, o, w_g, w_o, "tiled T=300")
    od, wgd, wod = dev_bf16(o), dev_bf16(w_g), dev_bf16(w_o)
    for lo, hi in ((0, 16), (250, 300), (37, 101)):
        part = torch.empty((hi - lo, 256), dtype=torch.bfloat16, device=DEV)
        pm = L.lca_grouped_out_proj(od[lo:hi].contiguous(), wgd, wod, part)
        torch.cuda.synchronize()
        assert torch.equal(pm, mid[lo:hi]), f"intermediate rows {lo}:{hi}"
        assert torch.equal(part, full[lo:hi]), f"rows {lo}:{hi}"


@pytest.mark.parametrize("T,g", [(256, 2), (513, 3)])
def test_grouped_out_proj_tiled_edges(T, g):
    # the tiled kernel at exactly one 256-row block, and at three groups of
    # three row blocks each (nine (group, row block) pairs, padded to 16 in the
    # XCD-aware order) with a one-row tail
    L = need_gpu()
    rng = np.random.default_rng(240 + T + g)
    o, w_g, w_o = _case(rng, T, 4 * g, 64, g, 256, 128)
    say(f"grouped out proj tiled edges: T={T} g={g}")
    mid, full = _check(L, o, w_g, w_o, f"tiled T={T} g={g}")
    od, wgd, wod = dev_bf16(o), dev_bf16(w_g), dev_bf16(w_o)
    lo, hi = T - 40, T
    part = torch.empty((hi - lo, 128), dtype=torch.bfloat16, device=DEV)
    pm = L.lca_grouped_out_proj(od[lo:hi].contiguous(), wgd, wod, part)
    torch.cuda.synchronize()
    assert torch.equal(pm, mid[lo:hi]) and torch.equal(part, full[lo:hi]), f"rows {lo}:{hi}"


def test_grouped_out_proj_column_tiles_keep_their_bits():
    # 100 rows (two 64-row blocks) give the first stage 256 workgroups with
    # four 16-column tiles each; 64 rows (one block) take two tiles per
    # workgroup: a column's MFMA chain is the same, so are its bits
    L = need_gpu()
    rng = np.random.default_rng(250)
    o, w_g, w_o = _case(rng, 100, 16, 128, 8, 1024, 64)
    say("grouped out proj: column tiles per workgroup vs row subsets")
    mid, full = _check(L, o, w_g, w_o, "column tiles T=100")
    od, wgd, wod = dev_bf16(o), dev_bf16(w_g), dev_bf16(w_o)
    for lo, hi in ((0, 64), (36, 100), (50, 66)):
        part = torch.empty((hi - lo, 64), dtype=torch.bfloat16, device=DEV)
        pm = L.lca_grouped_out_proj(od[lo:hi].contiguous(), wgd, wod, part)
        torch.cuda.synchronize()
        assert torch.equal(pm, mid[lo:hi]), f"intermediate rows {lo}:{hi}"
        assert torch.equal(part, full[lo:hi]), f"rows {lo}:{hi}"
