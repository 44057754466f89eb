"""csa_attend_noalloc (split partials in the library's static device array,
nothing allocated) against csa_attend (caller workspace): the same kernels
and split plan, so out and lse must agree bit for bit. Two calls in a row,
the second smaller than the first, so the second reads an array that still
holds the first call's partials."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, host, need_gpu, row_tol_check, say

pytestmark = pytest.mark.gpu


def _inputs(B, ctx, seed, H=64, D=512, k=512, W=128, m=4):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    N = ctx // m
    r = lambda *s, sc=1.0: (torch.randn(*s, generator=g, device=DEV) * sc).to(torch.bfloat16)
    q = r(B, 1, H, D, sc=8.0 / math.sqrt(D))
    E = r(B, N, D, sc=1 / math.sqrt(D))
    win = r(B, W, D, sc=1 / math.sqrt(D))
    sink = torch.randn(H, generator=g, device=DEV)
    # k - 3 distinct visible entries per sequence, -1 in the last three slots
    sel = torch.argsort(torch.rand(B, N, generator=g, device=DEV), dim=1)[:, :k - 3].to(torch.int32)
    idx = torch.full((B, 1, k), -1, dtype=torch.int32, device=DEV)
    idx[:, 0, :k - 3] = sel
    return dict(q=q, E=E, win=win, sink=sink, idx=idx, B=B, H=H, D=D, k=k, W=W, m=m, ctx=ctx)


def _run(L, d, noalloc):
    B, H, D = d["B"], d["H"], d["D"]
    out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, 1, H), dtype=torch.float32, device=DEV)
    kw = dict(m=d["m"], W=d["W"], q_pos0=d["ctx"], scale=1 / math.sqrt(D), flags=L.INV_ROPE, rope_dims=64,
              lse_out=lse)
    fn = L.csa_attend_noalloc if noalloc else L.csa_attend
    fn(L.BF16, L.BF16, d["q"], d["E"], d["idx"], d["win"], d["sink"], out, **kw)
    torch.cuda.synchronize()
    return out, lse


def test_noalloc_matches_workspace_call_twice():
    L = need_gpu()
    for B, ctx, seed in ((16, 131072, 41), (3, 8192, 42)):
        say(f"csa_attend_noalloc B={B} ctx={ctx}")
        d = _inputs(B, ctx, seed)
        ref_out, ref_lse = _run(L, d, noalloc=False)
        out, lse = _run(L, d, noalloc=True)
        assert torch.equal(out, ref_out), f"out differs at B={B}"
        assert torch.equal(lse, ref_lse), f"lse differs at B={B}"
    # the smaller call also meets the oracle's bar on one sequence
    b = 1
    E, win = host(d["E"][b]), host(d["win"][b])
    ref, _ = O.csa_attend_query(host(d["q"][b, 0]), E, d["idx"][b, 0].cpu().numpy(), win,
                                d["sink"].cpu().numpy().astype(np.float64), 1 / math.sqrt(d["D"]), ctx, ctx,
                                d["W"], True, 10000.0, 64)
    row_tol_check(host(out[b, 0]), ref, 2e-2, "csa_attend_noalloc B=3")


def test_noalloc_rejects_calls_beyond_the_array():
    L = need_gpu()
    d = _inputs(2, 8192, 43)
    big = L.csa_attend_workspace(L.BF16, L.BF16, 52, 1, 64, 512, 32768, 4, 512, 128, 131072)
    assert big > L.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((52, 1, 64, 512), dtype=torch.bfloat16, device=DEV)
    E = torch.zeros((52, 32768, 512), dtype=torch.bfloat16, device=DEV)
    win = torch.zeros((52, 128, 512), dtype=torch.bfloat16, device=DEV)
    idx = torch.full((52, 1, 512), -1, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(L.LcaError) as e:
        L.csa_attend_noalloc(L.BF16, L.BF16, q, E, idx, win, d["sink"], out, m=4, W=128, q_pos0=131072,
                             scale=0.04, flags=L.INV_ROPE, rope_dims=64)
    assert e.value.status == -4 and "static array" in str(e.value)
