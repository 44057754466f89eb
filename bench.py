"""Benchmark of the CSA decode step on one MI355X.

Workload (headline): CSA decode, V4-Flash shaped: batch 16, one new token per
sequence after 131072 context tokens (32768 compressed entries), 64 query
heads, KV entry dim 512 bf16, indexer 4 heads x 128 bf16, top-k 512, window
128, sink on. One step = csa_index_topk (indexer scores of every entry + top-k)
followed by csa_attend (MQA over selected entries + window + sink, combine with
inverse RoPE). Inputs are seeded synthetic tensors resident in HBM; several
copies are rotated so the 256 MB last-level cache cannot serve a step from the
previous one.

Also measured (secondary, same line): HCA decode, V4-Pro shaped: batch 8,
1048576 context tokens (8192 entries), 128 heads; both decode workloads again
as ragged batches (each sequence at its own position, the context as bound).

Prints one JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Counter runs: rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) over
``bench.py --no-secondary --no-prefill --no-mixed --no-ragged --no-placement --no-outproj --no-backward --copy-calibration 1024``,
then ``bench.py --pmc-summary F.csv W.csv --copy-calibration 1024``.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import long_context_attention_12_amd as L  # noqa: E402
import workloads as WL  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
COPY_REPS = 3                  # calibration copies per counter run
DEV = "cuda"
MFMA_BF16_PEAK = 2.5e15        # dense bf16 MFMA, FLOP/s
N_CU = 256
N_XCD = 8
# sources of each kernel: stored counter readings hold for these bytes only
_HDRS = ["long_context_attention_12_amd/csrc/lca_device.h", "long_context_attention_12_amd/csrc/lca_internal.h"]
SCORE_SOURCES = ["long_context_attention_12_amd/csrc/index_topk.hip"] + _HDRS
ATTEND_SOURCES = ["long_context_attention_12_amd/csrc/attend.hip"] + _HDRS
# kernels whose HBM traffic (FETCH_SIZE, WRITE_SIZE) a counter run of one leg
# records: leg -> [(key, kernel-name substring, sources)]
TRAFFIC_KERNELS = {
    "csa": ("csa_decode_b16_ctx131072", [("index_score", "index_score_bf16_kernel", SCORE_SOURCES),
                                         ("topk_select", "topk_select_kernel", SCORE_SOURCES),
                                         ("csa_attend", "attend_dma_kernel<1>", ATTEND_SOURCES),
                                         ("csa_combine", "combine4_kernel<true>", ATTEND_SOURCES)]),
    "hca": ("hca_decode_b8_ctx1048576", [("hca_attend", "attend_dma_kernel<1>", ATTEND_SOURCES),
                                         ("hca_combine", "combine4_kernel<true>", ATTEND_SOURCES)]),
    "mixed": ("mixed_csa_hca_pair_b64_ctx1048576", [("index_score", "index_score_fp4_kernel", SCORE_SOURCES),
                                                    ("attend_mixed", "attend_mixed_dma_kernel<2>", ATTEND_SOURCES)]),
}
# kernels whose MFMA counters the prefill counter run records
MFMA_KERNELS = {"prefill": ("csa_prefill_tq4096_ctx1048576",
                            [("index_score_tiled_maxima", "index_score_tiled_kernel<4, 1, false>", SCORE_SOURCES),
                             ("index_score_tiled_cands", "index_score_tiled_kernel<4, 2, false>", SCORE_SOURCES),
                             ("csa_attend", "attend_dma_kernel<2>", ATTEND_SOURCES)])}
SQ_COUNTERS = ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVES",
               "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE"]


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def _f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def set_recall(ref, got):
    """Mean over rows of |ref set & got set| / |ref set| (entries >= 0)."""
    ref, got = ref.reshape(-1, ref.shape[-1]).cpu().numpy(), got.reshape(-1, got.shape[-1]).cpu().numpy()
    fr = []
    for a, b in zip(ref, got):
        a = a[a >= 0]
        fr.append(len(np.intersect1d(a, b[b >= 0])) / max(1, len(a)))
    return float(np.mean(fr))


def csa_decode_setup(d, copies, q_pos=None):
    """One CSA decode step over d; q_pos (int64 [B] on the GPU) makes the batch
    ragged, with d["q_pos0"] as the bound."""
    base = {"E": _bf16(d["E"]), "kI": _bf16(d["kI"]), "q": _bf16(d["q"]), "qI": _bf16(d["qI"]),
            "win": _bf16(d["win"]), "w": _f32(d["w"]), "sink": _f32(d["sink"])}
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]
    B, H, D, m, k = d["B"], d["H"], d["D"], d["m"], d["k"]
    N = d["E"].shape[1]
    ws_i = torch.empty(L.csa_index_topk_workspace(L.BF16, B, 1, d["H_I"], d["d_I"], N, m, k, d["q_pos0"]),
                       dtype=torch.uint8, device=DEV)
    ws_a = torch.empty(L.csa_attend_workspace(L.BF16, L.BF16, B, 1, H, D, N, m, k, d["W"], d["q_pos0"]),
                       dtype=torch.uint8, device=DEV)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=DEV)

    def step(i):
        s = sets[i % copies]
        L.csa_index_topk(L.BF16, s["qI"], s["w"], s["kI"], idx, m=m, k=k, q_pos0=d["q_pos0"], ws=ws_i,
                         q_pos=q_pos)
        L.csa_attend(L.BF16, L.BF16, s["q"], s["E"], idx, s["win"], s["sink"], out, m=m, W=d["W"],
                     q_pos0=d["q_pos0"], scale=1 / math.sqrt(D), flags=L.INV_ROPE, rope_dims=64, ws=ws_a,
                     q_pos=q_pos)

    def recall():
        """Top-k on bf16-rounded scores against top-k on fp32 scores, same inputs."""
        got = {}
        for fl in (0, L.SCORE_BF16):
            got[fl] = torch.empty_like(idx)
            L.csa_index_topk(L.BF16, base["qI"], base["w"], base["kI"], got[fl], m=m, k=k, q_pos0=d["q_pos0"],
                             flags=fl, ws=ws_i)
        torch.cuda.synchronize()
        return set_recall(got[0], got[L.SCORE_BF16])
    step.recall = recall
    return step


def hca_decode_setup(d, copies, q_pos=None):
    base = {"E": _bf16(d["E"]), "q": _bf16(d["q"]), "win": _bf16(d["win"]), "sink": _f32(d["sink"])}
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]
    B, H, D = d["B"], d["H"], d["D"]
    N = d["E"].shape[1]
    ws = torch.empty(L.hca_attend_workspace(L.BF16, L.BF16, B, 1, H, D, N, d["m"], d["W"], d["q_pos0"]),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=DEV)

    def step(i):
        s = sets[i % copies]
        L.hca_attend(L.BF16, L.BF16, s["q"], s["E"], s["win"], s["sink"], out, m=d["m"], W=d["W"],
                     q_pos0=d["q_pos0"], scale=1 / math.sqrt(D), flags=L.INV_ROPE, rope_dims=64, ws=ws,
                     q_pos=q_pos)
    return step


def mixed_pair_setup(B=64, ctx=1048576, H=128, D=512, H_I=4, d_I=128, k=1024, m=4, m2=128, W=128, seed=5):
    """Mixed-precision CSA + HCA layer pair at decode (B = 64, 1048576 tokens).

    Same recipe as the parity workload (entries, keys and windows N(0,1)/sqrt(dim)
    in float32, queries with Student-t (3) norms, head weights N(0,1)/sqrt(H_I)),
    but the 10 GB of sources are drawn on the GPU with torch's seeded generator,
    one sequence at a time, and quantised by the library (KV_MIXED rows, MXFP4
    indexer operands) as the path stores them. The small query tensors come from
    numpy streams default_rng([seed, 2_000_000 + b]).
    """
    N, N2 = ctx // m, ctx // m2
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    u8 = dict(dtype=torch.uint8, device=DEV)
    Eq = torch.empty((B, N, D + 64), **u8)
    Es = torch.empty((B, N), dtype=torch.float32, device=DEV)
    kc = torch.empty((B, N, d_I // 2), **u8)
    ks = torch.empty((B, N, d_I // 32), **u8)
    Wq = torch.empty((B, W, D + 64), **u8)
    Ws = torch.empty((B, W), dtype=torch.float32, device=DEV)
    E2q = torch.empty((B, N2, D + 64), **u8)
    E2s = torch.empty((B, N2), dtype=torch.float32, device=DEV)
    W2q = torch.empty((B, W, D + 64), **u8)
    W2s = torch.empty((B, W), dtype=torch.float32, device=DEV)
    qc = torch.empty((B, 1, H_I, d_I // 2), **u8)
    qs = torch.empty((B, 1, H_I, d_I // 32), **u8)

    def randn(*shape):
        return torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32) / math.sqrt(shape[-1])

    def student_t_rows(r, shape):
        g = r.standard_normal(size=shape)
        tau = r.standard_t(3, size=shape[:-1])
        return (g / np.linalg.norm(g, axis=-1, keepdims=True) * np.abs(tau)[..., None]).astype(np.float32)

    q = np.empty((B, 1, H, D), np.float32)
    q2 = np.empty((B, 1, H, D), np.float32)
    qI = np.empty((B, 1, H_I, d_I), np.float32)
    w = np.empty((B, 1, H_I), np.float32)
    for b in range(B):
        L.lca_quantize_rows(L.KV_MIXED, randn(N, D), Eq[b], Es[b])
        L.lca_quantize_rows(L.MXFP4, randn(N, d_I), kc[b], ks[b])
        L.lca_quantize_rows(L.KV_MIXED, randn(W, D), Wq[b], Ws[b])
        L.lca_quantize_rows(L.KV_MIXED, randn(N2, D), E2q[b], E2s[b])
        L.lca_quantize_rows(L.KV_MIXED, randn(W, D), W2q[b], W2s[b])
        r = np.random.default_rng([seed, 2_000_000 + b])
        q[b] = student_t_rows(r, (1, H, D))
        qI[b] = student_t_rows(r, (1, H_I, d_I))
        w[b] = r.standard_normal((1, H_I)) / np.sqrt(H_I)
        q2[b] = student_t_rows(r, (1, H, D))
    torch.cuda.synchronize()
    L.lca_quantize_rows(L.MXFP4, _f32(qI), qc, qs)
    q_t, q2_t, w_t = _bf16(q), _bf16(q2), _f32(w)
    r = np.random.default_rng([seed, 1_000_000])
    sink, sink2 = _f32(r.standard_normal(H)), _f32(r.standard_normal(H))
    ws_i = torch.empty(L.csa_index_topk_workspace(L.MXFP4, B, 1, H_I, d_I, N, m, k, ctx, L.SCORE_BF16), **u8)
    ws_c = torch.empty(L.csa_attend_workspace(L.BF16, L.KV_MIXED, B, 1, H, D, N, m, k, W, ctx), **u8)
    ws_h = torch.empty(L.hca_attend_workspace(L.BF16, L.KV_MIXED, B, 1, H, D, N2, m2, W, ctx), **u8)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=DEV)
    out2 = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=DEV)
    scale = 1 / math.sqrt(D)

    def step(i):
        L.csa_index_topk(L.MXFP4, qc, w_t, kc, idx, m=m, k=k, q_pos0=ctx, d_I=d_I, qI_scale=qs, kI_scale=ks,
                         flags=L.SCORE_BF16, ws=ws_i)
        L.csa_attend(L.BF16, L.KV_MIXED, q_t, Eq, idx, Wq, sink, out, m=m, W=W, q_pos0=ctx, scale=scale,
                     kv_scale=Es, win_scale=Ws, flags=L.INV_ROPE, rope_dims=64, ws=ws_c)
        L.hca_attend(L.BF16, L.KV_MIXED, q2_t, E2q, W2q, sink2, out2, m=m2, W=W, q_pos0=ctx, scale=scale,
                     kv_scale=E2s, win_scale=W2s, flags=L.INV_ROPE, rope_dims=64, ws=ws_h)

    def recall():
        """MXFP4 indexer: top-k on bf16-rounded scores against top-k on fp32 scores."""
        got = {}
        for fl in (0, L.SCORE_BF16):
            got[fl] = torch.empty_like(idx)
            L.csa_index_topk(L.MXFP4, qc, w_t, kc, got[fl], m=m, k=k, q_pos0=ctx, d_I=d_I, qI_scale=qs,
                             kI_scale=ks, flags=fl, ws=ws_i)
        torch.cuda.synchronize()
        return set_recall(got[0], got[L.SCORE_BF16])
    step.recall = recall

    # algorithmic bytes: every MXFP4 key (64 B + 4 B scales), the selected and
    # window mixed rows (576 B + 4 B scale), every HCA mixed row, q and out
    row = D + 64 + 4
    nbytes = B * (N * (d_I // 2 + d_I // 32) + H_I * (d_I // 2 + d_I // 32) + H_I * 4
                  + (k + W) * row + (N2 + W) * row + 2 * 2 * H * D * 2)
    flops = B * (2.0 * N * H_I * d_I + 4.0 * H * (k + W) * D + 4.0 * H * (N2 + W) * D)
    return step, nbytes, flops


def csa_prefill_setup(d):
    """CSA chunked prefill: compress the 4096 new tokens (entries with RMSNorm
    and RoPE, indexer keys plain) into the cache after the 262144-entry prefix,
    score and select top-1024 for every new query, attend."""
    m, D, dI, Tq, N0, N_cap = d["m"], d["D"], d["d_I"], d["Tq"], d["N0"], d["N_cap"]
    E = torch.empty((1, N_cap, D), dtype=torch.bfloat16, device=DEV)
    KI = torch.empty((1, N_cap, dI), dtype=torch.bfloat16, device=DEV)
    E[:, :N0] = _bf16(d["E_prefix"])
    KI[:, :N0] = _bf16(d["kI_prefix"])
    t = {n: _bf16(d[n]) for n in ("cb", "ca", "prev_ca", "icb", "ica", "iprev_ca", "q", "qI", "win")}
    t.update({n: _f32(d[n]) for n in ("zb", "za", "prev_za", "izb", "iza", "iprev_za", "w", "sink", "norm_w")})
    k, H = d["k"], d["H"]
    ws_i = torch.empty(L.csa_index_topk_workspace(L.BF16, 1, Tq, d["H_I"], dI, N_cap, m, k, d["q_pos0"]),
                       dtype=torch.uint8, device=DEV)
    ws_a = torch.empty(L.csa_attend_workspace(L.BF16, L.BF16, 1, Tq, H, D, N_cap, m, k, d["W"], d["q_pos0"]),
                       dtype=torch.uint8, device=DEV)
    idx = torch.empty((1, Tq, k), dtype=torch.int32, device=DEV)
    out = torch.empty((1, Tq, H, D), dtype=torch.bfloat16, device=DEV)

    def step(i):
        L.csa_compress(L.BF16, L.BF16, t["cb"], t["zb"], m, ca=t["ca"], za=t["za"], prev_ca=t["prev_ca"],
                       prev_za=t["prev_za"], pos0=d["pos0"], flags=L.NORM | L.ROPE, norm_w=t["norm_w"],
                       eps=d["eps"], rope_base=d["rope_base"], rope_dims=d["rope_dims"], out=E[:, N0:],
                       out_rows=N_cap)
        L.csa_compress(L.BF16, L.BF16, t["icb"], t["izb"], m, ca=t["ica"], za=t["iza"], prev_ca=t["iprev_ca"],
                       prev_za=t["iprev_za"], pos0=d["pos0"], out=KI[:, N0:], out_rows=N_cap)
        L.csa_index_topk(L.BF16, t["qI"], t["w"], KI, idx, m=m, k=k, q_pos0=d["q_pos0"], ws=ws_i)
        L.csa_attend(L.BF16, L.BF16, t["q"], E, idx, t["win"], t["sink"], out, m=m, W=d["W"], q_pos0=d["q_pos0"],
                     scale=1 / math.sqrt(D), flags=L.INV_ROPE, rope_dims=d["rope_dims"], ws=ws_a)

    # algorithmic FLOPs: indexer QK over every visible key for every query and
    # head, attention QK + PV over the k selected + window rows of every query
    nv = [(d["q_pos0"] + tt + 1) // m for tt in range(Tq)]
    flops = 2.0 * d["H_I"] * dI * sum(nv) + 4.0 * H * D * Tq * (k + d["W"])
    return step, flops


def small_layer_leg(steps, warmup):
    """Workload 1: one fp32 CSA layer forward over 1024 causal tokens from
    position 0 (8 heads, D = 128, indexer 4 x 64, k = 64): both compressions
    (entries with RMSNorm + RoPE, indexer keys), index top-k and attention.
    Returns the generated inputs (the oracle sample reuses them) and the leg."""
    d = WL.make_csa_layer()
    B, T, D, m, dI, H_I, k, H, W = d["B"], d["T"], d["D"], d["m"], d["d_I"], d["H_I"], d["k"], d["H"], d["W"]
    t = {n: _f32(d[n]) for n in ("ca", "za", "cb", "zb", "ica", "iza", "icb", "izb", "q", "qI", "w", "win",
                                 "sink", "norm_w")}
    N = T // m
    E = torch.empty((B, N, D), dtype=torch.float32, device=DEV)
    KI = torch.empty((B, N, dI), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    out = torch.empty((B, T, H, D), dtype=torch.float32, device=DEV)
    ws_i = torch.empty(L.csa_index_topk_workspace(L.F32, B, T, H_I, dI, N, m, k, 0), dtype=torch.uint8, device=DEV)
    ws_a = torch.empty(L.csa_attend_workspace(L.F32, L.F32, B, T, H, D, N, m, k, W, 0), dtype=torch.uint8,
                       device=DEV)

    def step(i):
        L.csa_compress(L.F32, L.F32, t["cb"], t["zb"], m, ca=t["ca"], za=t["za"], pos0=0, flags=L.NORM | L.ROPE,
                       norm_w=t["norm_w"], eps=d["eps"], rope_base=d["rope_base"], rope_dims=d["rope_dims"], out=E)
        L.csa_compress(L.F32, L.F32, t["icb"], t["izb"], m, ca=t["ica"], za=t["iza"], pos0=0, out=KI)
        L.csa_index_topk(L.F32, t["qI"], t["w"], KI, idx, m=m, k=k, q_pos0=0, ws=ws_i)
        L.csa_attend(L.F32, L.F32, t["q"], E, idx, t["win"], t["sink"], out, m=m, W=W, q_pos0=0,
                     scale=1 / math.sqrt(D), flags=L.INV_ROPE, rope_dims=d["rope_dims"], ws=ws_a)

    el = timed(step, steps, warmup)
    ms = 1e3 * el / steps
    kt = kernel_times(step, steps)
    progress(f"csa layer fp32: {ms:.4f} ms/step")
    return d, {"workload": "csa_layer_fp32_t1024_h8_d128", "tokens_per_s": B * T / (ms * 1e-3), "ms_per_step": ms,
               "kernels_us": per_step(kt), "kernel_launches_per_step": launches(kt), "dtype": "f32"}


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def timed(step, steps, warmup):
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def kernel_times(step, steps):
    """Per-kernel durations from HIP events the library records around its
    launches on the caller's stream: launches per step, the average duration
    of one launch, and the time per step (a chunked call launches a kernel
    several times per step)."""
    torch.cuda.synchronize()
    L.lca_profile_collect()
    L.lca_profile_enable(True)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    L.lca_profile_enable(False)
    stats = L.lca_profile_collect()
    return {name: {"launches_per_step": n / steps, "avg_us": 1e3 * ms / n, "us_per_step": 1e3 * ms / steps}
            for name, (n, ms) in stats.items()}


def per_step(kt, nd=3):
    """{kernel: microseconds per step} (the sum over a step's launches)."""
    return {k: round(v["us_per_step"], nd) for k, v in kt.items()}


def launches(kt):
    """{kernel: launches per step}."""
    return {k: v["launches_per_step"] for k, v in kt.items()}


def csa_decode_bytes(d):
    """Algorithmic HBM bytes of one CSA decode step (what the method must move)."""
    B, H, D, k, W = d["B"], d["H"], d["D"], d["k"], d["W"]
    N, H_I, d_I = d["E"].shape[1], d["H_I"], d["d_I"]
    index = B * (N * d_I * 2 + H_I * d_I * 2 + H_I * 4)      # every indexer key once, queries, weights
    attend = B * ((k + W) * D * 2 + 2 * H * D * 2)           # selected + window rows, q and out
    return index, attend


def hca_decode_bytes(d):
    B, H, D, W = d["B"], d["H"], d["D"], d["W"]
    N = d["E"].shape[1]
    return B * ((N + W) * D * 2 + 2 * H * D * 2)


def decode_state_leg(d, copies, steps, warmup, headline_ms):
    """The headline step preceded by the decode-time state updates of the token
    it decodes: append it to the entry compressor (RMSNorm + RoPE, bf16 cache)
    and to the indexer-key compressor (both m = 4 with overlap), store its raw
    row in the 128-row window ring, then index top-k + attention reading the
    window from the ring. The token sits at position ctx - 1, so each step
    closes a block and writes one entry and one key per sequence (the most
    work an append does)."""
    B, H, D, m, k, W = d["B"], d["H"], d["D"], d["m"], d["k"], d["W"]
    N, H_I, d_I = d["E"].shape[1], d["H_I"], d["d_I"]
    p = d["q_pos0"] - 1
    g = torch.Generator(device=DEV)
    g.manual_seed(21)

    def rnd(*shape, scale=1.0):
        return (torch.randn(*shape, generator=g, device=DEV) * scale).to(torch.bfloat16)
    sets = []
    for c in range(copies):
        sets.append({"E": _bf16(d["E"]), "kI": _bf16(d["kI"]), "q": _bf16(d["q"]), "qI": _bf16(d["qI"]),
                     "w": _f32(d["w"]), "ring": rnd(B, W, D, scale=D ** -0.5),
                     "ca": rnd(B, D, scale=D ** -0.5), "cb": rnd(B, D, scale=D ** -0.5),
                     "ica": rnd(B, d_I, scale=d_I ** -0.5), "icb": rnd(B, d_I, scale=d_I ** -0.5),
                     "kvw": rnd(B, D, scale=D ** -0.5),
                     "z": torch.randn(4, B, generator=g, device=DEV)})
    sink = _f32(d["sink"])
    norm_w = torch.ones(D, dtype=torch.float32, device=DEV)
    stE = torch.zeros(L.csa_compress_state_bytes(L.BF16, B, D, m, True), dtype=torch.uint8, device=DEV)
    stK = torch.zeros(L.csa_compress_state_bytes(L.BF16, B, d_I, m, True), dtype=torch.uint8, device=DEV)
    qp = torch.full((B,), p, dtype=torch.int64, device=DEV)
    ws_i = torch.empty(L.csa_index_topk_workspace(L.BF16, B, 1, H_I, d_I, N, m, k, p), dtype=torch.uint8,
                       device=DEV)
    ws_a = torch.empty(L.csa_attend_workspace(L.BF16, L.BF16, B, 1, H, D, N, m, k, W, p), dtype=torch.uint8,
                       device=DEV)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=DEV)

    for s in sets:                 # the three appends of a step as one launch (lca_decode_append)
        s["jobs"] = [L.append_job_compress(L.BF16, L.BF16, s["cb"], s["z"][1], m, stE, s["E"], ca=s["ca"],
                                           za=s["z"][0], flags=L.NORM | L.ROPE, norm_w=norm_w, rope_dims=64),
                     L.append_job_compress(L.BF16, L.BF16, s["icb"], s["z"][3], m, stK, s["kI"], ca=s["ica"],
                                           za=s["z"][2]),
                     L.append_job_window(L.BF16, L.BF16, s["kvw"], s["ring"])]

    def decode(s):
        L.csa_index_topk(L.BF16, s["qI"], s["w"], s["kI"], idx, m=m, k=k, q_pos0=p, ws=ws_i)
        L.csa_attend(L.BF16, L.BF16, s["q"], s["E"], idx, s["ring"], sink, out, m=m, W=W, q_pos0=p,
                     scale=1 / math.sqrt(D), flags=L.INV_ROPE | L.WIN_RING, rope_dims=64, ws=ws_a)

    def step(i):
        s = sets[i % copies]
        L.lca_decode_append(s["jobs"], qp, pos_max=p)
        decode(s)

    def step_separate(i):
        s = sets[i % copies]
        L.csa_compress_append(L.BF16, L.BF16, s["cb"], s["z"][1], m, qp, stE, s["E"], pos_max=p, ca=s["ca"],
                              za=s["z"][0], flags=L.NORM | L.ROPE, norm_w=norm_w, rope_dims=64)
        L.csa_compress_append(L.BF16, L.BF16, s["icb"], s["z"][3], m, qp, stK, s["kI"], pos_max=p, ca=s["ica"],
                              za=s["z"][2])
        L.lca_window_append(L.BF16, L.BF16, s["kvw"], qp, s["ring"], pos_max=p)
        decode(s)
    ms = 1e3 * timed(step, steps, warmup) / steps
    kt = kernel_times(step, steps)
    ms_sep = 1e3 * timed(step_separate, steps, warmup) / steps
    kt_sep = kernel_times(step_separate, steps)
    progress(f"csa decode step with state updates: {ms:.4f} ms/step ({ms_sep:.4f} with separate appends)")
    return {"workload": "csa_decode_step_with_state_b16_ctx131072", "tokens_per_s": B / (ms * 1e-3),
            "ms_per_step": ms, "headline_ms": headline_ms, "state_update_ms": ms - headline_ms,
            "kernels_us": per_step(kt, 3),
            "separate_appends": {"ms_per_step": ms_sep,
                                 "kernels_us": per_step(kt_sep, 3)}}


def placement_leg(batches=(16, 64, 256, 512), steps=50, warmup=5, ctx=131072, H=64, D=512, k=512, W=128, m=4):
    """CSA attention (csa_attend: selected entries + window + sink) at decode,
    with the query's splits placed one workgroup per split + combine
    (LCA_SPLITS_MANY_WG) or all in one workgroup (LCA_SPLITS_ONE_WG), at
    growing batch sizes; both give the same bits. Inputs are drawn on the GPU
    (bf16 N(0,1)/sqrt(D) rows, uniform random selections); four selection sets
    rotate so that the 256 MB last-level cache cannot hold a step's rows."""
    N = ctx // m
    g = torch.Generator(device=DEV)
    g.manual_seed(31)
    res = {}
    for B in batches:
        E = torch.randn(B, N, D, generator=g, device=DEV, dtype=torch.bfloat16) * (D ** -0.5)
        q = torch.randn(B, 1, H, D, generator=g, device=DEV, dtype=torch.bfloat16) * (D ** -0.5)
        win = torch.randn(B, W, D, generator=g, device=DEV, dtype=torch.bfloat16) * (D ** -0.5)
        sink = torch.randn(H, generator=g, device=DEV)
        idxs = [torch.randint(0, N, (B, 1, k), generator=g, device=DEV, dtype=torch.int32) for _ in range(4)]
        ws = torch.empty(L.csa_attend_workspace(L.BF16, L.BF16, B, 1, H, D, N, m, k, W, ctx), dtype=torch.uint8,
                         device=DEV)
        out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=DEV)
        row = {}
        for name, fl in (("split_per_workgroup", L.SPLITS_MANY_WG), ("query_per_workgroup", L.SPLITS_ONE_WG)):
            def step(i, fl=fl):
                L.csa_attend(L.BF16, L.BF16, q, E, idxs[i % 4], win, sink, out, m=m, W=W, q_pos0=ctx,
                             scale=1 / math.sqrt(D), flags=L.INV_ROPE | fl, rope_dims=64, ws=ws)
            us = 1e6 * timed(step, steps, warmup) / steps
            kt = kernel_times(step, steps)
            row[name] = {"us_per_call": round(us, 2), "kernels_us": per_step(kt, 2)}
        rows_bytes = B * (k + W) * D * 2
        for v in row.values():
            v["rows_GBs"] = round(rows_bytes / (v["us_per_call"] * 1e-6) / 1e9, 1)
        row["speedup_query_per_workgroup"] = round(row["split_per_workgroup"]["us_per_call"] /
                                                   row["query_per_workgroup"]["us_per_call"], 3)
        res[f"B{B}"] = row
        progress(f"placement B={B}: {row['split_per_workgroup']['us_per_call']:.1f} us split / "
                 f"{row['query_per_workgroup']['us_per_call']:.1f} us one workgroup")
        del E, q, win, idxs, ws, out
        torch.cuda.empty_cache()
    return res


def outproj_leg(steps=50, warmup=5):
    """Grouped output projection (lca_grouped_out_proj) at the pages' shapes:
    Flash (64 heads x 512 -> 8 groups x 1024 -> 4096) at decode batch 16 and
    a 4096-row prefill chunk, Pro (128 heads -> 16 x 1024 -> 7168) at batch
    64. bf16 weights drawn on the GPU; enough weight copies rotate that the
    256 MB last-level cache cannot serve a step's weights from the last one."""
    g_ = torch.Generator(device=DEV)
    g_.manual_seed(41)
    res = {}
    for name, T, n_h, g, d_model in (("flash_decode_b16", 16, 64, 8, 4096), ("pro_decode_b64", 64, 128, 16, 7168),
                                     ("flash_prefill_t4096", 4096, 64, 8, 4096)):
        c, d_g = 512, 1024
        kg = n_h // g * c
        wbytes = 2 * (g * d_g * kg + d_model * g * d_g)
        copies = max(1, -(-3 * 256 * 2 ** 20 // wbytes)) if T <= 64 else 1
        sets = [(torch.randn(g, d_g, kg, generator=g_, device=DEV, dtype=torch.bfloat16) * kg ** -0.5,
                 torch.randn(d_model, g * d_g, generator=g_, device=DEV, dtype=torch.bfloat16) * (g * d_g) ** -0.5)
                for _ in range(copies)]
        o = torch.randn(T, n_h, c, generator=g_, device=DEV, dtype=torch.bfloat16)
        mid = torch.empty((T, g * d_g), dtype=torch.bfloat16, device=DEV)
        out = torch.empty((T, d_model), dtype=torch.bfloat16, device=DEV)

        def step(i):
            wg, wo = sets[i % copies]
            L.lca_grouped_out_proj(o, wg, wo, out, mid=mid)
        n = steps if T <= 64 else 5
        us = 1e6 * timed(step, n, warmup if T <= 64 else 1) / n
        kt = kernel_times(step, n)
        abytes = wbytes + 2 * (T * n_h * c + 2 * T * g * d_g + T * d_model)
        flops = 2.0 * T * (g * d_g * kg + d_model * g * d_g)
        res[name] = {"rows": T, "us_per_call": round(us, 2), "weight_copies_rotated": copies,
                     "kernels_us": per_step(kt, 2),
                     "algorithmic_bytes": abytes, "achieved_GBs": round(abytes / (us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(abytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
                     "flops": flops, "achieved_TFLOPs": round(flops / (us * 1e-6) / 1e12, 1),
                     "mfma_bf16_frac": round(flops / (us * 1e-6) / 2.5e15, 3)}
        progress(f"grouped out proj {name}: {us:.1f} us")
        del sets, o, mid, out
        torch.cuda.empty_cache()
    return res


def backward_leg(T=4096, H=64, D=512, k=512, W=128, m=4, H_I=4, d_I=128, reps=5):
    """Training-shaped CSA attention backward: one sequence of T = 4096 tokens
    from the start (causal: query t reads the top-k of its (t + 1) // 4
    visible entries, made by the library's own indexer from random indexer
    inputs, plus its window), Flash shape (64 heads x 512, k = 512). The
    forward runs first (untimed) to give out and lse; the timed call is
    csa_attend_backward (dq, entry and window gradients, dsink)."""
    g = torch.Generator(device=DEV)
    g.manual_seed(51)
    N = T // m
    q = torch.randn(1, T, H, D, generator=g, device=DEV, dtype=torch.bfloat16) * (4 * D ** -0.5)
    E = torch.randn(1, N, D, generator=g, device=DEV, dtype=torch.bfloat16) * (D ** -0.5)
    win = torch.randn(1, W - 1 + T, D, generator=g, device=DEV, dtype=torch.bfloat16) * (D ** -0.5)
    sink = torch.randn(H, generator=g, device=DEV)
    qI = torch.randn(1, T, H_I, d_I, generator=g, device=DEV, dtype=torch.bfloat16) * (d_I ** -0.5)
    kI = torch.randn(1, N, d_I, generator=g, device=DEV, dtype=torch.bfloat16) * (d_I ** -0.5)
    w = torch.randn(1, T, H_I, generator=g, device=DEV) * (H_I ** -0.5)
    idx = torch.empty((1, T, k), dtype=torch.int32, device=DEV)
    L.csa_index_topk(L.BF16, qI, w, kI, idx, m=m, k=k, q_pos0=0)
    out = torch.empty((1, T, H, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, T, H), dtype=torch.float32, device=DEV)
    kw = dict(m=m, W=W, q_pos0=0, scale=1 / math.sqrt(D), flags=L.INV_ROPE, rope_dims=64)
    L.csa_attend(L.BF16, L.BF16, q, E, idx, win, sink, out, lse_out=lse, **kw)
    dout = torch.randn(1, T, H, D, generator=g, device=DEV, dtype=torch.bfloat16)
    need = int(L.lib().csa_attend_backward_workspace(L.BF16, L.BF16, 1, T, H, D, N, m, k, W, 0))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)

    def step(i):
        L.attend_backward("csa", q, E, win, sink, out, lse, dout, idx=idx, ws=ws, **kw)
    ms = 1e3 * timed(step, reps, 1) / reps
    kt = kernel_times(step, reps)
    # rows read: each query's selected entries (k, fewer early on) and its window
    rows = sum(min(k, (t + 1) // m) + min(W, t + 1) for t in range(T))
    flops = 2.0 * rows * H * D * 5                  # S, dP, dq (query side) + two head sums (row side)
    progress(f"csa attend backward T={T}: {ms:.3f} ms")
    return {"workload": "csa_attend_backward_t4096_flash", "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
            "kernels_us": per_step(kt, 1), "rows_read": rows, "flops": flops,
            "achieved_TFLOPs": flops / (ms * 1e-3) / 1e12, "mfma_bf16_frac": flops / (ms * 1e-3) / 2.5e15,
            "workspace_bytes": need}


def ragged_bytes(d, pos):
    """Algorithmic bytes of a ragged decode step: each sequence moves what its
    own position makes visible (indexer keys and, for HCA, entries)."""
    H, D, W, m = d["H"], d["D"], d["W"], d["m"]
    nv = [min((int(p) + 1) // m, d["E"].shape[1]) for p in pos]
    if "kI" in d:
        k, H_I, d_I = d["k"], d["H_I"], d["d_I"]
        return sum(n * d_I * 2 + H_I * d_I * 2 + H_I * 4 + (min(k, n) + W) * D * 2 + 2 * H * D * 2
                   for n in nv)
    return sum((n + W) * D * 2 + 2 * H * D * 2 for n in nv)


def ragged_leg(d, copies, steps, warmup, seed, uniform_ms):
    """The same decode batch with each sequence at its own position, drawn
    uniformly from [window, context] (last one at the context: the bound)."""
    pos = WL.ragged_positions(seed, d["B"], d["W"], d["q_pos0"])
    qp = torch.from_numpy(pos).to(DEV)
    setup = csa_decode_setup if "kI" in d else hca_decode_setup
    rstep = setup(d, copies, q_pos=qp)
    rms = 1e3 * timed(rstep, steps, warmup) / steps
    rk = kernel_times(rstep, steps)
    rb = ragged_bytes(d, pos)
    progress(f"ragged {'csa' if 'kI' in d else 'hca'} decode: {rms:.4f} ms/step")
    return {"tokens_per_s": d["B"] / (rms * 1e-3), "ms_per_step": rms,
            "mean_context": float(np.mean(pos)), "bound": d["q_pos0"],
            "uniform_at_bound_ms": uniform_ms, "speedup_vs_uniform_at_bound": uniform_ms / rms,
            "kernels_us": per_step(rk, 3),
            "algorithmic_bytes": rb, "achieved_GBs": rb / (rms * 1e-3) / 1e9,
            "hbm_frac": rb / (rms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def csa_prefill_flops_split(Tq=4096, ctx=1048576, m=4, H_I=4, d_I=128, H=128, D=512, k=1024, W=128):
    """Algorithmic flops of the prefill's indexer scoring (every visible key of
    every query, H_I heads of d_I) and of its attention (k selected + W window
    rows per query and head, QK^T and PV)."""
    nv = sum((ctx + t + 1) // m for t in range(Tq))
    return 2.0 * nv * H_I * d_I, 4.0 * Tq * H * (k + W) * D


def mixed_hca_work(B=64, ctx=1048576, m2=128, H=128, D=512, W=128):
    """Flops and HBM bytes of the mixed pair's HCA attention: every entry and
    window row (576 stored bytes + a 4-byte scale) for all heads, q in, out."""
    rows = ctx // m2 + W
    return 4.0 * B * H * rows * D, B * (rows * (D + 64 + 4) + 2 * H * D * 2)


def hca_decode_flops(d):
    B, H, D, W = d["B"], d["H"], d["D"], d["W"]
    N = d["E"].shape[1]
    return 4.0 * B * H * (N + W) * D


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, src_hash):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        rec = json.load(open(path))[workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration(mib, reps=COPY_REPS):
    """Plain device-to-device copies of a known size, for scaling the HBM byte
    counters (FETCH_SIZE, WRITE_SIZE) that rocprofv3 reports per dispatch."""
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=DEV)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return n


def _read_counter_csv(path, counter):
    """(dispatch id, kernel name, grid size, value in KiB) of every dispatch in a
    rocprofv3 counter_collection.csv, for one counter, in dispatch order."""
    import csv
    rows = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                rows.append((int(row["Dispatch_Id"]), row["Kernel_Name"], int(row["Grid_Size"]),
                             float(row["Counter_Value"])))
    rows.sort()
    return rows


def _merge_json(path, workload, recs):
    try:
        allrec = json.load(open(path))
    except (OSError, ValueError):
        allrec = {}
    allrec.setdefault(workload, {}).update(recs)
    with open(path, "w") as f:
        json.dump(allrec, f, indent=1)


def pmc_summary(leg, fetch_csv, write_csv, copy_mib, out_json):
    """Turn two rocprofv3 --pmc runs of ``bench.py --only LEG --copy-calibration
    MIB`` (one with FETCH_SIZE, one with WRITE_SIZE) into HBM bytes per launch of
    the leg's kernels. Each counter is scaled by what it reads for the plain copy
    of known size: the last COPY_REPS copy dispatches of the run."""
    n = copy_mib << 20
    workload, kernels = TRAFFIC_KERNELS[leg]

    def stats(path, counter):
        rows = _read_counter_csv(path, counter)
        copies = [r for r in rows if "copyBuffer" in r[1]][-COPY_REPS:]
        if len(copies) < COPY_REPS:
            raise SystemExit(f"{path}: calibration copies missing")
        out = {}
        for key, pat, _ in kernels:
            ks = [r for r in rows if pat in r[1]]
            if ks:
                out[key] = (sum(r[3] for r in ks) / len(ks), ks[0][1], len(ks))
        return sum(r[3] for r in copies) / len(copies), out

    cf, kf = stats(fetch_csv, "FETCH_SIZE")
    cw, kw = stats(write_csv, "WRITE_SIZE")
    f_scale, w_scale = n / (cf * 1024.0), n / (cw * 1024.0)
    recs = {}
    for key, pat, srcs in kernels:
        if key not in kf or key not in kw:
            continue
        fb, wb = kf[key][0] * 1024.0 * f_scale, kw[key][0] * 1024.0 * w_scale
        recs[key] = {"source_hash": source_hash(srcs), "kernel": kf[key][1], "dispatches": kf[key][2],
                     "fetch_kib_raw": kf[key][0], "write_kib_raw": kw[key][0], "copy_bytes": n,
                     "copy_fetch_kib_raw": cf, "copy_write_kib_raw": cw,
                     "fetch_scale": f_scale, "write_scale": w_scale,
                     "hbm_read_bytes_per_launch": fb, "hbm_write_bytes_per_launch": wb,
                     "hbm_bytes_per_launch": fb + wb}
    _merge_json(out_json, workload, recs)
    print(json.dumps({workload: recs}, indent=1))


def sq_summary(leg, csv_path, out_json):
    """MFMA counters per dispatch (averaged over the leg's dispatches of each
    kernel) from one rocprofv3 --pmc run with SQ_COUNTERS. MFMA busy is
    SQ_VALU_MFMA_BUSY_CYCLES (SIMD-cycles of matrix-core work: the bf16 flops
    over 1024) over the kernel's cycles times the 4 SIMDs of each of the 256
    CUs; the kernel's cycles are GRBM_GUI_ACTIVE over the 8 XCDs, whose
    counts it sums. Flops are the bf16 MFMA ops counter times 512."""
    import csv
    workload, kernels = MFMA_KERNELS[leg]
    per = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            for key, pat, _ in kernels:
                if pat in row["Kernel_Name"]:
                    d = per.setdefault(key, {"kernel": row["Kernel_Name"], "dispatch": set(), "sum": {}})
                    d["dispatch"].add(row["Dispatch_Id"])
                    d["sum"][row["Counter_Name"]] = d["sum"].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    recs = {}
    for key, pat, srcs in kernels:
        if key not in per:
            continue
        d = per[key]
        nd = len(d["dispatch"])
        c = {k: v / nd for k, v in d["sum"].items()}
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / max(1.0, c.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD * N_CU * 4)
        recs[key] = {"source_hash": source_hash(srcs), "kernel": d["kernel"], "dispatches": nd,
                     "counters_per_dispatch": c, "mfma_busy_frac": busy,
                     "mfma_bf16_flops_per_dispatch": c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512}
    _merge_json(out_json, workload, recs)
    print(json.dumps({workload: recs}, indent=1))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(d, h, layer=None, samples=True, reps=3):
    """The float64 oracle on the host cores, on the same workloads: the whole
    CSA decode batch (indexer scores, top-k, attention for every sequence) and
    the whole HCA decode batch, each run ``reps`` times (median reported), with
    the BLAS threads numpy has by default and again with one thread. Beside
    them, with the default threads: the whole fp32 layer of workload 1 (median
    of ``reps``), and one run each of bounded samples of the prefill and the
    mixed pair (inputs generated outside the timed region)."""
    import oracle as O

    def csa_batch():
        D, m, k, W, B = d["D"], d["m"], d["k"], d["W"], d["B"]
        for b in range(B):
            nv = O.n_visible(d["q_pos0"], m)
            s = O.index_scores(d["qI"][b, 0], d["w"][b, 0], d["kI"][b], nv)
            sel = O.topk_select(s, k)
            O.csa_attend_query(d["q"][b, 0], d["E"][b], sel, d["win"][b], d["sink"], 1 / math.sqrt(D),
                               d["q_pos0"], d["q_pos0"], W, True, 10000.0, 64)
        return B

    def hca_batch():
        for b in range(h["B"]):
            O.hca_attend(h["q"][b], h["E"][b], h["m"], h["win"][b], h["sink"], 1 / math.sqrt(h["D"]),
                         h["q_pos0"], h["W"], True, 10000.0, 64)
        return h["B"]

    def median_rate(fn):
        rates = []
        for _ in range(reps):
            t0 = time.perf_counter()
            n = fn()
            rates.append(n / (time.perf_counter() - t0))
        return float(np.median(rates))

    def layer_run():
        x = layer
        m, R, T = x["m"], x["rope_dims"], x["T"]
        Eo = O.compress_epilogue(O.compress_sequence(x["cb"][0], x["zb"][0], m, x["ca"][0], x["za"][0]),
                                 0, m, x["norm_w"], x["eps"], x["rope_base"], R)
        Ko = O.compress_sequence(x["icb"][0], x["izb"][0], m, x["ica"][0], x["iza"][0])
        idx = np.full((T, x["k"]), -1, np.int64)
        for t in range(T):
            sel = O.topk_select(O.index_scores(x["qI"][0, t], x["w"][0, t], Ko, O.n_visible(t, m)), x["k"])
            idx[t, :len(sel)] = sel
        O.csa_attend(x["q"][0], Eo, idx, x["win"][0], x["sink"], 1 / math.sqrt(x["D"]), 0, x["W"], True,
                     x["rope_base"], R)
        return T

    cores = _blas_threads()
    res = {"csa": median_rate(csa_batch), "hca": median_rate(hca_batch)}
    extra = {}
    if layer is not None:
        extra["csa_layer_fp32"] = {"value": median_rate(layer_run), "unit": "tokens/s",
                                   "sample": f"the whole layer of 1024 tokens (both compressions, every query's "
                                             f"scores, top-k and attention), median of {reps} runs"}
    if samples:
        extra.update(oracle_samples(O))
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            res["csa_1t"] = median_rate(csa_batch)
            res["hca_1t"] = median_rate(hca_batch)
    except Exception:
        res["csa_1t"] = res["hca_1t"] = None
    return {"value": res["csa"], "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"the whole CSA decode batch ({d['B']} sequences at {d['q_pos0']} tokens), float64 numpy "
                      f"oracle (indexer scores, top-k, attention), median of {reps} runs",
            "value_1thread": res["csa_1t"], "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count(),
            "hca_decode": {"value": res["hca"], "value_1thread": res["hca_1t"], "unit": "tokens/s",
                           "sample": f"the whole HCA decode batch ({h['B']} sequences at {h['q_pos0']} tokens), "
                                     f"median of {reps} runs"}, **extra}


PREFILL_SAMPLE_ROWS = [0, 1, 1024, 2047, 3000, 4093, 4094, 4095]


def oracle_samples(O):
    """One run each (the cfg 4 / 5 rule) of the oracle on bounded samples:
    the prefill's compression of its 4096 new tokens (both streams) plus 8 of
    its queries (scores over 263168 keys, top-k 1024, attention over 1152 rows
    x 128 heads), reported as queries per second with the compression charged
    at 8/4096 of its time; and one sequence of the mixed pair (MXFP4 indexer
    operands, bf16 scores, top-k, attention over KV_MIXED rows, and the HCA
    layer over 8192 + 128 rows)."""
    out = {}
    pd = WL.make_csa_prefill(q_rows=PREFILL_SAMPLE_ROWS)
    m, D, R = pd["m"], pd["D"], pd["rope_dims"]
    t0 = time.perf_counter()
    E_new = O.compress_epilogue(O.compress_sequence(pd["cb"][0], pd["zb"][0], m, pd["ca"][0], pd["za"][0],
                                                    pd["prev_ca"][0], pd["prev_za"][0]),
                                pd["pos0"], m, pd["norm_w"], pd["eps"], pd["rope_base"], R)
    K_new = O.compress_sequence(pd["icb"][0], pd["izb"][0], m, pd["ica"][0], pd["iza"][0], pd["iprev_ca"][0],
                                pd["iprev_za"][0])
    t_comp = time.perf_counter() - t0
    E_all = np.concatenate([pd["E_prefix"][0], O.bf16_round(E_new)])
    K_all = np.concatenate([pd["kI_prefix"][0], O.bf16_round(K_new)])
    t0 = time.perf_counter()
    for t in PREFILL_SAMPLE_ROWS:
        p = pd["q_pos0"] + t
        sel = O.topk_select(O.index_scores(pd["qI"][0, t], pd["w"][0, t], K_all, O.n_visible(p, m)), pd["k"])
        O.csa_attend_query(pd["q"][0, t], E_all, sel, pd["win"][0], pd["sink"], 1 / math.sqrt(D), p, pd["q_pos0"],
                           pd["W"], True, pd["rope_base"], R)
    t_q = time.perf_counter() - t0
    nq = len(PREFILL_SAMPLE_ROWS)
    out["csa_prefill"] = {"value": nq / (t_q + t_comp * nq / pd["Tq"]), "unit": "tokens/s",
                          "compress_s": t_comp, "queries_s": t_q,
                          "sample": f"compression of the {pd['Tq']} new tokens + {nq} queries of the 4096 "
                                    f"(rows {PREFILL_SAMPLE_ROWS}), one run"}
    del pd, E_all, K_all
    x = WL.make_mixed_pair(seqs=[0])
    q_pos0, m, m2, k, W, D = x["q_pos0"], x["m"], x["m2"], x["k"], x["W"], x["D"]
    scale = 1 / math.sqrt(D)
    t0 = time.perf_counter()
    qd = O.mxfp4_decode(*O.mxfp4_quantize(x["qI"][0, 0]))
    kd = O.mxfp4_decode(*O.mxfp4_quantize(x["kI"][0]))
    s = O.bf16_round(O.index_scores(qd, x["w"][0, 0], kd, O.n_visible(q_pos0, m)))
    sel = O.topk_select(s, k)
    Esel = O.kv_mixed_decode(*O.kv_mixed_quantize(x["E"][0][sel], 64))
    Wd = O.kv_mixed_decode(*O.kv_mixed_quantize(x["win"][0], 64))
    O.csa_attend_query(x["q"][0, 0], Esel, np.arange(len(sel)), Wd, x["sink"], scale, q_pos0, q_pos0, W, True,
                       10000.0, 64)
    E2d = O.kv_mixed_decode(*O.kv_mixed_quantize(x["E2"][0], 64))
    W2d = O.kv_mixed_decode(*O.kv_mixed_quantize(x["win2"][0], 64))
    O.hca_attend_query(x["q2"][0, 0], E2d, O.n_visible(q_pos0, m2), W2d, x["sink2"], scale, q_pos0, q_pos0, W,
                       True, 10000.0, 64)
    t_m = time.perf_counter() - t0
    out["mixed_pair"] = {"value": 1.0 / t_m, "unit": "tokens/s",
                         "sample": "sequence 0 of the 64 (both layers, the quantisation of its rows and indexer "
                                   "operands included), one run"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-mixed", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-ragged", action="store_true")
    ap.add_argument("--no-placement", action="store_true")
    ap.add_argument("--no-outproj", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-small-layer", action="store_true")
    ap.add_argument("--no-oracle-samples", action="store_true",
                    help="cpu_baseline without the prefill and mixed-pair samples")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the run, copy MIB MiB device to device (counter calibration)")
    ap.add_argument("--only", choices=["csa", "hca", "prefill", "mixed"],
                    help="run one leg's timed loop only (for counter runs); prints its ms per step")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("LEG", "FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs of --only LEG into profiles/counters.json (no GPU)")
    ap.add_argument("--sq-summary", nargs=2, metavar=("LEG", "CSV"),
                    help="summarise a rocprofv3 --pmc run of SQ_COUNTERS into profiles/counters.json (no GPU)")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.pmc_summary[2], args.copy_calibration or 1024,
                    os.path.join(ROOT, "profiles", "counters.json"))
        return
    if args.sq_summary:
        sq_summary(args.sq_summary[0], args.sq_summary[1], os.path.join(ROOT, "profiles", "counters.json"))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the decode workloads shard by sequence with no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    L.lib()
    if args.only:
        if args.only == "csa":
            step, warm = csa_decode_setup(WL.make_csa_decode(), args.copies), args.warmup
        elif args.only == "hca":
            step, warm = hca_decode_setup(WL.make_hca_decode(), args.copies), args.warmup
        elif args.only == "prefill":
            step, warm = csa_prefill_setup(WL.make_csa_prefill())[0], 1
        else:
            step, warm = mixed_pair_setup()[0], 2
        el = timed(step, args.steps, warm)
        if args.copy_calibration:
            copy_calibration(args.copy_calibration)
        print(json.dumps({"only": args.only, "steps": args.steps, "ms_per_step": 1e3 * el / args.steps}), flush=True)
        return

    d = WL.make_csa_decode()
    step = csa_decode_setup(d, args.copies)
    elapsed = timed(step, args.steps, args.warmup)
    ms = 1e3 * elapsed / args.steps
    B = d["B"]
    kt = kernel_times(step, args.steps)
    progress(f"csa decode: {ms:.4f} ms/step")
    ib, ab = csa_decode_bytes(d)
    score = kt.get("index_score", {"avg_us": float("nan")})
    achieved = ib / (score["avg_us"] * 1e-6) / 1e9
    src = source_hash(SCORE_SOURCES)
    traffic = load_traffic("index_score", "csa_decode_b16_ctx131072", src)
    result = {
        "metric": "CSA/HCA decode tokens/s at 128K-1M ctx; achieved HBM GB/s vs peak (1 GPU)",
        "value": B / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian, 1% 4x-norm spikes)",
        "config": {"workload": "csa_decode_b16_ctx131072", "batch": B, "context": d["q_pos0"],
                   "entries": d["E"].shape[1], "heads": d["H"], "head_dim": d["D"], "index_topk": d["k"],
                   "indexer_heads": d["H_I"], "indexer_dim": d["d_I"], "window": d["W"],
                   "input_copies_rotated": args.copies},
        "roofline": {"bound": "hbm", "kernel": "index_score", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": ib},
        "step_roofline": {"algorithmic_bytes": ib + ab,
                          "achieved_GBs": (ib + ab) / (ms * 1e-3) / 1e9,
                          "frac": (ib + ab) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "kernels_us": per_step(kt, 3),
        "kernel_launches_per_step": launches(kt),
        # secondary statistic: recall of the bf16-score top-k against the fp32-score top-k
        # (the pages report 99.7% on real-model data; here seeded synthetic inputs)
        "bf16_score_topk_recall": {"csa_decode": step.recall(), "pages": 0.997},
    }
    if not args.no_placement:
        result["placement"] = placement_leg()
    if not args.no_outproj:
        result["grouped_out_proj"] = outproj_leg()
    if not args.no_backward:
        result["backward"] = backward_leg()
    if not args.no_ragged:
        result["ragged"] = {"csa_decode_b16_ctx_le131072": ragged_leg(d, args.copies, args.steps, args.warmup,
                                                                      12, ms)}
        result["decode_state"] = decode_state_leg(d, args.copies, args.steps, args.warmup, ms)
    if not args.no_secondary:
        h = WL.make_hca_decode()
        hstep = hca_decode_setup(h, args.copies)
        he = timed(hstep, max(20, args.steps // 2), args.warmup)
        hms = 1e3 * he / max(20, args.steps // 2)
        hk = kernel_times(hstep, max(20, args.steps // 2))
        progress(f"hca decode: {hms:.4f} ms/step")
        hb, hf = hca_decode_bytes(h), hca_decode_flops(h)
        att = hk.get("hca_attend", {"avg_us": float("nan")})["avg_us"]
        hga = hb / (att * 1e-6) / 1e9
        result["secondary"] = {
            "workload": "hca_decode_b8_ctx1048576", "tokens_per_s": h["B"] / (hms * 1e-3),
            "ms_per_step": hms, "kernels_us": per_step(hk, 3),
            "roofline": {"bound": "hbm", "kernel": "hca_attend", "achieved": hga, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": hga / HBM_PEAK_GBS,
                         "traffic": load_traffic("hca_attend", "hca_decode_b8_ctx1048576",
                                                 source_hash(ATTEND_SOURCES)),
                         "algorithmic_bytes_per_launch": hb,
                         "mfma_bf16_frac": hf / (att * 1e-6) / MFMA_BF16_PEAK},
            "hca_attend_GBs": hb / (att * 1e-6) / 1e9, "hca_attend_hbm_frac": hb / (att * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "hca_attend_TFLOPs": hf / (att * 1e-6) / 1e12, "mfma_bf16_frac": hf / (att * 1e-6) / 2.5e15,
            "algorithmic_bytes": hb, "flops": hf,
        }
        if not args.no_ragged:
            result.setdefault("ragged", {})["hca_decode_b8_ctx_le1048576"] = ragged_leg(
                h, args.copies, max(20, args.steps // 2), args.warmup, 13, hms)
    layer_d = None
    if not args.no_small_layer:
        layer_d, result["small_layer"] = small_layer_leg(max(20, args.steps // 4), max(2, args.warmup // 4))
    if not args.no_prefill:
        pd = WL.make_csa_prefill()
        pstep, pflops = csa_prefill_setup(pd)
        del pd
        n_p = 3
        pe = timed(pstep, n_p, 1)
        pms = 1e3 * pe / n_p
        pk = kernel_times(pstep, n_p)
        progress(f"csa prefill: {pms:.3f} ms/step")
        pks = per_step(pk, 3)
        pfi, pfa = csa_prefill_flops_split()
        i_us, a_us = pks.get("index_score", float("nan")), pks.get("csa_attend", float("nan"))
        result["prefill"] = {
            "workload": "csa_prefill_tq4096_ctx1048576", "tokens_per_s": 4096 / (pms * 1e-3),
            "ms_per_step": pms, "kernels_us": pks, "kernel_launches_per_step": launches(pk),
            "roofline": {"bound": "mfma", "kernel": "index_score", "achieved": pfi / (i_us * 1e-6) / 1e12,
                         "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s",
                         "frac": pfi / (i_us * 1e-6) / MFMA_BF16_PEAK, "traffic": None,
                         "algorithmic_flops_per_step": pfi,
                         "note": "scores are never stored: two tiled passes (group maxima, then candidates) "
                                 "each do these flops; achieved counts them once"},
            "csa_attend_roofline": {"bound": "mfma", "achieved": pfa / (a_us * 1e-6) / 1e12,
                                    "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s",
                                    "frac": pfa / (a_us * 1e-6) / MFMA_BF16_PEAK,
                                    "algorithmic_flops_per_step": pfa},
            "flops": pflops, "achieved_TFLOPs": pflops / (pms * 1e-3) / 1e12,
            "mfma_bf16_frac": pflops / (pms * 1e-3) / 2.5e15,
        }
    if not args.no_mixed:
        mstep, mbytes, mflops = mixed_pair_setup()
        n_m = max(10, args.steps // 10)
        me = timed(mstep, n_m, max(2, args.warmup // 4))
        mms = 1e3 * me / n_m
        mk = kernel_times(mstep, n_m)
        progress(f"mixed pair: {mms:.4f} ms/step")
        mks = per_step(mk, 3)
        hfl, hby = mixed_hca_work()
        h_us = mks.get("hca_attend", float("nan"))
        result["mixed_pair"] = {
            "workload": "mixed_csa_hca_pair_b64_ctx1048576", "tokens_per_s": 64 / (mms * 1e-3),
            "ms_per_step": mms, "kernels_us": mks,
            "roofline": {"bound": "mfma", "kernel": "hca_attend", "achieved": hfl / (h_us * 1e-6) / 1e12,
                         "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s",
                         "frac": hfl / (h_us * 1e-6) / MFMA_BF16_PEAK,
                         "traffic": None, "algorithmic_flops_per_launch": hfl,
                         "algorithmic_bytes_per_launch": hby,
                         "hbm_frac": hby / (h_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         "note": "fp8 channels are widened to bf16 before the MFMA: priced at the bf16 peak"},
            "algorithmic_bytes": mbytes, "flops": mflops,
            "achieved_GBs": mbytes / (mms * 1e-3) / 1e9, "hbm_frac": mbytes / (mms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        }
        result["bf16_score_topk_recall"]["mixed_pair_mxfp4"] = mstep.recall()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d, WL.make_hca_decode(), layer=layer_d,
                                              samples=not args.no_oracle_samples)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
