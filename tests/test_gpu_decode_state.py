"""Decode-time state on the GPU ([kwkr] §4.4: state cache and classical KV
cache): the token-at-a-time compressor (csa_compress_append), the
sliding-window ring (lca_window_append, LCA_WIN_RING) and a ragged decode loop
built from them. Entries appended one token at a time must carry the same bits
as the one-shot compressor over the whole sequence; attention over the ring
must carry the same bits as over the linear window; the loop is checked
against the oracle's own decode-time compressor and attention, per sequence
and per step."""

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


def _rows(rng, T, D):
    return (rng.standard_normal((T, D)) / np.sqrt(D)).astype(np.float32), rng.standard_normal(T).astype(np.float32)


# ---------------------------------------------------------------------------
# token-at-a-time compressor == one-shot compressor, bit for bit
# ---------------------------------------------------------------------------

_APPEND_CASES = {
    # dt_in, dt_out, m, overlap, D, flags, rope_dims, lengths
    "csa_bf16_norm_rope": ("bf16", "bf16", 4, True, 512, "norm_rope", 64, [37, 30, 9]),
    "csa_index_mxfp4": ("bf16", "mxfp4", 4, True, 128, "", 0, [41, 4, 3]),
    "hca_kv_mixed": ("bf16", "mixed", 128, False, 512, "norm_rope", 64, [300, 256, 130]),
    "csa_f32": ("f32", "f32", 4, True, 64, "norm", 0, [23, 16, 1]),
}


def _out_buffers(L, dt_out, B, rows, D, R):
    if dt_out == "f32":
        return torch.empty((B, rows, D), dtype=torch.float32, device=DEV), None, L.F32
    if dt_out == "bf16":
        return torch.empty((B, rows, D), dtype=torch.bfloat16, device=DEV), None, L.BF16
    if dt_out == "mixed":
        return (torch.empty((B, rows, D + R), dtype=torch.uint8, device=DEV),
                torch.empty((B, rows), dtype=torch.float32, device=DEV), L.KV_MIXED)
    return (torch.empty((B, rows, D // 2), dtype=torch.uint8, device=DEV),
            torch.empty((B, rows, D // 32), dtype=torch.uint8, device=DEV), L.MXFP4)


def _fill(t):
    if t is None:
        return
    if t.dtype in (torch.uint8,):
        t.fill_(0xA5)
    else:
        t.fill_(float("nan"))


@pytest.mark.parametrize("case", list(_APPEND_CASES))
def test_compress_append_equals_one_shot(case):
    L = need_gpu()
    dt_in, dt_out, m, overlap, D, fl, R, lengths = _APPEND_CASES[case]
    B = len(lengths)
    T = max(lengths)
    rng = np.random.default_rng(110 + len(case))
    cast = WL.bf16_exact if dt_in == "bf16" else (lambda a: a)
    up = dev_bf16 if dt_in == "bf16" else dev_f32
    dti = L.BF16 if dt_in == "bf16" else L.F32
    ca, za, cb, zb = [], [], [], []
    for _ in range(B):
        x, z = _rows(rng, T, D)
        ca.append(cast(x)); za.append(z * 2)
        x, z = _rows(rng, T, D)
        cb.append(cast(x)); zb.append(z * 2)
    ca, za, cb, zb = map(np.stack, (ca, za, cb, zb))
    norm_w = dev_f32(1 + 0.1 * rng.standard_normal(D).astype(np.float32))
    flags = {"norm_rope": L.NORM | L.ROPE, "norm": L.NORM, "": 0}[fl]
    rows = T // m + 1
    out, osc, dto = _out_buffers(L, dt_out, B, rows, D, R)
    _fill(out); _fill(osc)
    state = torch.empty(L.csa_compress_state_bytes(dti, B, D, m, overlap), dtype=torch.uint8, device=DEV)
    state.fill_(0x7F)                         # no initialisation is needed: stale bytes must not leak in
    ca_d, za_d, cb_d, zb_d = up(ca), dev_f32(za), up(cb), dev_f32(zb)
    pos_max = T - 1
    say(f"compress append {case}: {T} steps, lengths {lengths}")
    for t in range(T):
        pos = [t if t < lengths[b] else -1 for b in range(B)]
        L.csa_compress_append(dti, dto, cb_d[:, t].contiguous(), zb_d[:, t].contiguous(), m, _qp(pos), state,
                              out, pos_max=pos_max, ca=ca_d[:, t].contiguous() if overlap else None,
                              za=za_d[:, t].contiguous() if overlap else None, overlap=overlap, flags=flags,
                              norm_w=norm_w, eps=1e-6, rope_base=10000.0, rope_dims=R, out_scale=osc,
                              out_rows=rows)
    torch.cuda.synchronize()
    for b in range(B):
        n = lengths[b] // m
        ref, rsc, _ = _out_buffers(L, dt_out, 1, rows, D, R)
        _fill(ref); _fill(rsc)
        L.csa_compress(dti, dto, cb_d[b:b + 1, :lengths[b]].contiguous(), zb_d[b:b + 1, :lengths[b]].contiguous(),
                       m, ca=ca_d[b:b + 1, :lengths[b]].contiguous() if overlap else None,
                       za=za_d[b:b + 1, :lengths[b]].contiguous() if overlap else None, overlap=overlap, pos0=0,
                       flags=flags, norm_w=norm_w, eps=1e-6, rope_base=10000.0, rope_dims=R, out=ref,
                       out_scale=rsc, out_rows=rows)
        torch.cuda.synchronize()
        got, exp = out[b, :n].view(torch.uint8), ref[0, :n].view(torch.uint8)
        assert torch.equal(got, exp), f"{case} seq {b}: appended entries differ from the one-shot compressor"
        if osc is not None:
            assert torch.equal(osc[b, :n], rsc[0, :n])
        # rows past the last closed block are untouched
        tail = out[b, n:]
        if tail.dtype == torch.uint8:
            assert bool((tail == 0xA5).all())
        else:
            assert bool(torch.isnan(tail.float()).all())
        if dt_out in ("f32", "bf16"):
            st = O.CompressorState(m, overlap)
            ents = []
            for t in range(lengths[b]):
                r = st.append(cb[b, t], zb[b, t], ca[b, t] if overlap else None, za[b, t] if overlap else None)
                if r is not None:
                    ents.append(r[1])
            if ents:
                e = O.compress_epilogue(np.array(ents), 0, m, host(norm_w) if flags & L.NORM else None, 1e-6,
                                        10000.0, R if flags & L.ROPE else 0)
                row_tol_check(host(out[b, :n]), e, 1e-5 if dt_out == "f32" else 2 ** -8, f"{case} seq {b}")


# ---------------------------------------------------------------------------
# attention over the window ring == over the linear window, bit for bit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind,kv,Tq", [("csa", "bf16", 1), ("hca", "bf16", 1), ("csa", "bf16", 2),
                                         ("csa", "mixed", 1), ("hca", "f32", 1)])
def test_window_ring_equals_linear_window(kind, kv, Tq):
    L = need_gpu()
    rng = np.random.default_rng(120 + Tq + len(kind + kv))
    B, W, k = 3, 128, 300
    H, D = (8, 128) if kv == "f32" else ((128, 512) if kv == "mixed" else (64, 512))
    m = 4 if kind == "csa" else 128
    bound = 4 * 3000 + 1 if kind == "csa" else 40001
    pos = [bound, 61, bound // 2 + 3]            # 61: a clipped window
    N_cap = (bound + Tq) // m + 1
    nr = W - 1 + Tq
    cast = (lambda a: a) if kv == "f32" else WL.bf16_exact
    q = cast((rng.standard_normal((B, Tq, H, D)) * 4 / np.sqrt(D)).astype(np.float32))
    E = cast((rng.standard_normal((B, N_cap, D)) / np.sqrt(D)).astype(np.float32))
    tok = (rng.standard_normal((B, nr, D)) / np.sqrt(D)).astype(np.float32)   # rows of positions pos-(W-1) ..
    if kv != "mixed":
        tok = cast(tok)
    sink = dev_f32(rng.standard_normal(H).astype(np.float32))
    dtv = {"f32": L.F32, "bf16": L.BF16, "mixed": L.KV_MIXED}[kv]
    wdt = torch.float32 if kv == "f32" else torch.bfloat16
    # linear window and ring from the same rows
    if kv == "mixed":
        lin = torch.empty((B, nr, D + 64), dtype=torch.uint8, device=DEV)
        lsc = torch.empty((B, nr), dtype=torch.float32, device=DEV)
        L.lca_quantize_rows(L.KV_MIXED, dev_f32(tok), lin, lsc)
        ring = torch.empty_like(lin)
        rsc = torch.empty_like(lsc)
        Eq = torch.empty((B, N_cap, D + 64), dtype=torch.uint8, device=DEV)
        Es = torch.empty((B, N_cap), dtype=torch.float32, device=DEV)
        L.lca_quantize_rows(L.KV_MIXED, dev_f32(E), Eq, Es)
        E_d, src_dt = Eq, L.F32
        src = dev_f32(tok)
    else:
        lin = dev_f32(tok).to(wdt)
        lsc = rsc = Es = None
        ring = torch.empty_like(lin)
        E_d = dev_f32(E).to(wdt)
        src_dt = L.F32 if kv == "f32" else L.BF16
        src = lin
    say(f"window ring {kind} {kv} Tq={Tq}")
    for r in range(nr):
        p_r = [p - (W - 1) + r for p in pos]              # negative: skipped
        L.lca_window_append(src_dt, dtv, src[:, r].contiguous(), _qp(p_r), ring, pos_max=bound + Tq - 1,
                            win_scale=rsc, rope_dims=64)
    torch.cuda.synchronize()
    idx = None
    if kind == "csa":
        idx = np.full((B, Tq, k), -1, np.int32)
        for b in range(B):
            for t in range(Tq):
                nv = O.n_visible(pos[b] + t, m)
                sel = rng.choice(nv, size=min(k - 3, nv), replace=False)
                idx[b, t, :len(sel)] = sel
        idx = torch.from_numpy(idx).to(DEV)
    res = []
    for win, wsc, ring_flag in ((lin, lsc, 0), (ring, rsc, L.WIN_RING)):
        out = torch.empty((B, Tq, H, D), dtype=wdt if kv != "mixed" else torch.bfloat16, device=DEV)
        lse = torch.empty((B, Tq, H), dtype=torch.float32, device=DEV)
        qd = dev_f32(q).to(wdt) if kv != "mixed" else dev_bf16(q)
        kw = dict(m=m, W=W, q_pos0=bound, scale=1 / math.sqrt(D), N_cap=N_cap, kv_scale=Es, win_scale=wsc,
                  flags=L.INV_ROPE | ring_flag, rope_dims=64, lse_out=lse, q_pos=_qp(pos))
        dq = L.F32 if kv == "f32" else L.BF16
        if kind == "csa":
            L.csa_attend(dq, dtv, qd, E_d, idx, win, sink, out, **kw)
        else:
            L.hca_attend(dq, dtv, qd, E_d, win, sink, out, **kw)
        torch.cuda.synchronize()
        res.append((out, lse))
    if kv == "mixed":
        # the ring's quantised rows equal the linear window's, row for row
        for b in range(B):
            for r in range(nr):
                p_r = pos[b] - (W - 1) + r
                if p_r >= 0:
                    assert torch.equal(ring[b, p_r % nr], lin[b, r])
    assert torch.equal(res[0][0], res[1][0]), "ring window output differs"
    assert torch.equal(res[0][1], res[1][1])


# ---------------------------------------------------------------------------
# a ragged decode loop from the first token, against the oracle
# ---------------------------------------------------------------------------

def _loop_inputs(seed, B, T, D, H, H_I, d_I):
    seqs = []
    for b in range(B):
        r = WL.seq_rng(seed, b)
        s = {}
        for n in ("ca", "cb", "ica", "icb"):
            s[n] = WL.gauss(r, (T, d_I if n.startswith("i") else D))
        for n in ("za", "zb", "iza", "izb"):
            s[n] = r.standard_normal(T, dtype=np.float32)
        s["kvw"] = WL.gauss(r, (T, D))
        s["q"] = WL.gauss(r, (T, H, D)) * np.float32(8.0)
        s["qI"] = WL.gauss(r, (T, H_I, d_I))
        s["w"] = r.standard_normal((T, H_I), dtype=np.float32) * np.float32(1 / np.sqrt(H_I))
        seqs.append(s)
    return seqs


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_ragged_decode_loop_matches_oracle(kind):
    # fp32 throughout. Each step appends one token per active sequence to the
    # entry compressor, the indexer-key compressor (CSA) and the window ring,
    # then decodes it: index top-k + attention for CSA, dense attention for HCA,
    # with every sequence at its own position (some idle: position -1).
    L = need_gpu()
    B, D, H, H_I, d_I, W, R = 3, 128, 8, 4, 64, 128, 64
    m, overlap, k = (4, True, 16) if kind == "csa" else (8, False, 0)
    T = 220
    lengths, starts = [220, 150, 97], [0, 30, 95]
    steps = max(s + n for s, n in zip(starts, lengths))
    seqs = _loop_inputs(130 + m, B, T, D, H, H_I, d_I)
    rng = WL.shared_rng(130 + m)
    sink = rng.standard_normal(H, dtype=np.float32)
    norm_w = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    bound, N_cap = T - 1, T // m
    E = torch.zeros((B, N_cap, D), dtype=torch.float32, device=DEV)
    KI = torch.zeros((B, N_cap, d_I), dtype=torch.float32, device=DEV)
    ring = torch.zeros((B, W, D), dtype=torch.float32, device=DEV)
    stE = torch.empty(L.csa_compress_state_bytes(L.F32, B, D, m, overlap), dtype=torch.uint8, device=DEV)
    stK = torch.empty(L.csa_compress_state_bytes(L.F32, B, d_I, m, overlap), dtype=torch.uint8, device=DEV)
    dev = [{n: dev_f32(v) for n, v in s.items()} for s in seqs]
    sink_d, nw_d = dev_f32(sink), dev_f32(norm_w)
    oE = [O.CompressorState(m, overlap) for _ in range(B)]
    oK = [O.CompressorState(m, overlap) for _ in range(B)]
    entE = [[] for _ in range(B)]
    entK = [[] for _ in range(B)]
    scale = 1 / math.sqrt(D)
    checked = 0
    say(f"ragged decode loop {kind}: {steps} steps")

    def gather(name, pos):
        return torch.stack([dev[b][name][max(p, 0)] for b, p in enumerate(pos)]).contiguous()

    for s in range(steps):
        pos = [s - starts[b] if 0 <= s - starts[b] < lengths[b] else -1 for b in range(B)]
        qp = _qp(pos)
        L.csa_compress_append(L.F32, L.F32, gather("cb", pos), gather("zb", pos), m, qp, stE, E, pos_max=bound,
                              ca=gather("ca", pos) if overlap else None, za=gather("za", pos) if overlap else None,
                              overlap=overlap, flags=L.NORM | L.ROPE, norm_w=nw_d, eps=1e-6, rope_dims=R)
        if kind == "csa":
            L.csa_compress_append(L.F32, L.F32, gather("icb", pos), gather("izb", pos), m, qp, stK, KI,
                                  pos_max=bound, ca=gather("ica", pos), za=gather("iza", pos))
        L.lca_window_append(L.F32, L.F32, gather("kvw", pos), qp, ring, pos_max=bound)
        out = torch.empty((B, 1, H, D), dtype=torch.float32, device=DEV)
        q = gather("q", pos)[:, None].contiguous()
        idx = None
        if kind == "csa":
            idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
            L.csa_index_topk(L.F32, gather("qI", pos)[:, None].contiguous(), gather("w", pos)[:, None].contiguous(),
                             KI, idx, m=m, k=k, q_pos0=bound, q_pos=qp)
            L.csa_attend(L.F32, L.F32, q, E, idx, ring, sink_d, out, m=m, W=W, q_pos0=bound, scale=scale,
                         flags=L.INV_ROPE | L.WIN_RING, rope_dims=R, q_pos=qp)
        else:
            L.hca_attend(L.F32, L.F32, q, E, ring, sink_d, out, m=m, W=W, q_pos0=bound, scale=scale,
                         flags=L.INV_ROPE | L.WIN_RING, rope_dims=R, q_pos=qp)
        # oracle: the same tokens through its own decode-time compressor
        for b in range(B):
            p = pos[b]
            if p < 0:
                continue
            x = seqs[b]
            r = oE[b].append(x["cb"][p], x["zb"][p], x["ca"][p] if overlap else None,
                             x["za"][p] if overlap else None)
            if r is not None:
                entE[b].append(O.compress_epilogue(r[1][None], r[0] * m, m, norm_w, 1e-6, 10000.0, R)[0])
            if kind == "csa":
                r = oK[b].append(x["icb"][p], x["izb"][p], x["ica"][p], x["iza"][p])
                if r is not None:
                    entK[b].append(r[1])
        check = s % 11 == 0 or s >= steps - 2 or any(p == lengths[b] - 1 for b, p in enumerate(pos))
        if not check:
            continue
        torch.cuda.synchronize()
        out_h = host(out)
        idx_h = idx.cpu().numpy() if idx is not None else None
        for b in range(B):
            p = pos[b]
            if p < 0:
                continue
            x = seqs[b]
            Eo = np.array(entE[b]).reshape(-1, D)
            nv = O.n_visible(p, m)
            assert Eo.shape[0] == nv
            win = np.zeros((W, D))                         # linear window: row r = position p - (W-1) + r
            for r_ in range(W):
                pp = p - (W - 1) + r_
                if pp >= 0:
                    win[r_] = x["kvw"][pp]
            if kind == "csa":
                Ko = np.array(entK[b]).reshape(-1, d_I)
                sc = O.index_scores(x["qI"][p], x["w"][p], Ko, nv)
                check_topk_set(idx_h[b, 0], sc, k)
                # attention of the oracle over the GPU's (checked) selection
                ref, _ = O.csa_attend_query(x["q"][p], Eo, idx_h[b, 0], win, sink, scale, p, p, W, True, 10000.0, R)
            else:
                ref, _ = O.hca_attend_query(x["q"][p], Eo, nv, win, sink, scale, p, p, W, True, 10000.0, R)
            row_tol_check(out_h[b, 0], ref, 1e-4, f"decode loop {kind} seq {b} pos {p}")
            checked += 1
    say(f"  {checked} (sequence, step) outputs checked")
    assert checked > 40


def test_state_checkpoint_restore_replays_bitwise():
    # Copying the state buffer and the ring takes a checkpoint; restoring it and
    # replaying the same tokens gives the same entries and window bit for bit.
    L = need_gpu()
    B, D, m, W = 2, 256, 4, 128
    rng = np.random.default_rng(140)
    T = 1100
    cb = dev_bf16(WL.bf16_exact((rng.standard_normal((T, B, D)) / 16).astype(np.float32)))
    ca = dev_bf16(WL.bf16_exact((rng.standard_normal((T, B, D)) / 16).astype(np.float32)))
    za = dev_f32(rng.standard_normal((T, B)).astype(np.float32))
    zb = dev_f32(rng.standard_normal((T, B)).astype(np.float32))
    st = torch.empty(L.csa_compress_state_bytes(L.BF16, B, D, m, True), dtype=torch.uint8, device=DEV)
    E = torch.zeros((B, T // m, D), dtype=torch.bfloat16, device=DEV)
    ring = torch.zeros((B, W, D), dtype=torch.bfloat16, device=DEV)

    def run(t0, t1):
        for t in range(t0, t1):
            qp = _qp([t, t])
            L.csa_compress_append(L.BF16, L.BF16, cb[t], zb[t], m, qp, st, E, pos_max=T - 1, ca=ca[t], za=za[t])
            L.lca_window_append(L.BF16, L.BF16, cb[t], qp, ring, pos_max=T - 1)

    say("state checkpoint / restore")
    run(0, 1024)                                  # checkpoint at a 1024-token boundary
    ck = (st.clone(), ring.clone())
    run(1024, T)
    torch.cuda.synchronize()
    E1, R1 = E.clone(), ring.clone()
    E[:, 1024 // m:].zero_()
    st.copy_(ck[0])
    ring.copy_(ck[1])
    run(1024, T)
    torch.cuda.synchronize()
    assert torch.equal(E, E1)
    assert torch.equal(ring, R1)


def test_fused_decode_append_equals_separate_calls():
    # One lca_decode_append launch with three jobs (KV_MIXED entries with
    # RMSNorm + RoPE from bf16 rows, MXFP4 indexer keys, a KV_MIXED window ring
    # from fp32 rows) against the three separate calls: every cache, ring and
    # state byte equal, over a ragged batch (one sequence idle part of the time).
    L = need_gpu()
    B, D, d_I, m, W, R = 4, 512, 128, 4, 128, 64
    T = 41
    rng = np.random.default_rng(150)
    starts = [0, 3, 10, 0]
    cb = dev_bf16(WL.bf16_exact((rng.standard_normal((T, B, D)) / np.sqrt(D)).astype(np.float32)))
    ca = dev_bf16(WL.bf16_exact((rng.standard_normal((T, B, D)) / np.sqrt(D)).astype(np.float32)))
    icb = dev_bf16(WL.bf16_exact((rng.standard_normal((T, B, d_I)) / np.sqrt(d_I)).astype(np.float32)))
    ica = dev_bf16(WL.bf16_exact((rng.standard_normal((T, B, d_I)) / np.sqrt(d_I)).astype(np.float32)))
    z = dev_f32(rng.standard_normal((4, T, B)).astype(np.float32))
    kvw = dev_f32((rng.standard_normal((T, B, D)) / np.sqrt(D)).astype(np.float32))
    nw = dev_f32(1 + 0.1 * rng.standard_normal(D).astype(np.float32))
    rows = T // m + 1

    def buffers():
        return {"E": torch.zeros((B, rows, D + R), dtype=torch.uint8, device=DEV),
                "Es": torch.zeros((B, rows), dtype=torch.float32, device=DEV),
                "K": torch.zeros((B, rows, d_I // 2), dtype=torch.uint8, device=DEV),
                "Ks": torch.zeros((B, rows, d_I // 32), dtype=torch.uint8, device=DEV),
                "ring": torch.zeros((B, W, D + R), dtype=torch.uint8, device=DEV),
                "rs": torch.zeros((B, W), dtype=torch.float32, device=DEV),
                "stE": torch.zeros(L.csa_compress_state_bytes(L.BF16, B, D, m, True), dtype=torch.uint8, device=DEV),
                "stK": torch.zeros(L.csa_compress_state_bytes(L.BF16, B, d_I, m, True), dtype=torch.uint8,
                                   device=DEV)}
    sep, fus = buffers(), buffers()
    say("fused decode append vs separate calls")
    for t in range(T):
        pos = [t - s_ if t - s_ >= 0 else -1 for s_ in starts]
        if 12 <= t < 20:
            pos[3] = -1                                   # sequence 3 idle for a while
        qp = _qp(pos)
        L.csa_compress_append(L.BF16, L.KV_MIXED, cb[t], z[1, t], m, qp, sep["stE"], sep["E"], pos_max=T - 1,
                              ca=ca[t], za=z[0, t], flags=L.NORM | L.ROPE, norm_w=nw, rope_dims=R,
                              out_scale=sep["Es"])
        L.csa_compress_append(L.BF16, L.MXFP4, icb[t], z[3, t], m, qp, sep["stK"], sep["K"], pos_max=T - 1,
                              ca=ica[t], za=z[2, t], out_scale=sep["Ks"])
        L.lca_window_append(L.F32, L.KV_MIXED, kvw[t], qp, sep["ring"], pos_max=T - 1, win_scale=sep["rs"],
                            rope_dims=R)
        jobs = [L.append_job_compress(L.BF16, L.KV_MIXED, cb[t], z[1, t], m, fus["stE"], fus["E"], ca=ca[t],
                                      za=z[0, t], flags=L.NORM | L.ROPE, norm_w=nw, rope_dims=R,
                                      out_scale=fus["Es"]),
                L.append_job_compress(L.BF16, L.MXFP4, icb[t], z[3, t], m, fus["stK"], fus["K"], ca=ica[t],
                                      za=z[2, t], out_scale=fus["Ks"]),
                L.append_job_window(L.F32, L.KV_MIXED, kvw[t], fus["ring"], win_scale=fus["rs"], rope_dims=R)]
        L.lca_decode_append(jobs, qp, pos_max=T - 1)
    torch.cuda.synchronize()
    for n in sep:
        assert torch.equal(sep[n], fus[n]), f"fused append differs in {n}"
    assert bool((sep["Es"][0, :T // m] > 0).all())        # entries were written
