"""Plain float64 reference of the CSA / HCA hot path.

TEST INFRASTRUCTURE ONLY (see package docstring). Slow and obvious on purpose:
no blocking, fusion or reordering beyond what each definition states.

Conventions (all arrays are numpy; every computation is float64 unless a
function says otherwise):

* One sequence at a time. ``T`` tokens, ``D`` channels per KV row, ``m`` the
  compression ratio, ``R`` the number of RoPE channels (the last ``R`` of ``D``).
* Query ``t`` sits at absolute position ``p = q_pos0 + t``.
* Compressed entry ``j`` covers tokens ``[j*m, (j+1)*m)`` and is visible to a
  query at position ``p`` iff its whole block is at or before ``p``:
  ``j < (p + 1) // m``.
* The sliding window holds the raw rows of positions ``[max(0, p-W+1), p]``;
  window buffer row ``r`` holds position ``q_pos0 - (W - 1) + r``.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "n_visible",
    "compress_sequence",
    "CompressorState",
    "rms_norm",
    "rope_rotate",
    "compress_epilogue",
    "compress_backward",
    "index_scores",
    "topk_select",
    "topk_classes",
    "sink_attention",
    "window_positions",
    "csa_attend_query",
    "hca_attend_query",
    "csa_attend",
    "hca_attend",
    "bf16_round",
    "bf16_next",
    "e4m3fn_encode",
    "e4m3fn_decode",
    "kv_mixed_quantize",
    "kv_mixed_decode",
    "e2m1_encode",
    "e2m1_decode",
    "mxfp4_quantize",
    "mxfp4_decode",
    "grouped_output_projection",
    "attend_backward_query",
    "csa_attend_backward",
    "hca_attend_backward",
    "E4M3_MAX",
    "E2M1_GRID",
]


# ---------------------------------------------------------------------------
# Causality of compressed entries
# ---------------------------------------------------------------------------

def n_visible(p: int, m: int) -> int:
    """Number of compressed entries a query at absolute position ``p`` may use.

    [PACMAN] §3.1 and [Qiaomu] 混合注意力机制: every ``m`` consecutive tokens fold
    into one entry. An entry exists only once its whole block has been seen,
    so entries ``0 .. (p+1)//m - 1`` are visible. At p = 131072, m = 4 this is
    32768; at p = 1048576, m = 128 it is 8192 (the decode shapes).
    """
    return (p + 1) // m


# ---------------------------------------------------------------------------
# Token compressor (CSA: m = 4 with overlap over two streams; HCA: m = 128)
# ---------------------------------------------------------------------------

def _softmax(logits: np.ndarray) -> np.ndarray:
    z = np.asarray(logits, dtype=np.float64)
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def compress_sequence(cb, zb, m, ca=None, za=None, prev_ca=None, prev_za=None,
                      overlap=True):
    """Gated softmax-weighted merge of token KV rows into compressed entries.

    [kwkr] §3.1 (CSA 的工作方式): compression merges two independent KV
    sequences with softmax-normalised gate weights, and adjacent compressed
    blocks share part of their indices (overlapping compression).
    [Qiaomu] 混合注意力机制: the compressor computes two groups of information
    with their importance weights, then merges them by weighted sum.
    [PACMAN] §3.2 and [kwkr] §3.2: HCA folds every 128 tokens into one entry,
    without the sparse selection (and, in this reading, without overlap).

    Reading used (stated in the design doc): entry j takes stream ``a``'s rows of
    block j-1 and stream ``b``'s rows of block j; one joint softmax runs over
    their 2m per-token gate logits. For j = 0 the block j-1 rows come from
    ``prev_ca`` / ``prev_za`` (the last block before this call) or, when those
    are None, are absent (masked). ``overlap=False`` uses stream ``b`` only
    (the HCA compressor). A trailing partial block emits nothing.

    Args:
      cb: [T, D] stream b rows; zb: [T] gate logits of stream b.
      ca, za: stream a (required when overlap).
      prev_ca: [m, D], prev_za: [m] or None.
    Returns: [T // m, D] float64 entries.

    Pinned by: constant sequence compresses to itself, equal logits give the
    arithmetic mean, a dominant logit selects its row, linearity in the rows,
    chunked == one-shot with carried state (tests/test_oracle_compress.py).
    """
    cb = np.asarray(cb, dtype=np.float64)
    zb = np.asarray(zb, dtype=np.float64)
    T, D = cb.shape
    n_out = T // m
    out = np.zeros((n_out, D), dtype=np.float64)
    if overlap:
        ca = np.asarray(ca, dtype=np.float64)
        za = np.asarray(za, dtype=np.float64)
    for j in range(n_out):
        rows = []
        logits = []
        if overlap:
            if j == 0:
                if prev_ca is not None:
                    rows.append(np.asarray(prev_ca, dtype=np.float64))
                    logits.append(np.asarray(prev_za, dtype=np.float64))
            else:
                rows.append(ca[(j - 1) * m: j * m])
                logits.append(za[(j - 1) * m: j * m])
        rows.append(cb[j * m: (j + 1) * m])
        logits.append(zb[j * m: (j + 1) * m])
        x = np.concatenate(rows, axis=0)
        w = _softmax(np.concatenate(logits))
        out[j] = w @ x
    return out


class CompressorState:
    """Decode-time compressor of one sequence: tokens arrive one at a time.

    [kwkr] §4.4: a request's KV cache splits into a state cache and a
    classical KV cache. Reading used (stated in the design doc): the state cache
    holds what the compressor has not yet folded into an entry -- both
    streams' rows of the block in progress -- plus stream a's rows of the
    last complete block, which the next entry still needs because adjacent
    blocks overlap ([kwkr] §3.1). The classical cache receives entry j when
    the token at position j*m + m - 1 closes block j; the entry is the same
    gated softmax merge as ``compress_sequence`` (one joint softmax over
    stream a of block j-1 and stream b of block j; block 0 has no stream-a
    half). ``overlap=False`` keeps stream b only (HCA).

    Pinned by: feeding a sequence token by token emits exactly the entries of
    the one-shot ``compress_sequence`` (tests/test_oracle_compress.py), for
    CSA (m = 4, overlap) and HCA (m = 128) shapes.
    """

    def __init__(self, m, overlap=True):
        self.m = m
        self.overlap = overlap
        self.pos = 0                  # position of the next token
        self.tail_a = None            # (rows [m, D], logits [m]) of stream a, last complete block
        self.cur = []                 # (ca, za, cb, zb) of the block in progress

    def append(self, cb_row, zb, ca_row=None, za=None):
        """Take the token at position ``self.pos``. Returns ``(j, entry)``
        when it closes block j, else None."""
        self.cur.append((ca_row, za, np.asarray(cb_row, dtype=np.float64), float(zb)))
        self.pos += 1
        if len(self.cur) < self.m:
            return None
        j = self.pos // self.m - 1
        rows, logits = [], []
        if self.overlap and self.tail_a is not None:
            rows.extend(self.tail_a[0])
            logits.extend(self.tail_a[1])
        rows.extend(t[2] for t in self.cur)
        logits.extend(t[3] for t in self.cur)
        w = _softmax(np.array(logits))
        entry = np.zeros_like(rows[0])
        for wi, r in zip(w, rows):
            entry = entry + wi * r
        if self.overlap:
            self.tail_a = ([np.asarray(t[0], dtype=np.float64) for t in self.cur],
                           [float(t[1]) for t in self.cur])
        self.cur = []
        return j, entry


def rms_norm(x, weight, eps):
    """Root-mean-square normalisation of one row, then per-channel gain.

    [Qiaomu] 混合注意力机制: queries and KV entries are normalised to keep the
    logits from blowing up. The exact form (RMSNorm, eps) is a reading.
    Pinned by: output RMS equals 1 for unit gain and tiny eps.
    """
    x = np.asarray(x, dtype=np.float64)
    r = math.sqrt(float(np.mean(x * x)) + eps)
    return x / r * np.asarray(weight, dtype=np.float64)


def rope_rotate(x, pos, base, rope_dims):
    """Rotate the last ``rope_dims`` channels of row(s) ``x`` by position ``pos``.

    [cdjax] §1.1 and [Qiaomu] 混合注意力机制: rotary position encoding acts on
    part of the channels only, the last 64. Reading: channels pair up as
    (D-R+2i, D-R+2i+1) with frequency base**(-2i/R); pair (u, v) rotates by
    angle pos*freq. ``pos`` may be negative (inverse rotation).

    Pinned by: agreement with the complex-exponential form, norm preservation,
    R(-p) R(p) = identity, and relative-position invariance of dot products
    (tests/test_oracle_rope.py). Its match with the real model is unpinned.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    D = x.shape[-1]
    R = rope_dims
    for i in range(R // 2):
        freq = base ** (-2.0 * i / R)
        ang = pos * freq
        c, s = math.cos(ang), math.sin(ang)
        u = x[..., D - R + 2 * i].copy()
        v = x[..., D - R + 2 * i + 1].copy()
        x[..., D - R + 2 * i] = u * c - v * s
        x[..., D - R + 2 * i + 1] = u * s + v * c
    return x


def compress_epilogue(entries, pos0, m, norm_w=None, eps=1e-6, rope_base=None,
                      rope_dims=0):
    """Optional per-entry post-processing after the merge: RMSNorm then RoPE.

    Order (reading): merge -> RMSNorm -> RoPE at the block start position
    ``pos0 + j*m``. [Qiaomu] 混合注意力机制 (normalised entries, partial RoPE),
    [cdjax] §1.1 (RoPE on the last 64 channels).

    Pinned by: chunked calls (pos0 = T1 with the overlap carried) equal one
    call; entry j of a constant sequence equals the row rotated to pos0 + j*m
    by an independent complex-exponential rotation, and its dot with a query
    depends only on the relative position; rotating the output back gives a
    row parallel to g * e with unit RMS after dividing by g (norm before
    RoPE under a non-uniform gain); unit gain keeps unit RMS
    (tests/test_oracle_compress.py).
    """
    e = np.array(entries, dtype=np.float64, copy=True)
    for j in range(e.shape[0]):
        if norm_w is not None:
            e[j] = rms_norm(e[j], norm_w, eps)
        if rope_dims:
            e[j] = rope_rotate(e[j], pos0 + j * m, rope_base, rope_dims)
    return e


# ---------------------------------------------------------------------------
# Lightning Indexer scores and top-k
# ---------------------------------------------------------------------------

def index_scores(qI, w, kI, n_vis):
    """Index score of every visible compressed entry for one query.

    [Qiaomu] 混合注意力机制: the Lightning Indexer produces cheap query vectors
    and scores every compressed block. [kwkr] §3.1: CSA runs DeepSeek Sparse
    Attention over the compressed entries. Reading (the pages print no
    formula): s_j = sum_h w_h * max(0, qI_h . kI_j) for j < n_vis, one shared
    indexer key per entry, per-head weights ``w`` given as inputs.

    Args: qI [H_I, d_I], w [H_I], kI [>=n_vis, d_I].
    Returns: [n_vis] float64.
    Pinned by: brute-force scalar loops and, for one head with w = 1 and
    positive dots, plain inner products (tests/test_oracle_index.py).
    """
    qI = np.asarray(qI, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = np.asarray(kI[:n_vis], dtype=np.float64)
    dots = k @ qI.T                      # [n_vis, H_I]
    return np.maximum(dots, 0.0) @ w


def topk_select(scores, k):
    """Indices of the k_eff = min(k, n) largest scores; ties go to lower index.

    [PACMAN] §3.1: only the top-k compressed entries are attended;
    [Qiaomu] 训练配置: k = 512 (Flash) / 1024 (Pro). Tie rule and short-list
    rule are readings. Returns int64 indices in (score desc, index asc) order.
    Pinned by: exhaustive comparison with Python's stable sort and with
    torch.topk on tie-free data (tests/test_oracle_topk.py).
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    order = np.lexsort((np.arange(n), -s))
    return order[: min(k, n)]


def topk_classes(scores, k, tau_rel=1e-3, bf16_scores=False, mid_rel=1e-5):
    """Split visible entries into certain-in / certain-out / ambiguous.

    A GPU set G passes when certain_in is a subset of G, G holds no
    certain_out entry, |G| = min(k, n) and G has no duplicates. Entries whose
    score is within ``tau_rel * |s_(k)|`` of the k-th score are ambiguous: fp32
    accumulation order on the GPU may legitimately reorder them.
    In bf16-score mode ([Qiaomu] FP4量化感知训练 and [kwkr] §4.4: index scores go
    FP32 -> BF16 before top-k), every entry whose bf16 value equals bf16(s_(k))
    is ambiguous, and so is any entry whose float64 score sits within
    ``mid_rel`` of a bf16 rounding midpoint next to that value.
    Returns (certain_in, certain_out, ambiguous) as boolean masks.
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    k_eff = min(k, n)
    if k_eff == n:
        return np.ones(n, bool), np.zeros(n, bool), np.zeros(n, bool)
    order = topk_select(s, k)
    if bf16_scores:
        sb = bf16_round(s)
        kth = sb[order[k_eff - 1]]
        amb = sb == kth
        # neighbours of kth on the bf16 grid and the midpoints between them
        up = bf16_next(kth, +1)
        dn = bf16_next(kth, -1)
        for mid in (0.5 * (kth + up), 0.5 * (kth + dn)):
            amb |= np.abs(s - mid) <= mid_rel * max(abs(mid), 1e-30)
        cin = (sb > kth) & ~amb
        cout = (sb < kth) & ~amb
        return cin, cout, amb
    kth = s[order[k_eff - 1]]
    tau = tau_rel * abs(kth)
    cin = s > kth + tau
    cout = s < kth - tau
    amb = ~(cin | cout)
    return cin, cout, amb


# ---------------------------------------------------------------------------
# Core attention with sliding window and sink
# ---------------------------------------------------------------------------

def sink_attention(q, X, sink, scale):
    """One head's softmax attention over rows X with a value-less sink logit.

    K = V = X (MQA over compressed entries whose row serves as key and value:
    [cdjax] §1.1 (Multi-Query Attention form), [fwf] §2 (each entry acts as
    both key and value)). The sink is one learnable logit added to the softmax
    denominator only ([cdjax] §1.1: lets a head push total attention toward 0;
    [kwkr] §3.3: learnable denominator term).

      l_x = scale * q.x ; M = max(sink, max l) ; Z = e^(sink-M) + sum e^(l-M)
      o = sum e^(l-M) x / Z ; lse = M + log Z

    Returns (o [D], lse, weights [n_rows]). With no rows, o = 0 and lse = sink.
    Pinned by: torch float64 scaled_dot_product_attention with an extra
    zero-key / zero-value column whose additive mask equals the sink, sum of
    weights = sigmoid(lse_rows - sink), brute-force loops
    (tests/test_oracle_attend.py).
    """
    q = np.asarray(q, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    if X.shape[0] == 0:
        return np.zeros(q.shape[0]), float(sink), np.zeros(0)
    logits = scale * (X @ q)
    M = max(float(sink), float(logits.max()))
    e = np.exp(logits - M)
    Z = math.exp(float(sink) - M) + float(e.sum())
    wts = e / Z
    return wts @ X, M + math.log(Z), wts


def window_positions(p, W):
    """Positions of the raw sliding-window rows seen by a query at ``p``.

    [Qiaomu] 混合注意力机制 and [kwkr] §3.3: both CSA and HCA keep a branch over
    the most recent 128 uncompressed tokens, which joins the core attention.
    Reading: the window includes the query's own token and is clipped at 0.
    """
    return np.arange(max(0, p - W + 1), p + 1)


def _query_rows(E, sel, win, W, p, q_pos0):
    win_pos = window_positions(p, W)
    win_rows = win[win_pos - (q_pos0 - (W - 1))]
    ent_rows = E[sel] if len(sel) else np.zeros((0, E.shape[1]))
    return np.concatenate([ent_rows, win_rows], axis=0)


def csa_attend_query(q, E, sel, win, sink, scale, p, q_pos0, W=128,
                     inv_rope=False, rope_base=10000.0, rope_dims=0):
    """CSA core attention of one query (all heads) over selected entries.

    [PACMAN] §3.1: attention over the top-k compressed entries plus a recent
    uncompressed window; [kwkr] §3.3: the window rows join the core
    computation, with the sink; [cdjax] §1.1: the core-attention output gets
    RoPE at the negative query position to restore relative position.

    Args: q [H, D]; E [N, D] entries; sel: selected entry indices (-1 ignored);
      win [W-1+Tq, D]; sink [H].
    Returns (out [H, D], lse [H]).
    Pinned by: CSA with k >= n_vis equals HCA over all entries, permuting
    ``sel`` changes nothing (tests/test_oracle_attend.py).
    """
    sel = np.asarray([s for s in np.asarray(sel).tolist() if s >= 0], dtype=np.int64)
    X = _query_rows(np.asarray(E, dtype=np.float64), sel,
                    np.asarray(win, dtype=np.float64), W, p, q_pos0)
    H = q.shape[0]
    out = np.zeros((H, X.shape[1]))
    lse = np.zeros(H)
    for h in range(H):
        o, l, _ = sink_attention(q[h], X, sink[h], scale)
        if inv_rope and rope_dims:
            o = rope_rotate(o, -p, rope_base, rope_dims)
        out[h] = o
        lse[h] = l
    return out, lse


def hca_attend_query(q, E, n_vis, win, sink, scale, p, q_pos0, W=128,
                     inv_rope=False, rope_base=10000.0, rope_dims=0):
    """HCA core attention of one query: dense MQA over every visible entry.

    [PACMAN] §3.2 and [kwkr] §3.2: no top-k; dense attention over all heavily
    compressed entries, plus the same sliding window and sink.
    """
    return csa_attend_query(q, E, np.arange(n_vis), win, sink, scale, p, q_pos0,
                            W, inv_rope, rope_base, rope_dims)


def csa_attend(q, E, idx, win, sink, scale, q_pos0, W=128, inv_rope=False,
               rope_base=10000.0, rope_dims=0, rows=None):
    """Batch wrapper: q [Tq, H, D], idx [Tq, k] -> out [Tq, H, D], lse [Tq, H].

    ``rows`` optionally restricts evaluation to a list of query indices (the
    other rows of the result stay NaN).
    """
    Tq, H, D = q.shape
    out = np.full((Tq, H, D), np.nan)
    lse = np.full((Tq, H), np.nan)
    for t in (range(Tq) if rows is None else rows):
        out[t], lse[t] = csa_attend_query(q[t], E, idx[t], win, sink, scale,
                                          q_pos0 + t, q_pos0, W, inv_rope,
                                          rope_base, rope_dims)
    return out, lse


def hca_attend(q, E, m, win, sink, scale, q_pos0, W=128, inv_rope=False,
               rope_base=10000.0, rope_dims=0, rows=None):
    """Batch wrapper for HCA: every query attends all its visible entries."""
    Tq, H, D = q.shape
    out = np.full((Tq, H, D), np.nan)
    lse = np.full((Tq, H), np.nan)
    for t in (range(Tq) if rows is None else rows):
        p = q_pos0 + t
        out[t], lse[t] = hca_attend_query(q[t], E, n_visible(p, m), win, sink,
                                          scale, p, q_pos0, W, inv_rope,
                                          rope_base, rope_dims)
    return out, lse


# ---------------------------------------------------------------------------
# Backward of the core attention (training)
# ---------------------------------------------------------------------------

def attend_backward_query(q, X, sink, scale, p, dout, inv_rope=False, rope_base=10000.0, rope_dims=0):
    """Gradients of one query's attention (all heads) over rows X, given the
    gradient ``dout`` of its output.

    The forward is ``sink_attention`` per head, then (with inv_rope) the
    output turned by -p ([cdjax] §1.1). With K = V = X shared by the heads
    (MQA), each row's gradient sums a value part and a key part over heads.
    For head h, P_j = softmax weight of row j, P_s = the sink's weight:
      do = dout turned back by +p (the adjoint of the turn by -p),
      D = do . o,  dl_j = P_j (do . x_j - D),
      dq = scale sum_j dl_j x_j,  dx_j = sum_h (P_j do + scale dl_j q),
      dsink = -P_s D   (the sink has a logit and no value).
    [kwkr] §4.3 and [Qiaomu] 批不变 kernel: the backward is deterministic; here
    it is the plain chain rule of the forward.

    Args: q [H, D], X [n, D], sink [H], dout [H, D].
    Returns (dq [H, D], dX [n, D], dsink [H]) in float64.
    Pinned by: central finite differences of sum(dout * out) on tiny inputs,
    float64 torch autograd through an independent forward, and closed forms
    (tests/test_oracle_backward.py).
    """
    q = np.asarray(q, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    H, D = q.shape
    dq = np.zeros((H, D))
    dX = np.zeros_like(X)
    dsink = np.zeros(H)
    for h in range(H):
        o, lse, wts = sink_attention(q[h], X, sink[h], scale)
        do = rope_rotate(dout[h], p, rope_base, rope_dims) if (inv_rope and rope_dims) else dout[h]
        Dv = float(do @ o)
        if X.shape[0]:
            dl = wts * (X @ do - Dv)
            dq[h] = scale * (dl @ X)
            dX += np.outer(wts, do) + scale * np.outer(dl, q[h])
        dsink[h] = -math.exp(float(sink[h]) - lse) * Dv
    return dq, dX, dsink


def _backward_rows(E, sel, win, W, p, q_pos0):
    """Sources of a query's rows: (kind, index) per row, entries then window."""
    src = [("e", int(s)) for s in np.asarray(sel).tolist() if s >= 0]
    src += [("w", int(pp - (q_pos0 - (W - 1)))) for pp in window_positions(p, W)]
    return src


def _attend_backward(q, E, sels, win, sink, scale, q_pos0, W, inv_rope, rope_base, rope_dims, dout):
    Tq, H, D = q.shape
    E = np.asarray(E, dtype=np.float64)
    win = np.asarray(win, dtype=np.float64)
    dq = np.zeros((Tq, H, D))
    dE = np.zeros_like(E)
    dwin = np.zeros_like(win)
    dsink = np.zeros(H)
    for t in range(Tq):
        p = q_pos0 + t
        src = _backward_rows(E, sels[t], win, W, p, q_pos0)
        X = np.array([E[i] if k == "e" else win[i] for k, i in src]).reshape(len(src), D)
        dq[t], dX, ds = attend_backward_query(q[t], X, sink, scale, p, dout[t], inv_rope, rope_base, rope_dims)
        dsink += ds
        for (k, i), g in zip(src, dX):
            if k == "e":
                dE[i] += g
            else:
                dwin[i] += g
    return dq, dE, dwin, dsink


def csa_attend_backward(q, E, idx, win, sink, scale, q_pos0, dout, W=128, inv_rope=False,
                        rope_base=10000.0, rope_dims=0):
    """Backward of ``csa_attend`` for one sequence: q [Tq, H, D], E [N, D],
    idx [Tq, k] (-1 absent), win [W-1+Tq, D], dout [Tq, H, D].
    Returns (dq, dE, dwin, dsink); entries and window rows collect the
    gradients of every query that read them."""
    return _attend_backward(q, E, list(idx), win, sink, scale, q_pos0, W, inv_rope, rope_base, rope_dims, dout)


def hca_attend_backward(q, E, m, win, sink, scale, q_pos0, dout, W=128, inv_rope=False,
                        rope_base=10000.0, rope_dims=0):
    """Backward of ``hca_attend``: every query reads all its visible entries."""
    Tq = q.shape[0]
    sels = [np.arange(n_visible(q_pos0 + t, m)) for t in range(Tq)]
    return _attend_backward(q, E, sels, win, sink, scale, q_pos0, W, inv_rope, rope_base, rope_dims, dout)


def compress_backward(dout, cb, zb, m, ca=None, za=None, prev_ca=None, prev_za=None, overlap=True,
                      pos0=0, norm_w=None, eps=1e-6, rope_base=None, rope_dims=0):
    """Gradients of ``compress_epilogue(compress_sequence(...))`` with respect to
    its inputs, given ``dout`` = dL/d(entries) [T // m, D].

    [kwkr] §4.3 names the backward of the whole attention block as a training
    workload; this is the compressor's part, written from the forward's own
    definition by the chain rule, block by block:
      RoPE at pos0 + j*m is a rotation, so its adjoint turns dy back by the
      same angle; RMSNorm y = e g / r with r = sqrt(mean(e^2) + eps) gives
      de = g dy / r - e (sum g dy e) / (D r^3) and dg += dy e / r;
      the merge e = sum_i w_i x_i with w = softmax(l) gives dx_i = w_i de and
      dl_i = w_i (x_i . de - e . de).
    Every stream-a row feeds one entry (the next block's) and every stream-b
    row one (its own), so nothing sums across blocks but dnorm_w. Rows no
    entry reads (stream a of the last block, a trailing partial block) get 0.

    Returns a dict of float64 arrays: dcb [T, D], dzb [T], and with overlap
    dca [T, D], dza [T], dprev_ca [m, D] and dprev_za [m] (when prev_ca is
    given); dnorm_w [D] when norm_w is given.

    Pinned by: central finite differences of the forward on small random
    inputs for every output, with and without the epilogue and the carried
    rows, CSA and HCA shapes; equal logits give dx_i = de / n and
    dl_i = (x_i - mean x) . de / n (tests/test_oracle_compress_backward.py).
    """
    cb = np.asarray(cb, dtype=np.float64)
    zb = np.asarray(zb, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    T, D = cb.shape
    n_out = T // m
    res = {"dcb": np.zeros((T, D)), "dzb": np.zeros(T)}
    if overlap:
        ca = np.asarray(ca, dtype=np.float64)
        za = np.asarray(za, dtype=np.float64)
        res["dca"] = np.zeros((T, D))
        res["dza"] = np.zeros(T)
        if prev_ca is not None:
            res["dprev_ca"] = np.zeros((m, D))
            res["dprev_za"] = np.zeros(m)
    if norm_w is not None:
        g = np.asarray(norm_w, dtype=np.float64)
        res["dnorm_w"] = np.zeros(D)
    for j in range(n_out):
        # the block's rows and logits, with where each goes back to
        parts = []                                   # (rows, logits, grad rows, grad logits, offset)
        if overlap:
            if j == 0:
                if prev_ca is not None:
                    parts.append((np.asarray(prev_ca, dtype=np.float64), np.asarray(prev_za, dtype=np.float64),
                                  res["dprev_ca"], res["dprev_za"], 0))
            else:
                parts.append((ca[(j - 1) * m: j * m], za[(j - 1) * m: j * m], res["dca"], res["dza"], (j - 1) * m))
        parts.append((cb[j * m: (j + 1) * m], zb[j * m: (j + 1) * m], res["dcb"], res["dzb"], j * m))
        x = np.concatenate([p_[0] for p_ in parts], axis=0)
        w = _softmax(np.concatenate([p_[1] for p_ in parts]))
        e = w @ x
        dy = dout[j].copy()
        if rope_dims:
            dy = rope_rotate(dy, -(pos0 + j * m), rope_base, rope_dims)
        if norm_w is not None:
            r = math.sqrt(float(np.mean(e * e)) + eps)
            res["dnorm_w"] += dy * e / r
            gdy = g * dy
            de = gdy / r - e * float(np.dot(gdy, e)) / (D * r ** 3)
        else:
            de = dy
        dx = w[:, None] * de[None, :]
        dl = w * (x @ de - float(np.dot(e, de)))
        i = 0
        for rows, _, grows, glog, off in parts:
            n = rows.shape[0]
            grows[off: off + n] = dx[i: i + n]
            glog[off: off + n] = dl[i: i + n]
            i += n
    return res


# ---------------------------------------------------------------------------
# Storage precisions
# ---------------------------------------------------------------------------

def bf16_round(x):
    """Round to the nearest bfloat16 value, ties to even; returns float64.

    Used for the BF16 index scores ([Qiaomu] FP4量化感知训练, [kwkr] §4.4) and
    for the BF16 RoPE channels of a mixed KV row ([cdjax] §1.1). bfloat16 keeps
    8 significant bits (7 stored) and float32's exponent range (subnormal
    spacing 2**-133). Written from that definition with frexp and
    round-half-even (np.rint), not from float bit patterns.
    Pinned by: torch's float32 -> bfloat16 cast (tests/test_oracle_quant.py).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, exp = np.frexp(a)                 # a in [2**(exp-1), 2**exp)
    exp = np.maximum(exp, -125)          # below 2**-126 the grid is uniform
    step = np.ldexp(1.0, exp - 8)        # spacing of 8 significant bits
    q = np.rint(a / step) * step
    q = np.where(a == 0, 0.0, q)
    return np.copysign(q, x)


def bf16_next(v, direction):
    """Neighbouring bfloat16 value of bf16 value ``v`` (direction +1 / -1)."""
    v = float(v)
    if v == 0.0:
        return direction * 2.0 ** -133
    mant, exp = math.frexp(abs(v))
    step = 2.0 ** (max(exp, -125) - 8)
    if direction * v > 0:
        return v + direction * step
    if mant == 0.5 and exp > -125:      # at a power of two the step below halves
        step /= 2
    return v + direction * step


E4M3_MAX = 448.0


def e4m3fn_encode(x):
    """Encode float values as OCP FP8 E4M3FN codes (uint8), RNE, saturating.

    [cdjax] §1.1: channels other than the RoPE ones are stored in FP8. E4M3FN
    (OCP 8-bit floating point spec): 1 sign, 4 exponent bits with bias 7,
    3 mantissa bits, no infinities, largest finite value 448 (1.75 * 2**8),
    smallest normal 2**-6, subnormal step 2**-9. Magnitudes beyond 448 clamp
    to 448. Written from that definition (frexp + round-half-even).
    Pinned by: torch.float8_e4m3fn casts after clamping and an exhaustive
    decode/encode round trip of all finite codes (tests/test_oracle_quant.py).
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # subnormal range [0, 2**-6): value = q * 2**-9, q in 0..8 (8 = first normal)
    q_sub = np.rint(a / 2.0 ** -9).astype(np.int64)
    # normal range: a = 1.f * 2**e, keep 3 fraction bits
    _, exp = np.frexp(np.where(a > 0, a, 1.0))
    e = exp - 1
    q = np.rint(a / np.ldexp(1.0, e - 3)).astype(np.int64)    # in [8, 16]
    carry = q == 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8, q)
    ef = e + 7
    sat = (ef > 15) | ((ef == 15) & (q - 8 > 6))
    ef = np.where(sat, 15, ef)
    q = np.where(sat, 14, q)
    normal_code = (ef << 3) | (q - 8)
    code = np.where(a < 2.0 ** -6, q_sub, normal_code)   # q_sub == 8 is code 0x08
    return (sign | code).astype(np.uint8)


def e4m3fn_decode(codes):
    """Exact float64 value of E4M3FN codes (NaN codes 0x7F/0xFF -> nan)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mt = c & 0x7
    mag = np.where(ef == 0, mt * 2.0 ** -9, (8 + mt) * np.ldexp(1.0, ef - 10))
    mag = np.where((ef == 15) & (mt == 7), np.nan, mag)
    return s * mag


def kv_mixed_quantize(rows, rope_dims=64):
    """Quantise KV rows to the mixed storage format.

    [cdjax] §1.1: RoPE channels stay in BF16, the other channels go to FP8;
    with the FP4 indexer this brings the KV cache to about 2% of a BF16 GQA8
    cache. Reading (the pages fix neither the scale granularity nor its
    precision): one float32 scale per row, s = amax / 448 over the non-RoPE
    channels (s = 1 when amax = 0), a float32 quantity because it is stored
    as float32; each non-RoPE channel stores e4m3fn(float32(x / s)), the
    quotient taken as one IEEE float32 division so that the stored code is a
    function of the stored scale alone; RoPE channels store bf16(x). Input
    rows are float32 values.

    Pinned by: the scale and codes of hand-built rows (amax exactly 448,
    zero rows, a row whose amax sits on one channel) and the decode bound
    |x - decode| <= half an e4m3 step times s (tests/test_oracle_quant.py).

    Returns (fp8 codes [N, D-R] uint8, bf16 values [N, R] float64,
    scale [N] float32).
    """
    rows = np.asarray(rows, dtype=np.float32)
    n, D = rows.shape
    nq = D - rope_dims
    amax = np.max(np.abs(rows[:, :nq]), axis=1).astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    scaled = (rows[:, :nq] / s[:, None]).astype(np.float32)    # IEEE float32 division
    codes = e4m3fn_encode(scaled.astype(np.float64))
    rope = bf16_round(rows[:, nq:].astype(np.float64))
    return codes, rope, s


def kv_mixed_decode(codes, rope, scales):
    """Float64 rows of the mixed format: e4m3 value * scale, then bf16 tail."""
    body = e4m3fn_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]
    return np.concatenate([body, np.asarray(rope, dtype=np.float64)], axis=1)


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_encode(v):
    """Encode floats to E2M1 (FP4) codes, round to nearest even, saturate.

    OCP Microscaling v1.0 FP4 element: 1 sign, 2 exponent bits (bias 1),
    1 mantissa bit; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}. A value halfway
    between two magnitudes goes to the one whose mantissa bit (code bit 0) is
    0. Magnitudes above 6 saturate to 6. Nearest-grid search, written from
    the table of magnitudes.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 6.0)
    d = np.abs(a[..., None] - E2M1_GRID)                 # [..., 8]
    # among equally near magnitudes prefer an even code: add a tiny tie-break
    # that never changes a strict ordering (grid gaps are >= 0.5)
    d = d + np.where(np.arange(8) % 2 == 1, 1e-12, 0.0)
    code = np.argmin(d, axis=-1).astype(np.int64)
    sign = np.where(np.signbit(v), 8, 0)
    return (sign | code).astype(np.uint8)


def e2m1_decode(code):
    c = np.asarray(code, dtype=np.int64)
    return np.where(c & 8, -1.0, 1.0) * E2M1_GRID[c & 7]


def mxfp4_quantize(x, block=32):
    """MXFP4 quantisation along the last axis (blocks of 32 elements).

    [Qiaomu] FP4量化感知训练 and [kwkr] §3.4 / §4.4: the indexer's QK path runs
    in FP4. Format reading: OCP Microscaling v1.0 MXFP4. Per block, shared
    scale X = 2**(floor(log2(amax)) - 2) stored as E8M0 (biased by 127);
    each element stores e2m1(x / X). amax = 0 gives E8M0 code 0 and zero
    elements. Inputs are float32 values; x / X is exact.

    Returns (codes uint8 [..., n] one code per element, e8m0 uint8 [..., n/32]).
    Packing two codes per byte is a storage detail of the kernel side.
    """
    x = np.asarray(x, dtype=np.float64)
    shp = x.shape
    n = shp[-1]
    blk = x.reshape(-1, n // block, block)
    amax = np.max(np.abs(blk), axis=-1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))      # amax in [2**(e-1), 2**e)
    E = np.clip((e - 1) - 2, -127, 127)
    scales = np.where(amax > 0, E + 127, 0).astype(np.uint8)
    X = np.ldexp(1.0, E)[..., None]
    codes = np.where((amax > 0)[..., None], e2m1_encode(blk / X), 0).astype(np.uint8)
    return codes.reshape(shp), scales.reshape(shp[:-1] + (n // block,))


def mxfp4_decode(codes, scales, block=32):
    """Exact float64 values of MXFP4 codes and E8M0 block scales."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.int64)
    shp = codes.shape
    n = shp[-1]
    vals = e2m1_decode(codes).reshape(-1, n // block, block)
    s = np.ldexp(1.0, scales.reshape(-1, n // block) - 127)[..., None]
    return (vals * s).reshape(shp)


# ---------------------------------------------------------------------------
# Grouped output projection (the step after core attention)
# ---------------------------------------------------------------------------

def grouped_output_projection(o, w_g, w_o, round_mid=True, return_mid=False):
    """Grouped output projection of the attention output.

    [Qiaomu] 预训练策略 (model configurations) and [cdjax] §1.1: the n_h heads
    split into g groups of n_h/g consecutive heads; each group's concatenated
    head outputs project to an intermediate width d_g (Flash: g = 8, Pro: 16,
    d_g = 1024), the g results concatenate, and one more projection maps them
    to the model width. [kwkr] §3.4: this cuts the output projection's
    parameters and FLOPs when heads are many.

    Args:
      o:   [T, n_h, c] attention output rows.
      w_g: [g, d_g, (n_h/g)*c] group projections, row j = intermediate channel j
           (the layout of a linear layer's weight).
      w_o: [d_model, g*d_g] the merging projection.
      round_mid: round the intermediate to bf16 (reading: it is stored in bf16
           between the two products, as the operand of the second one).
      return_mid: also return the intermediate [T, g*d_g] (before rounding).
    Returns: [T, d_model] float64 (and the intermediate with return_mid).

    Pinned by: g = 1 is the plain two-matrix product; the grouped form equals
    the product with the explicit block-diagonal matrix; permuting heads inside
    a group together with the matching weight columns changes nothing; scalar
    loops on tiny inputs (tests/test_oracle_outproj.py).
    """
    o = np.asarray(o, dtype=np.float64)
    w_g = np.asarray(w_g, dtype=np.float64)
    w_o = np.asarray(w_o, dtype=np.float64)
    T, n_h, c = o.shape
    g, d_g, kg = w_g.shape
    assert n_h % g == 0 and kg == (n_h // g) * c
    mids = []
    for gi in range(g):
        xg = o[:, gi * (n_h // g):(gi + 1) * (n_h // g), :].reshape(T, kg)
        mids.append(xg @ w_g[gi].T)
    mid = np.concatenate(mids, axis=1)
    out = (bf16_round(mid) if round_mid else mid) @ w_o.T
    return (out, mid) if return_mid else out

