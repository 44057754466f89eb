"""Seeded synthetic inputs for the CSA / HCA hot path.

This module is shared by the tests (which feed the oracle), the HIP-path
tests and the benchmark. It holds none of the method's arithmetic: it only
draws random numbers and casts them to their storage type (bf16 values are
returned as float32 arrays whose values are exactly representable in bf16,
so both sides read identical numbers).

Recipe (also in the design doc):
* Each sequence b of a workload draws from its own stream
  ``numpy.random.default_rng([seed, b])``, so any sequence regenerates alone;
  tensors shared by the batch (sinks, norm gains) come from
  ``default_rng([seed, 1_000_000])``. Draw order inside a stream is the order
  of the statements below and is part of the recipe.
* Unless noted, a tensor whose last axis has size n is drawn N(0, 1) / sqrt(n)
  in float32; gate logits, sinks are N(0, 1); indexer head weights are
  N(0, 1) / sqrt(H_I).
* "1% spikes" (CSA decode): per sequence floor(0.01 * N) entries, chosen
  without replacement, have both their KV row and their indexer key scaled
  by 4 before the bf16 cast.
* "Student-t query norms" (mixed pair): each query row is g / |g| * |tau|
  with g ~ N(0, I) and tau ~ Student-t with 3 degrees of freedom.
* Ragged decode batches: sequence positions drawn uniformly from the integers
  in [lo, hi] by ``default_rng([seed, 3_000_000])``; the last sequence sits at
  hi (the bound), so the batch always holds one full-length sequence.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_exact",
    "seq_rng",
    "shared_rng",
    "gauss",
    "make_csa_layer",
    "make_csa_decode",
    "make_hca_decode",
    "make_csa_prefill",
    "make_mixed_pair",
    "ragged_positions",
    "WINDOW",
]

WINDOW = 128


def bf16_exact(x) -> np.ndarray:
    """Storage cast: float32 -> nearest bfloat16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def seq_rng(seed: int, b: int) -> np.random.Generator:
    return np.random.default_rng([seed, b])


def shared_rng(seed: int) -> np.random.Generator:
    return np.random.default_rng([seed, 1_000_000])


def gauss(rng: np.random.Generator, shape, scale_last=True) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale_last:
        x *= np.float32(1.0 / np.sqrt(shape[-1]))
    return x


def _seqs(B, seqs):
    return list(range(B)) if seqs is None else list(seqs)


# ---------------------------------------------------------------------------
# Workload 1: one CSA layer forward in fp32 (prefill from position 0)
# ---------------------------------------------------------------------------

def make_csa_layer(seed=1, B=1, T=1024, H=8, D=128, H_I=4, d_I=64, k=64, m=4,
                   rope_dims=64, sharp=1.0, seqs=None):
    """Single CSA layer forward: compressor, indexer, top-k, attention; fp32.

    ``sharp`` multiplies the queries (1.0 reproduces the stated workload;
    larger values make the softmax peaked for stronger tests).
    """
    out = {"cfg": "csa_layer_fp32", "B": B, "T": T, "H": H, "D": D, "H_I": H_I,
           "d_I": d_I, "k": k, "m": m, "W": WINDOW, "rope_dims": rope_dims,
           "q_pos0": 0, "pos0": 0, "rope_base": 10000.0, "eps": 1e-6,
           "dtype": "f32"}
    names = ["ca", "za", "cb", "zb", "ica", "iza", "icb", "izb", "q", "qI", "w", "win"]
    per = {n: [] for n in names}
    for b in _seqs(B, seqs):
        r = seq_rng(seed, b)
        per["ca"].append(gauss(r, (T, D)))
        per["za"].append(r.standard_normal(T, dtype=np.float32))
        per["cb"].append(gauss(r, (T, D)))
        per["zb"].append(r.standard_normal(T, dtype=np.float32))
        per["ica"].append(gauss(r, (T, d_I)))
        per["iza"].append(r.standard_normal(T, dtype=np.float32))
        per["icb"].append(gauss(r, (T, d_I)))
        per["izb"].append(r.standard_normal(T, dtype=np.float32))
        per["q"].append(gauss(r, (T, H, D)) * np.float32(sharp))
        per["qI"].append(gauss(r, (T, H_I, d_I)))
        per["w"].append(r.standard_normal((T, H_I), dtype=np.float32)
                        * np.float32(1.0 / np.sqrt(H_I)))
        per["win"].append(gauss(r, (WINDOW - 1 + T, D)))
    for n in names:
        out[n] = np.ascontiguousarray(np.stack(per[n]))
    s = shared_rng(seed)
    out["sink"] = s.standard_normal(H, dtype=np.float32)
    out["norm_w"] = (np.float32(1.0 / np.sqrt(D))
                     * (1 + np.float32(0.1) * s.standard_normal(D, dtype=np.float32))).astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# Workload 2: CSA decode, V4-Flash shaped
# ---------------------------------------------------------------------------

def make_csa_decode(seed=2, B=16, ctx=131072, H=64, D=512, H_I=4, d_I=128, k=512,
                    m=4, spike_frac=0.01, sharp=1.0, seqs=None):
    """CSA decode: one new token per sequence after ``ctx`` tokens; bf16 data."""
    N = ctx // m
    q_pos0 = ctx
    out = {"cfg": "csa_decode_bf16", "B": B, "H": H, "D": D, "H_I": H_I, "d_I": d_I,
           "k": k, "m": m, "W": WINDOW, "N": N, "q_pos0": q_pos0, "rope_dims": 64,
           "rope_base": 10000.0, "dtype": "bf16"}
    E, KI, Q, QI, Wt, WIN = [], [], [], [], [], []
    for b in _seqs(B, seqs):
        r = seq_rng(seed, b)
        e = gauss(r, (N, D))
        ki = gauss(r, (N, d_I))
        n_spk = int(spike_frac * N)
        if n_spk:
            spk = r.choice(N, size=n_spk, replace=False)
            e[spk] *= np.float32(4.0)
            ki[spk] *= np.float32(4.0)
        E.append(bf16_exact(e))
        KI.append(bf16_exact(ki))
        Q.append(bf16_exact(gauss(r, (1, H, D)) * np.float32(sharp)))
        QI.append(bf16_exact(gauss(r, (1, H_I, d_I))))
        Wt.append(r.standard_normal((1, H_I), dtype=np.float32) * np.float32(1 / np.sqrt(H_I)))
        WIN.append(bf16_exact(gauss(r, (WINDOW, D))))
    out["E"] = np.stack(E)
    out["kI"] = np.stack(KI)
    out["q"] = np.stack(Q)
    out["qI"] = np.stack(QI)
    out["w"] = np.stack(Wt)
    out["win"] = np.stack(WIN)
    out["sink"] = shared_rng(seed).standard_normal(H, dtype=np.float32)
    return out


# ---------------------------------------------------------------------------
# Workload 3: HCA decode, V4-Pro shaped
# ---------------------------------------------------------------------------

def make_hca_decode(seed=3, B=8, ctx=1048576, H=128, D=512, m=128, sharp=1.0,
                    seqs=None):
    """HCA decode: dense MQA over ctx/128 compressed entries + window + sink."""
    N = ctx // m
    out = {"cfg": "hca_decode_bf16", "B": B, "H": H, "D": D, "m": m, "W": WINDOW,
           "N": N, "q_pos0": ctx, "rope_dims": 64, "rope_base": 10000.0,
           "dtype": "bf16"}
    E, Q, WIN = [], [], []
    for b in _seqs(B, seqs):
        r = seq_rng(seed, b)
        E.append(bf16_exact(gauss(r, (N, D))))
        Q.append(bf16_exact(gauss(r, (1, H, D)) * np.float32(sharp)))
        WIN.append(bf16_exact(gauss(r, (WINDOW, D))))
    out["E"] = np.stack(E)
    out["q"] = np.stack(Q)
    out["win"] = np.stack(WIN)
    out["sink"] = shared_rng(seed).standard_normal(H, dtype=np.float32)
    return out


# ---------------------------------------------------------------------------
# Workload 4: CSA chunked prefill, V4-Pro shaped
# ---------------------------------------------------------------------------

def make_csa_prefill(seed=4, ctx=1048576, Tq=4096, H=128, D=512, H_I=4, d_I=128,
                     k=1024, m=4, sharp=1.0, q_rows=None):
    """Chunked prefill of Tq new tokens after ``ctx`` context tokens (B = 1).

    The context's compressed prefix (ctx/m entries and indexer keys) is given;
    the new tokens' raw streams are compressed by the path itself. ``q_rows``
    restricts the drawn queries to a subset (others are left zero) to keep
    oracle-side memory small; the full draw order is kept either way.
    """
    N0 = ctx // m
    r = seq_rng(seed, 0)
    out = {"cfg": "csa_prefill_bf16", "B": 1, "Tq": Tq, "H": H, "D": D, "H_I": H_I,
           "d_I": d_I, "k": k, "m": m, "W": WINDOW, "N0": N0,
           "N_cap": N0 + Tq // m, "q_pos0": ctx, "pos0": ctx, "rope_dims": 64,
           "rope_base": 10000.0, "eps": 1e-6, "dtype": "bf16"}
    out["E_prefix"] = bf16_exact(gauss(r, (1, N0, D)))
    out["kI_prefix"] = bf16_exact(gauss(r, (1, N0, d_I)))
    out["ca"] = bf16_exact(gauss(r, (1, Tq, D)))
    out["za"] = r.standard_normal((1, Tq), dtype=np.float32)
    out["cb"] = bf16_exact(gauss(r, (1, Tq, D)))
    out["zb"] = r.standard_normal((1, Tq), dtype=np.float32)
    out["prev_ca"] = bf16_exact(gauss(r, (1, m, D)))
    out["prev_za"] = r.standard_normal((1, m), dtype=np.float32)
    out["ica"] = bf16_exact(gauss(r, (1, Tq, d_I)))
    out["iza"] = r.standard_normal((1, Tq), dtype=np.float32)
    out["icb"] = bf16_exact(gauss(r, (1, Tq, d_I)))
    out["izb"] = r.standard_normal((1, Tq), dtype=np.float32)
    out["iprev_ca"] = bf16_exact(gauss(r, (1, m, d_I)))
    out["iprev_za"] = r.standard_normal((1, m), dtype=np.float32)
    # queries: drawn in blocks of 256 rows so a subset costs little memory
    q = np.zeros((1, Tq, H, D), dtype=np.float32)
    qI = np.zeros((1, Tq, H_I, d_I), dtype=np.float32)
    want = None if q_rows is None else set(int(t) for t in q_rows)
    for t0 in range(0, Tq, 256):
        blk = gauss(r, (min(256, Tq - t0), H, D)) * np.float32(sharp)
        blkI = gauss(r, (min(256, Tq - t0), H_I, d_I))
        if want is None:
            q[0, t0:t0 + blk.shape[0]] = blk
            qI[0, t0:t0 + blk.shape[0]] = blkI
        else:
            for t in range(t0, t0 + blk.shape[0]):
                if t in want:
                    q[0, t] = blk[t - t0]
                    qI[0, t] = blkI[t - t0]
    out["q"] = bf16_exact(q)
    out["qI"] = bf16_exact(qI)
    out["w"] = r.standard_normal((1, Tq, H_I), dtype=np.float32) * np.float32(1 / np.sqrt(H_I))
    out["win"] = bf16_exact(gauss(r, (1, WINDOW - 1 + Tq, D)))
    s = shared_rng(seed)
    out["sink"] = s.standard_normal(H, dtype=np.float32)
    out["norm_w"] = (np.float32(1.0 / np.sqrt(D))
                     * (1 + np.float32(0.1) * s.standard_normal(D, dtype=np.float32))).astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# Workload 5: mixed-precision interleaved CSA + HCA layer pair, decode
# ---------------------------------------------------------------------------

def _student_t_rows(r, shape):
    g = r.standard_normal(size=shape, dtype=np.float32)
    tau = r.standard_t(3, size=shape[:-1]).astype(np.float32)
    nrm = np.sqrt(np.sum(g.astype(np.float64) ** 2, axis=-1)).astype(np.float32)
    return (g / nrm[..., None] * np.abs(tau)[..., None]).astype(np.float32)


def make_mixed_pair(seed=5, B=64, ctx=1048576, H=128, D=512, H_I=4, d_I=128,
                    k=1024, m=4, m2=128, seqs=None):
    """Mixed-precision CSA layer + HCA layer decode pair.

    All KV sources are float32; the path quantises them itself (fp8 e4m3 with
    per-row scale plus bf16 RoPE channels; MXFP4 indexer operands).
    """
    N = ctx // m
    N2 = ctx // m2
    out = {"cfg": "mixed_pair", "B": B, "H": H, "D": D, "H_I": H_I, "d_I": d_I,
           "k": k, "m": m, "m2": m2, "W": WINDOW, "N": N, "N2": N2, "q_pos0": ctx,
           "rope_dims": 64, "rope_base": 10000.0}
    names = ["E", "kI", "win", "q", "qI", "w", "E2", "win2", "q2"]
    per = {n: [] for n in names}
    for b in _seqs(B, seqs):
        r = seq_rng(seed, b)
        per["E"].append(gauss(r, (N, D)))
        per["kI"].append(gauss(r, (N, d_I)))
        per["win"].append(gauss(r, (WINDOW, D)))
        per["q"].append(bf16_exact(_student_t_rows(r, (1, H, D))))
        per["qI"].append(_student_t_rows(r, (1, H_I, d_I)))
        per["w"].append(r.standard_normal((1, H_I), dtype=np.float32) * np.float32(1 / np.sqrt(H_I)))
        per["E2"].append(gauss(r, (N2, D)))
        per["win2"].append(gauss(r, (WINDOW, D)))
        per["q2"].append(bf16_exact(_student_t_rows(r, (1, H, D))))
    for n in names:
        out[n] = np.stack(per[n])
    s = shared_rng(seed)
    out["sink"] = s.standard_normal(H, dtype=np.float32)
    out["sink2"] = s.standard_normal(H, dtype=np.float32)
    return out


def ragged_positions(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence positions of a ragged decode batch (int64 [B])."""
    pos = np.random.default_rng([seed, 3_000_000]).integers(lo, hi + 1, size=B, dtype=np.int64)
    pos[-1] = hi
    return pos
