"""Pins of the oracle's token compressor against closed forms and invariants.

The pages give the compressor only in words ([kwkr] §3.1: two independent KV
sequences, softmax-normalised gate weights, overlapping adjacent blocks). Each
test below fails for a plausible mistake: separate softmaxes per stream, the
wrong block for stream a, a missing or zero-padded first block, a dropped
normalisation, or a carry that does not resume exactly.
"""

import numpy as np
import pytest

import oracle as O


def _rand(rng, T, D):
    return rng.standard_normal((T, D)), rng.standard_normal(T)


@pytest.mark.parametrize("with_prev", [False, True])
def test_constant_sequence_compresses_to_itself(with_prev):
    # A constant sequence must compress to itself for any gate logits: the
    # weights are softmax-normalised (sum to 1). Zero-padding the missing
    # block j-1 at j = 0, or two separate softmaxes, would break this.
    rng = np.random.default_rng(0)
    T, D, m = 32, 8, 4
    c = rng.standard_normal(D)
    ca = np.tile(c, (T, 1))
    cb = np.tile(c, (T, 1))
    za, zb = rng.standard_normal(T) * 3, rng.standard_normal(T) * 3
    prev = (np.tile(c, (m, 1)), rng.standard_normal(m)) if with_prev else (None, None)
    e = O.compress_sequence(cb, zb, m, ca, za, prev[0], prev[1], overlap=True)
    assert e.shape == (T // m, D)
    np.testing.assert_allclose(e, np.tile(c, (T // m, 1)), rtol=0, atol=1e-14)


def test_equal_logits_give_mean_of_overlapping_rows():
    rng = np.random.default_rng(1)
    T, D, m = 24, 5, 4
    ca, _ = _rand(rng, T, D)
    cb, _ = _rand(rng, T, D)
    z = np.full(T, 0.7)
    e = O.compress_sequence(cb, z, m, ca, z, overlap=True)
    # j = 0: only block 0 of stream b (block -1 is absent) -> mean of 4 rows
    np.testing.assert_allclose(e[0], cb[0:4].mean(axis=0), atol=1e-14)
    for j in range(1, T // m):
        want = (ca[(j - 1) * m: j * m].sum(0) + cb[j * m:(j + 1) * m].sum(0)) / (2 * m)
        np.testing.assert_allclose(e[j], want, atol=1e-14)


def test_dominant_logit_selects_its_row():
    rng = np.random.default_rng(2)
    T, D, m = 16, 6, 4
    ca, za = _rand(rng, T, D)
    cb, zb = _rand(rng, T, D)
    # make row 5 of stream a dominate entry 2 (stream a block 1 = rows 4..7)
    za = za.copy()
    za[5] = 60.0
    e = O.compress_sequence(cb, zb, m, ca, za, overlap=True)
    np.testing.assert_allclose(e[2], ca[5], atol=1e-12)
    # ... and row 9 of stream b dominates entry 2 (stream b block 2 = rows 8..11)
    zb = zb.copy()
    zb[9] = 200.0
    e = O.compress_sequence(cb, zb, m, ca, za, overlap=True)
    np.testing.assert_allclose(e[2], cb[9], atol=1e-12)


def test_stream_roles_closed_form():
    # Silencing one stream leaves a plain softmax-weighted mean of the other,
    # over block j-1 (stream a) or block j (stream b).
    rng = np.random.default_rng(3)
    T, D, m = 20, 3, 4
    ca, za = _rand(rng, T, D)
    cb, zb = _rand(rng, T, D)
    e = O.compress_sequence(cb, np.full(T, -1e4), m, ca, za, overlap=True)
    for j in range(1, T // m):
        lg = za[(j - 1) * m: j * m]
        w = np.exp(lg - lg.max()) / np.exp(lg - lg.max()).sum()
        np.testing.assert_allclose(e[j], w @ ca[(j - 1) * m: j * m], atol=1e-12)
    e = O.compress_sequence(cb, zb, m, ca, np.full(T, -1e4), overlap=True)
    for j in range(T // m):
        lg = zb[j * m:(j + 1) * m]
        w = np.exp(lg - lg.max()) / np.exp(lg - lg.max()).sum()
        np.testing.assert_allclose(e[j], w @ cb[j * m:(j + 1) * m], atol=1e-12)


def test_linear_in_rows_for_fixed_gates():
    rng = np.random.default_rng(4)
    T, D, m = 32, 7, 4
    a1, za = _rand(rng, T, D)
    b1, zb = _rand(rng, T, D)
    a2, _ = _rand(rng, T, D)
    b2, _ = _rand(rng, T, D)
    al, be = 0.3, -1.7
    lhs = O.compress_sequence(al * b1 + be * b2, zb, m, al * a1 + be * a2, za)
    rhs = al * O.compress_sequence(b1, zb, m, a1, za) + be * O.compress_sequence(b2, zb, m, a2, za)
    np.testing.assert_allclose(lhs, rhs, atol=1e-13)


def test_shift_of_all_logits_changes_nothing():
    rng = np.random.default_rng(5)
    T, D, m = 16, 4, 4
    ca, za = _rand(rng, T, D)
    cb, zb = _rand(rng, T, D)
    e1 = O.compress_sequence(cb, zb, m, ca, za)
    e2 = O.compress_sequence(cb, zb + 3.25, m, ca, za + 3.25)
    np.testing.assert_allclose(e1, e2, atol=1e-13)


@pytest.mark.parametrize("T1", [4, 8, 12, 28])
def test_chunked_equals_one_shot(T1):
    # Compressing [0, T1) and then [T1, T) with the last block of stream a
    # carried over must equal compressing [0, T) at once.
    rng = np.random.default_rng(6)
    T, D, m = 32, 6, 4
    ca, za = _rand(rng, T, D)
    cb, zb = _rand(rng, T, D)
    full = O.compress_sequence(cb, zb, m, ca, za)
    first = O.compress_sequence(cb[:T1], zb[:T1], m, ca[:T1], za[:T1])
    second = O.compress_sequence(cb[T1:], zb[T1:], m, ca[T1:], za[T1:],
                                 prev_ca=ca[T1 - m:T1], prev_za=za[T1 - m:T1])
    np.testing.assert_allclose(np.concatenate([first, second]), full, atol=1e-14)


@pytest.mark.parametrize("m,overlap,T", [(4, True, 37), (128, False, 300), (2, True, 9)])
def test_token_at_a_time_equals_one_shot(m, overlap, T):
    # The decode-time compressor, fed one token at a time, emits entry j when
    # token j*m + m - 1 arrives, and the entries are those of the one-shot
    # compressor over the whole sequence (the overlap tail carried in state).
    rng = np.random.default_rng(60 + m)
    D = 5
    ca, za = _rand(rng, T, D)
    cb, zb = _rand(rng, T, D)
    full = O.compress_sequence(cb, zb, m, ca, za, overlap=overlap) if overlap else \
        O.compress_sequence(cb, zb, m, overlap=False)
    st = O.CompressorState(m, overlap)
    got = []
    for t in range(T):
        r = st.append(cb[t], zb[t], ca[t] if overlap else None, za[t] if overlap else None)
        if (t + 1) % m == 0:
            assert r is not None and r[0] == t // m
            got.append(r[1])
        else:
            assert r is None
    assert len(got) == T // m
    np.testing.assert_allclose(np.array(got), full, atol=1e-14)


def test_token_at_a_time_overlap_tail_matters():
    # A wrong tail (a block other than j-1, or none) changes the entries: the
    # state must carry exactly stream a's previous block.
    rng = np.random.default_rng(61)
    T, D, m = 16, 3, 4
    ca, za = _rand(rng, T, D)
    cb, zb = _rand(rng, T, D)
    st = O.CompressorState(m, True)
    ents = [st.append(cb[t], zb[t], ca[t], za[t]) for t in range(T)]
    ents = [e[1] for e in ents if e is not None]
    no_overlap = O.compress_sequence(cb, zb, m, overlap=False)
    assert np.allclose(ents[0], no_overlap[0], atol=1e-14)          # block 0: no tail
    for j in range(1, T // m):
        assert not np.allclose(ents[j], no_overlap[j], atol=1e-3)


def test_trailing_partial_block_emits_nothing():
    rng = np.random.default_rng(7)
    ca, za = _rand(rng, 14, 3)
    cb, zb = _rand(rng, 14, 3)
    e = O.compress_sequence(cb, zb, 4, ca, za)
    assert e.shape == (3, 3)


def test_hca_compressor_is_blockwise_softmax_pool():
    # m' = 128, single stream, no overlap: equal logits give the block mean;
    # the block result equals numpy's softmax-weighted average.
    rng = np.random.default_rng(8)
    T, D, m = 384, 5, 128
    cb, zb = _rand(rng, T, D)
    e = O.compress_sequence(cb, np.zeros(T), m, overlap=False)
    np.testing.assert_allclose(e, cb.reshape(3, m, D).mean(axis=1), atol=1e-13)
    e = O.compress_sequence(cb, zb, m, overlap=False)
    for j in range(3):
        w = np.exp(zb[j * m:(j + 1) * m])
        np.testing.assert_allclose(e[j], np.average(cb[j * m:(j + 1) * m], axis=0, weights=w),
                                   atol=1e-13)


def test_brute_force_tiny():
    # Scalar loops over an explicit list of (row, logit) pairs per entry.
    rng = np.random.default_rng(9)
    T, D, m = 12, 2, 4
    ca, za = _rand(rng, T, D)
    cb, zb = _rand(rng, T, D)
    pa, pz = rng.standard_normal((m, D)), rng.standard_normal(m)
    e = O.compress_sequence(cb, zb, m, ca, za, pa, pz)
    for j in range(T // m):
        pairs = []
        for i in range(m):
            if j == 0:
                pairs.append((pa[i], pz[i]))
            else:
                pairs.append((ca[(j - 1) * m + i], za[(j - 1) * m + i]))
        for i in range(m):
            pairs.append((cb[j * m + i], zb[j * m + i]))
        den = sum(np.exp(z) for _, z in pairs)
        for d in range(D):
            num = sum(np.exp(z) * r[d] for r, z in pairs)
            assert abs(e[j, d] - num / den) < 1e-13


def test_rms_norm_unit_rms():
    rng = np.random.default_rng(10)
    x = rng.standard_normal(64) * 5
    y = O.rms_norm(x, np.ones(64), 0.0)
    assert abs(np.sqrt(np.mean(y * y)) - 1.0) < 1e-14
    g = rng.standard_normal(64)
    np.testing.assert_allclose(O.rms_norm(x, g, 0.0), y * g, atol=1e-14)


# ---------------------------------------------------------------------------
# Epilogue: merge -> RMSNorm -> RoPE at the block start pos0 + j*m
# ([Qiaomu] 混合注意力机制: normalised entries; [cdjax] §1.1: RoPE on the last
# 64 channels). Each test fails for a plausible slip: RoPE at j (or pos0 + j)
# instead of pos0 + j*m, the chunk offset pos0 dropped, RoPE applied before
# the norm under a gain that differs across the rotated channels, or a
# rotation that does not preserve the row's norm.
# ---------------------------------------------------------------------------

def _rope_ref(x, pos, base, R):
    """The rotation written from its complex-exponential definition, apart
    from the oracle: pair (u, v) = u + iv of the last R channels times
    exp(i * pos * base**(-2i/R))."""
    y = np.array(x, dtype=np.float64, copy=True)
    D = y.shape[-1]
    z = y[..., D - R::2] + 1j * y[..., D - R + 1::2]
    z = z * np.exp(1j * pos * base ** (-np.arange(0, R, 2) / R))
    y[..., D - R::2] = z.real
    y[..., D - R + 1::2] = z.imag
    return y


@pytest.mark.parametrize("T1", [4, 12, 20])
def test_epilogue_chunked_equals_one_shot(T1):
    # Compress + epilogue over [0, T1) at pos0 = 0, then over [T1, T) at
    # pos0 = T1 with stream a's last block carried, equals one call over
    # [0, T). A RoPE position that ignores pos0 or scales j by anything but m
    # breaks the second chunk.
    rng = np.random.default_rng(70)
    T, D, m, R, base = 32, 16, 4, 8, 10000.0
    ca, za = _rand(rng, T, D)
    cb, zb = _rand(rng, T, D)
    g = 0.5 + rng.random(D)
    ep = dict(norm_w=g, eps=1e-6, rope_base=base, rope_dims=R)
    full = O.compress_epilogue(O.compress_sequence(cb, zb, m, ca, za), 0, m, **ep)
    first = O.compress_epilogue(O.compress_sequence(cb[:T1], zb[:T1], m, ca[:T1], za[:T1]), 0, m, **ep)
    second = O.compress_epilogue(
        O.compress_sequence(cb[T1:], zb[T1:], m, ca[T1:], za[T1:], prev_ca=ca[T1 - m:T1],
                            prev_za=za[T1 - m:T1]), T1, m, **ep)
    np.testing.assert_allclose(np.concatenate([first, second]), full, atol=1e-13)


@pytest.mark.parametrize("m", [4, 128])
def test_epilogue_entry_sits_at_block_start(m):
    # A constant sequence compresses to itself, so every entry is the same
    # row before RoPE; after the epilogue, entry j's dot with a query rotated
    # to position p depends only on p - (pos0 + j*m). Checked against the
    # complex-exponential rotation written above, not the oracle's own.
    rng = np.random.default_rng(71)
    D, R, base, pos0 = 16, 8, 10000.0, 1048576
    n = 6
    T = n * m
    c = rng.standard_normal(D)
    rows = np.tile(c, (T, 1))
    e = O.compress_sequence(rows, rng.standard_normal(T), m, overlap=False)
    out = O.compress_epilogue(e, pos0, m, norm_w=None, rope_base=base, rope_dims=R)
    for j in range(n):
        np.testing.assert_allclose(out[j], _rope_ref(c, pos0 + j * m, base, R), atol=1e-9)
    q = rng.standard_normal(D)
    delta = 3 * m + 1
    dots = [out[j] @ _rope_ref(q, pos0 + j * m + delta, base, R) for j in range(n)]
    np.testing.assert_allclose(dots, dots[0], atol=1e-9)
    # the same dot at a position one token off differs (the test can see a shift)
    off = out[2] @ _rope_ref(q, pos0 + 2 * m + delta + 1, base, R)
    assert abs(off - dots[0]) > 1e-6


def test_epilogue_norm_before_rope_under_nonuniform_gain():
    # Rotating the output back by -(pos0 + j*m) must give g * e / rms(e): a
    # row parallel to g * e whose entry-wise ratio to g has unit RMS (eps 0).
    # With RoPE before the norm, a gain that differs between the two channels
    # of a rotated pair would leave a different row.
    rng = np.random.default_rng(72)
    D, R, m, pos0, base = 32, 16, 4, 4096, 10000.0
    e = rng.standard_normal((5, D)) * 3
    g = np.linspace(0.25, 4.0, D)
    out = O.compress_epilogue(e, pos0, m, norm_w=g, eps=0.0, rope_base=base, rope_dims=R)
    for j in range(5):
        back = _rope_ref(out[j], -(pos0 + j * m), base, R)
        u = back / g
        assert abs(np.sqrt(np.mean(u * u)) - 1.0) < 1e-12
        np.testing.assert_allclose(u * np.sqrt(np.mean(e[j] ** 2)), e[j], atol=1e-12)
    # the other order gives another row (the test discriminates)
    wrong = O.rms_norm(_rope_ref(e[1], pos0 + m, base, R), g, 0.0)
    assert np.max(np.abs(wrong - out[1])) > 1e-3


def test_epilogue_unit_gain_keeps_unit_rms():
    # RMSNorm with unit gain, then a rotation: the output RMS stays 1.
    rng = np.random.default_rng(73)
    e = rng.standard_normal((7, 64)) * 11
    out = O.compress_epilogue(e, 128, 4, norm_w=np.ones(64), eps=0.0, rope_base=10000.0, rope_dims=64)
    np.testing.assert_allclose(np.sqrt(np.mean(out ** 2, axis=1)), 1.0, atol=1e-13)
    # and without norm or RoPE the epilogue is the identity
    np.testing.assert_array_equal(O.compress_epilogue(e, 128, 4), e)
