"""The Python binding checks every tensor against the dimensions it passes to
the C library (dtype, contiguity, shape or byte size, device) and raises
before any pointer reaches it. These run on CPU tensors: a well-formed call
fails only on the device check, a malformed one on its own mismatch."""

import os

import pytest
import torch

import long_context_attention_12_amd as L

pytestmark = pytest.mark.skipif(not os.path.exists(L.lib_path), reason="liblca.so not built")

bf, f32, i32, u8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def _raises(fn, fragment):
    with pytest.raises((ValueError, TypeError)) as e:
        fn()
    assert fragment in str(e.value), str(e.value)


# CSA decode-like shapes, kept small: B=2, Tq=1, H=16, D=512, N=64 entries
B, Tq, H, D, N, W, k, HI, dI = 2, 1, 16, 512, 64, 8, 16, 4, 128


def attend_args(**over):
    a = dict(q=z(B, Tq, H, D), kv=z(B, N, D), idx=z(B, Tq, k, dtype=i32), win=z(B, W - 1 + Tq, D),
             sink=z(H, dtype=f32), out=z(B, Tq, H, D))
    a.update(over)
    return a


def call_attend(**over):
    a = attend_args(**over)
    extra = {kk: a.pop(kk) for kk in list(a) if kk not in ("q", "kv", "idx", "win", "sink", "out")}
    L.csa_attend(L.BF16, L.BF16, a["q"], a["kv"], a["idx"], a["win"], a["sink"], a["out"], m=4, W=W,
                 q_pos0=300, scale=0.04, **extra)


def test_attend_well_formed_fails_only_on_device():
    _raises(call_attend, "device memory only")


@pytest.mark.parametrize("over,fragment", [
    (dict(q=z(B, Tq, H, D, dtype=f32)), "q has dtype torch.float32"),
    (dict(q=z(B, Tq, H * D)), "q must be [B, Tq, H, D]"),
    (dict(kv=z(B, N, D // 2)), "kv rows hold 512 bytes; the call needs 1024"),
    (dict(kv=z(B + 1, N, D)), "kv has shape"),
    (dict(N_cap=N + 1), "kv holds 64 rows per sequence; the call needs 65"),
    (dict(win=z(B, W - 2 + Tq, D)), "win holds 7 rows per sequence; the call needs 8"),
    (dict(win=z(B, W - 1 + Tq, D).transpose(0, 1).contiguous().transpose(0, 1)), "win must be contiguous"),
    (dict(idx=z(B, Tq + 1, k, dtype=i32)), "idx must be [2, 1, k]"),
    (dict(idx=z(B, Tq, k, dtype=torch.int64)), "idx has dtype"),
    (dict(sink=z(H - 1, dtype=f32)), "sink has 15 elements; the call needs 16"),
    (dict(out=z(B, Tq, H, D - 32)), "out has"),
    (dict(out=z(B, Tq, H, D, dtype=f32)), "out has dtype"),
    (dict(lse_out=z(B, Tq, H + 1, dtype=f32)), "lse_out has"),
    (dict(q_pos=z(B + 1, dtype=torch.int64)), "q_pos has 3 elements"),
    (dict(ws=z(64, dtype=u8)[::2]), "ws must be contiguous"),
    (dict(sink=[0.0] * H), "sink must be a torch.Tensor"),
])
def test_attend_mismatch_raises(over, fragment):
    _raises(lambda: call_attend(**over), fragment)


def test_attend_kv_mixed_needs_scales_and_row_bytes():
    mixed = dict(kv=z(B, N, D + 64, dtype=u8), win=z(B, W - 1 + Tq, D + 64, dtype=u8))
    f = lambda **o: L.csa_attend(L.BF16, L.KV_MIXED, z(B, Tq, H, D), o.get("kv", mixed["kv"]),
                                 z(B, Tq, k, dtype=i32), o.get("win", mixed["win"]), z(H, dtype=f32),
                                 z(B, Tq, H, D), m=4, W=W, q_pos0=300, scale=0.04, rope_dims=64,
                                 kv_scale=o.get("kv_scale"), win_scale=o.get("win_scale", z(B, W, dtype=f32)))
    _raises(lambda: f(), "kv_scale is required")
    _raises(lambda: f(kv_scale=z(B, N - 1, dtype=f32)), "kv_scale has")
    _raises(lambda: f(kv=z(B, N, D, dtype=u8), kv_scale=z(B, N, dtype=f32)), "kv rows hold 512 bytes")
    _raises(lambda: f(kv_scale=z(B, N, dtype=f32)), "device memory only")


def test_hca_attend_checks():
    f = lambda **o: L.hca_attend(L.BF16, L.BF16, o.get("q", z(B, Tq, H, D)), o.get("kv", z(B, N, D)),
                                 o.get("win", z(B, W - 1 + Tq, D)), z(H, dtype=f32), z(B, Tq, H, D),
                                 m=128, W=W, q_pos0=300, scale=0.04, N_cap=o.get("N_cap"))
    _raises(lambda: f(), "device memory only")
    _raises(lambda: f(N_cap=N * 2), "the call needs 128")
    _raises(lambda: f(win=z(B, W + 5, D)), "win holds")


def call_index(**over):
    a = dict(qI=z(B, Tq, HI, dI), w=z(B, Tq, HI, dtype=f32), kI=z(B, N, dI), idx=z(B, Tq, k, dtype=i32))
    a.update(over)
    kw = {kk: a[kk] for kk in ("score_out", "qI_scale", "kI_scale", "d_I") if kk in a}
    L.csa_index_topk(a.get("dt", L.BF16), a["qI"], a["w"], a["kI"], a["idx"], m=4, k=a.get("k", k),
                     q_pos0=300, **kw)


@pytest.mark.parametrize("over,fragment", [
    (dict(), "device memory only"),
    (dict(k=k + 1), "idx_out has 32 elements; the call needs 34"),
    (dict(idx=z(B, Tq, k)), "idx_out has dtype"),
    (dict(w=z(B, Tq, HI + 1, dtype=f32)), "w has"),
    (dict(kI=z(B, N, dI // 2)), "kI rows hold 128 bytes; the call needs 256"),
    (dict(qI=z(B, Tq, HI, dI, dtype=f32)), "qI has dtype"),
    (dict(score_out=z(B, Tq, k + 1, dtype=f32)), "score_out has"),
    (dict(dt=L.MXFP4, qI=z(B, Tq, HI, 64, dtype=u8), kI=z(B, N, 64, dtype=u8)), "qI_scale is required"),
    (dict(dt=L.MXFP4, qI=z(B, Tq, HI, 64, dtype=u8), kI=z(B, N, 64, dtype=u8),
          qI_scale=z(B, Tq, HI, 4, dtype=u8), kI_scale=z(B, N, 3, dtype=u8)), "kI_scale has"),
    (dict(dt=L.MXFP4, qI=z(B, Tq, HI, 64, dtype=u8), kI=z(B, N, 64, dtype=u8),
          qI_scale=z(B, Tq, HI, 4, dtype=u8), kI_scale=z(B, N, 4, dtype=u8)), "device memory only"),
])
def test_index_topk_checks(over, fragment):
    _raises(lambda: call_index(**over), fragment)


def test_compress_checks():
    T, Dc, m = 16, 64, 4
    f = lambda **o: L.csa_compress(L.BF16, o.get("dt_out", L.BF16), z(B, T, Dc), z(B, T, dtype=f32), m,
                                   ca=o.get("ca", z(B, T, Dc)), za=z(B, T, dtype=f32), out=o.get("out"),
                                   out_scale=o.get("out_scale"), out_rows=o.get("out_rows", 0),
                                   flags=o.get("flags", 0), norm_w=o.get("norm_w"))
    _raises(lambda: f(out=z(B, T // m, Dc)), "device memory only")
    _raises(lambda: f(out=z(B, T // m - 1, Dc)), "out leaves")
    _raises(lambda: f(out=z(B, 10, Dc), out_rows=17), "out leaves")
    # a view into a larger cache (out_rows) passes the extent check ...
    cache = z(B, 10, Dc)
    _raises(lambda: f(out=cache[:, 6:], out_rows=10), "device memory only")
    # ... unless the last sequence's rows run past the cache's end
    _raises(lambda: f(out=cache[:, 7:], out_rows=10), "out leaves")
    _raises(lambda: f(ca=z(B, T, Dc + 1), out=z(B, T // m, Dc)), "ca has shape")
    _raises(lambda: f(out=z(B, T // m, Dc), flags=L.NORM), "norm_w is required")
    _raises(lambda: f(dt_out=L.MXFP4, out=z(B, T // m, Dc // 2, dtype=u8)), "out_scale is required")
    _raises(lambda: f(dt_out=L.MXFP4, out=z(B, T // m, Dc // 2, dtype=u8), out_scale=z(B, T // m, 1, dtype=u8)),
            "out_scale leaves")


def test_quantize_rows_checks():
    _raises(lambda: L.lca_quantize_rows(L.KV_MIXED, z(5, 512, dtype=f32), z(5, 575, dtype=u8), z(5, dtype=f32)),
            "out holds")
    _raises(lambda: L.lca_quantize_rows(L.KV_MIXED, z(5, 512, dtype=f32), z(5, 576, dtype=u8), z(4, dtype=f32)),
            "out_scale has")
    _raises(lambda: L.lca_quantize_rows(L.MXFP4, z(5, 128), z(5, 64, dtype=u8), z(5, 4, dtype=u8)),
            "src has dtype")
    _raises(lambda: L.lca_quantize_rows(L.MXFP4, z(5, 128, dtype=f32), z(5, 64, dtype=u8), z(5, 4, dtype=u8)),
            "device memory only")


def test_decode_state_checks():
    Dd, m = 64, 4
    st = z(L.csa_compress_state_bytes(L.BF16, B, Dd, m, True), dtype=u8)
    pos = z(B, dtype=torch.int64)
    f = lambda **o: L.csa_compress_append(L.BF16, L.BF16, z(B, Dd), z(B, dtype=f32), m, o.get("pos", pos),
                                          o.get("st", st), z(B, 10, Dd), pos_max=39, ca=z(B, Dd),
                                          za=z(B, dtype=f32))
    _raises(lambda: f(), "device memory only")
    _raises(lambda: f(st=st[:-16]), "state holds")
    _raises(lambda: f(pos=z(B, dtype=i32)), "q_pos has dtype")
    _raises(lambda: L.lca_window_append(L.BF16, L.BF16, z(B, Dd), pos, z(B, 7, Dd + 2), pos_max=9),
            "win rows hold")
    _raises(lambda: L.lca_window_append(L.BF16, L.KV_MIXED, z(B, Dd), pos, z(B, 7, Dd + 64, dtype=u8), pos_max=9),
            "win_scale is required")
    _raises(lambda: L.append_job_window(L.BF16, L.BF16, z(B, Dd), z(B, 7, Dd)), "device memory only")
    j = L.AppendJob()
    j.batch = B                     # as append_job_* records it for a batch of B
    _raises(lambda: L.lca_decode_append([j], z(B + 1, dtype=torch.int64), pos_max=9), "job 0 was made for 2")
    _raises(lambda: L.lca_decode_append([j], pos, pos_max=9), "device memory only")


def test_backward_and_outproj_checks():
    f = lambda **o: L.attend_backward("csa", z(B, Tq, 64, D), z(B, N, D), z(B, W - 1 + Tq, D), z(64, dtype=f32),
                                      z(B, Tq, 64, D), o.get("lse", z(B, Tq, 64, dtype=f32)),
                                      o.get("dout", z(B, Tq, 64, D)), idx=o.get("idx", z(B, Tq, k, dtype=i32)),
                                      m=4, W=W, q_pos0=300, scale=0.04)
    _raises(lambda: f(), "device memory only")
    _raises(lambda: f(lse=z(B, Tq, 63, dtype=f32)), "lse_out has")
    _raises(lambda: f(dout=z(B, Tq, 64, D, dtype=f32)), "dout has dtype")
    _raises(lambda: f(idx=None), "idx is required")
    T, nh, c, g, dg, dm = 4, 64, 512, 8, 1024, 4096
    _raises(lambda: L.lca_grouped_out_proj(z(T, nh, c), z(g, dg, nh // g * c), z(dm, g * dg), z(T, dm)),
            "device memory only")
    _raises(lambda: L.lca_grouped_out_proj(z(T, nh, c), z(g, dg, 100), z(dm, g * dg), z(T, dm)), "w_g has shape")
    _raises(lambda: L.lca_grouped_out_proj(z(T, nh, c), z(g, dg, nh // g * c), z(dm, g * dg), z(T, dm - 1)),
            "out has")
