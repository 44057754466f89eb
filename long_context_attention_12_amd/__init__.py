"""MI355X (gfx950) hybrid compressed attention: CSA / HCA hot path.

Thin ctypes binding over ``liblca.so`` (C ABI declared in ``include/lca.h``).
Each function here only marshals arguments: tensor pointers, shapes read from
the tensors, the current HIP stream, and a workspace tensor when the caller
gives none. Every step of the computation runs in the library's HIP kernels;
there is no fallback. If the library is missing, the first call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "F32", "BF16", "KV_MIXED", "MXFP4",
    "NORM", "ROPE", "INV_ROPE", "SCORE_BF16",
    "LcaError", "lib", "lib_path",
    "csa_compress", "lca_quantize_rows",
    "csa_index_topk", "csa_index_topk_workspace",
    "csa_attend", "csa_attend_workspace",
    "hca_attend", "hca_attend_workspace",
    "lca_version", "lca_profile_enable", "lca_profile_collect",
]

F32, BF16, KV_MIXED, MXFP4 = 0, 1, 2, 3
NORM, ROPE, INV_ROPE, SCORE_BF16, WIN_RING, SPLITS_ONE_WG, SPLITS_MANY_WG = 1, 2, 4, 8, 16, 32, 64

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "liblca.so")
_LIB = None


class LcaError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"lca status {status}: {text}")
        self.status = status


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class AppendJob(ctypes.Structure):
    """lca_append_job of include/lca.h (same field order and types)."""
    _fields_ = [("kind", ctypes.c_int), ("dt_in", ctypes.c_int), ("dt_out", ctypes.c_int), ("D", ctypes.c_int),
                ("m", ctypes.c_int), ("overlap", ctypes.c_int), ("flags", ctypes.c_uint32),
                ("rope_dims", ctypes.c_int), ("eps", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("ca", ctypes.c_void_p), ("za", ctypes.c_void_p), ("cb", ctypes.c_void_p),
                ("zb", ctypes.c_void_p), ("norm_w", ctypes.c_void_p), ("state", ctypes.c_void_p),
                ("state_bytes", ctypes.c_size_t), ("out", ctypes.c_void_p), ("out_scale", ctypes.c_void_p),
                ("out_rows", ctypes.c_int64)]


APPEND_COMPRESS, APPEND_WINDOW, MAX_APPEND_JOBS = 0, 1, 4


def _declare(L):
    vp, i32, i64, u32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float
    sz = ctypes.c_size_t
    L.csa_compress.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp,
                               u32, vp, f32, f32, i32, vp, vp, i64]
    L.csa_compress.restype = i32
    L.lca_quantize_rows.argtypes = [vp, i32, i64, i32, i32, vp, vp, vp]
    L.lca_quantize_rows.restype = i32
    L.csa_index_topk_workspace.argtypes = [i32, i32, i32, i32, i32, i64, i32, i32, i64, u32]
    L.csa_index_topk_workspace.restype = sz
    L.csa_index_topk.argtypes = [vp, i32, i32, i32, i32, i32, i64, i32, i32, i64, vp, vp, vp, vp, vp,
                                 u32, vp, vp, vp, sz]
    L.csa_index_topk.restype = i32
    L.csa_attend_workspace.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32, i32, i32, i64]
    L.csa_attend_workspace.restype = sz
    L.csa_attend.argtypes = [vp, i32, i32, i32, i32, i32, i32, i64, i32, i32, i32, i64, vp, vp, vp, vp,
                             vp, vp, vp, f32, u32, f32, i32, vp, vp, vp, sz]
    L.csa_attend.restype = i32
    L.hca_attend_workspace.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32, i32, i64]
    L.hca_attend_workspace.restype = sz
    L.hca_attend.argtypes = [vp, i32, i32, i32, i32, i32, i32, i64, i32, i32, i64, vp, vp, vp, vp, vp,
                             vp, f32, u32, f32, i32, vp, vp, vp, sz]
    L.hca_attend.restype = i32
    L.csa_index_topk_ragged.argtypes = [vp, i32, i32, i32, i32, i32, i64, i32, i32, i64, vp, vp, vp, vp,
                                        vp, vp, u32, vp, vp, vp, sz]
    L.csa_index_topk_ragged.restype = i32
    L.csa_attend_ragged.argtypes = [vp, i32, i32, i32, i32, i32, i32, i64, i32, i32, i32, i64, vp, vp, vp,
                                    vp, vp, vp, vp, vp, f32, u32, f32, i32, vp, vp, vp, sz]
    L.csa_attend_ragged.restype = i32
    L.hca_attend_ragged.argtypes = [vp, i32, i32, i32, i32, i32, i32, i64, i32, i32, i64, vp, vp, vp, vp,
                                    vp, vp, vp, f32, u32, f32, i32, vp, vp, vp, sz]
    L.hca_attend_ragged.restype = i32
    L.csa_compress_state_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.csa_compress_state_bytes.restype = sz
    L.csa_compress_append.argtypes = [vp, i32, i32, i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, sz,
                                      u32, vp, f32, f32, i32, vp, vp, i64]
    L.csa_compress_append.restype = i32
    L.lca_window_append.argtypes = [vp, i32, i32, i32, i32, i32, i32, i64, vp, vp, vp, vp]
    L.lca_window_append.restype = i32
    L.lca_decode_append.argtypes = [vp, i32, i64, vp, ctypes.POINTER(AppendJob), i32]
    L.lca_decode_append.restype = i32
    L.lca_grouped_out_proj.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
    L.lca_grouped_out_proj.restype = i32
    L.csa_attend_backward_workspace.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32, i32, i32, i64]
    L.csa_attend_backward_workspace.restype = sz
    L.hca_attend_backward_workspace.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32, i32, i64]
    L.hca_attend_backward_workspace.restype = sz
    L.csa_attend_backward.argtypes = [vp, i32, i32, i32, i32, i32, i32, i64, i32, i32, i32, i64, vp, vp, vp, vp,
                                      vp, f32, u32, f32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz]
    L.csa_attend_backward.restype = i32
    L.hca_attend_backward.argtypes = [vp, i32, i32, i32, i32, i32, i32, i64, i32, i32, i64, vp, vp, vp, vp,
                                      f32, u32, f32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz]
    L.hca_attend_backward.restype = i32
    L.lca_status_str.argtypes = [i32]
    L.lca_status_str.restype = ctypes.c_char_p
    L.lca_last_error.argtypes = []
    L.lca_last_error.restype = ctypes.c_char_p
    L.lca_version.argtypes = []
    L.lca_version.restype = i32
    L.lca_profile_enable.argtypes = [i32]
    L.lca_profile_enable.restype = i32
    L.lca_profile_collect.argtypes = [ctypes.POINTER(KernelStat), i32]
    L.lca_profile_collect.restype = i32


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is missing: build it with "
                               "`python -m long_context_attention_12_amd.build`")
        L = ctypes.CDLL(lib_path)
        _declare(L)
        _LIB = L
    return _LIB


def _check(status: int):
    if status != 0:
        raise LcaError(status, lib().lca_last_error().decode())


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _workspace(nbytes: int, like: torch.Tensor):
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=like.device)


# ---------------------------------------------------------------------------

def csa_compress(dt_in, dt_out, cb, zb, m, *, ca=None, za=None, prev_ca=None, prev_za=None,
                 overlap=True, pos0=0, flags=0, norm_w=None, eps=1e-6, rope_base=10000.0,
                 rope_dims=0, out=None, out_scale=None, out_rows=0, stream=None):
    """Token compressor; see csa_compress in include/lca.h. cb: [B, T, D]."""
    B, T, D = cb.shape
    st = lib().csa_compress(_stream(stream), dt_in, dt_out, B, T, D, m, 1 if overlap else 0, pos0,
                            _p(ca), _p(za), _p(cb), _p(zb), _p(prev_ca), _p(prev_za), flags,
                            _p(norm_w), eps, rope_base, rope_dims, _p(out), _p(out_scale), out_rows)
    _check(st)


def lca_quantize_rows(dt_out, src, out, out_scale, *, rope_dims=64, stream=None):
    """Quantise float32 rows [n, D] to KV_MIXED or MXFP4; see include/lca.h."""
    D = src.shape[-1]
    n = src.numel() // D
    _check(lib().lca_quantize_rows(_stream(stream), dt_out, n, D, rope_dims, _p(src), _p(out),
                                   _p(out_scale)))


def csa_compress_state_bytes(dt_in, B, D, m, overlap=True):
    return int(lib().csa_compress_state_bytes(dt_in, B, D, m, 1 if overlap else 0))


def csa_compress_append(dt_in, dt_out, cb, zb, m, pos, state, out, *, pos_max, ca=None, za=None,
                        overlap=True, flags=0, norm_w=None, eps=1e-6, rope_base=10000.0, rope_dims=0,
                        out_scale=None, out_rows=None, stream=None):
    """Append one token per sequence (cb [B, D], zb [B]) at positions pos (int64
    device tensor [B]); see csa_compress_append in include/lca.h. out holds
    out_rows entries per sequence (default: out.shape[1])."""
    B, D = cb.shape
    out_rows = out.shape[1] if out_rows is None else out_rows
    _check(lib().csa_compress_append(_stream(stream), dt_in, dt_out, B, D, m, 1 if overlap else 0, pos_max,
                                     _q_pos(pos, B), _p(ca), _p(za), _p(cb), _p(zb), _p(state),
                                     state.numel() * state.element_size(), flags, _p(norm_w), eps,
                                     rope_base, rope_dims, _p(out), _p(out_scale), out_rows))


def lca_window_append(dt_in, dt_out, src, pos, win, *, pos_max, win_scale=None, rope_dims=64, stream=None):
    """Store each sequence's token row src [B, D] into ring row pos[b] mod
    win.shape[1] of win; see lca_window_append in include/lca.h."""
    B, D = src.shape
    _check(lib().lca_window_append(_stream(stream), dt_in, dt_out, B, D, rope_dims, win.shape[1], pos_max,
                                   _q_pos(pos, B), _p(src), _p(win), _p(win_scale)))


def append_job_compress(dt_in, dt_out, cb, zb, m, state, out, *, ca=None, za=None, overlap=True, flags=0,
                        norm_w=None, eps=1e-6, rope_base=10000.0, rope_dims=0, out_scale=None, out_rows=None):
    """A compressor job for lca_decode_append (the tensors must outlive the call)."""
    return AppendJob(APPEND_COMPRESS, dt_in, dt_out, cb.shape[1], m, 1 if overlap else 0, flags, rope_dims, eps,
                     rope_base, _p(ca), _p(za), _p(cb), _p(zb), _p(norm_w), _p(state),
                     state.numel() * state.element_size(), _p(out), _p(out_scale),
                     out.shape[1] if out_rows is None else out_rows)


def append_job_window(dt_in, dt_out, src, win, *, win_scale=None, rope_dims=64):
    """A window-ring job for lca_decode_append: src [B, D] into ring win [B, rows, ...]."""
    return AppendJob(APPEND_WINDOW, dt_in, dt_out, src.shape[1], 0, 0, 0, rope_dims, 0.0, 0.0, None, None,
                     _p(src), None, None, None, 0, _p(win), _p(win_scale), win.shape[1])


def lca_decode_append(jobs, pos, *, pos_max, stream=None):
    """Run every append job of a decode step in one launch; see include/lca.h."""
    arr = (AppendJob * len(jobs))(*jobs)
    B = pos.numel()
    _check(lib().lca_decode_append(_stream(stream), B, pos_max, _q_pos(pos, B), arr, len(jobs)))


def csa_index_topk_workspace(dt, B, Tq, H_I, d_I, N_cap, m, k, q_pos0, flags=0):
    return int(lib().csa_index_topk_workspace(dt, B, Tq, H_I, d_I, N_cap, m, k, q_pos0, flags))


def _q_pos(q_pos, B):
    if q_pos.dtype != torch.int64 or q_pos.numel() != B or not q_pos.is_contiguous():
        raise ValueError(f"q_pos must be a contiguous int64 tensor of {B} positions")
    return _p(q_pos)


def csa_index_topk(dt, qI, w, kI, idx_out, *, m, k, q_pos0, d_I=None, qI_scale=None, kI_scale=None,
                   flags=0, score_out=None, ws=None, stream=None, q_pos=None):
    """Indexer scores + top-k. qI [B, Tq, H_I, d_I(/2)], kI [B, N_cap, d_I(/2)].

    q_pos: optional int64 device tensor [B] of per-sequence positions (a ragged
    batch, csa_index_topk_ragged); q_pos0 is then their bound."""
    B, Tq, H_I = qI.shape[0], qI.shape[1], qI.shape[2]
    if d_I is None:
        d_I = qI.shape[3] * (2 if dt == MXFP4 else 1)
    N_cap = kI.shape[1]
    need = csa_index_topk_workspace(dt, B, Tq, H_I, d_I, N_cap, m, k, q_pos0, flags)
    if ws is None:
        ws = _workspace(need, kI)
    if q_pos is not None:
        _check(lib().csa_index_topk_ragged(_stream(stream), dt, B, Tq, H_I, d_I, N_cap, m, k, q_pos0,
                                           _q_pos(q_pos, B), _p(qI), _p(qI_scale), _p(w), _p(kI),
                                           _p(kI_scale), flags, _p(idx_out), _p(score_out), _p(ws),
                                           ws.numel() * ws.element_size()))
        return
    _check(lib().csa_index_topk(_stream(stream), dt, B, Tq, H_I, d_I, N_cap, m, k, q_pos0, _p(qI),
                                _p(qI_scale), _p(w), _p(kI), _p(kI_scale), flags, _p(idx_out),
                                _p(score_out), _p(ws), ws.numel() * ws.element_size()))


def csa_attend_workspace(dt_q, dt_kv, B, Tq, H, D, N_cap, m, k, W, q_pos0):
    return int(lib().csa_attend_workspace(dt_q, dt_kv, B, Tq, H, D, N_cap, m, k, W, q_pos0))


def hca_attend_workspace(dt_q, dt_kv, B, Tq, H, D, N_cap, m, W, q_pos0):
    return int(lib().hca_attend_workspace(dt_q, dt_kv, B, Tq, H, D, N_cap, m, W, q_pos0))


def csa_attend(dt_q, dt_kv, q, kv, idx, win, sink, out, *, m, W, q_pos0, scale, N_cap=None,
               kv_scale=None, win_scale=None, flags=0, rope_base=10000.0, rope_dims=0, lse_out=None,
               ws=None, stream=None, q_pos=None):
    """CSA core attention; q [B, Tq, H, D], kv [B, N_cap, ...], idx [B, Tq, k].

    q_pos: optional int64 device tensor [B] (csa_attend_ragged); q_pos0 is its bound."""
    B, Tq, H, D = q.shape
    k = idx.shape[2]
    N_cap = kv.shape[1] if N_cap is None else N_cap
    need = csa_attend_workspace(dt_q, dt_kv, B, Tq, H, D, N_cap, m, k, W, q_pos0)
    if ws is None:
        ws = _workspace(need, q)
    if q_pos is not None:
        _check(lib().csa_attend_ragged(_stream(stream), dt_q, dt_kv, B, Tq, H, D, N_cap, m, k, W, q_pos0,
                                       _q_pos(q_pos, B), _p(q), _p(kv), _p(kv_scale), _p(idx), _p(win),
                                       _p(win_scale), _p(sink), scale, flags, rope_base, rope_dims,
                                       _p(out), _p(lse_out), _p(ws), ws.numel() * ws.element_size()))
        return
    _check(lib().csa_attend(_stream(stream), dt_q, dt_kv, B, Tq, H, D, N_cap, m, k, W, q_pos0,
                            _p(q), _p(kv), _p(kv_scale), _p(idx), _p(win), _p(win_scale), _p(sink),
                            scale, flags, rope_base, rope_dims, _p(out), _p(lse_out), _p(ws),
                            ws.numel() * ws.element_size()))


def hca_attend(dt_q, dt_kv, q, kv, win, sink, out, *, m, W, q_pos0, scale, N_cap=None, kv_scale=None,
               win_scale=None, flags=0, rope_base=10000.0, rope_dims=0, lse_out=None, ws=None,
               stream=None, q_pos=None):
    """HCA dense attention over every visible entry; arguments as csa_attend without idx."""
    B, Tq, H, D = q.shape
    N_cap = kv.shape[1] if N_cap is None else N_cap
    need = hca_attend_workspace(dt_q, dt_kv, B, Tq, H, D, N_cap, m, W, q_pos0)
    if ws is None:
        ws = _workspace(need, q)
    if q_pos is not None:
        _check(lib().hca_attend_ragged(_stream(stream), dt_q, dt_kv, B, Tq, H, D, N_cap, m, W, q_pos0,
                                       _q_pos(q_pos, B), _p(q), _p(kv), _p(kv_scale), _p(win),
                                       _p(win_scale), _p(sink), scale, flags, rope_base, rope_dims,
                                       _p(out), _p(lse_out), _p(ws), ws.numel() * ws.element_size()))
        return
    _check(lib().hca_attend(_stream(stream), dt_q, dt_kv, B, Tq, H, D, N_cap, m, W, q_pos0, _p(q),
                            _p(kv), _p(kv_scale), _p(win), _p(win_scale), _p(sink), scale, flags,
                            rope_base, rope_dims, _p(out), _p(lse_out), _p(ws),
                            ws.numel() * ws.element_size()))


def attend_backward(kind, q, kv, win, sink, out, lse, dout, *, m, W, q_pos0, scale, idx=None, N_cap=None,
                    flags=0, rope_base=10000.0, rope_dims=0, ws=None, stream=None):
    """Gradients of csa_attend (kind "csa", idx given) or hca_attend: returns
    (dq [B,Tq,H,D], dkv [B,N_cap,D], dwin [B,W-1+Tq,D], dsink [H]), all fp32;
    see csa_attend_backward in include/lca.h."""
    B, Tq, H, D = q.shape
    N_cap = kv.shape[1] if N_cap is None else N_cap
    dev = q.device
    dq = torch.empty((B, Tq, H, D), dtype=torch.float32, device=dev)
    dkv = torch.empty((B, N_cap, D), dtype=torch.float32, device=dev)
    dwin = torch.empty((B, W - 1 + Tq, D), dtype=torch.float32, device=dev)
    dsink = torch.empty((H,), dtype=torch.float32, device=dev)
    if kind == "csa":
        k = idx.shape[2]
        need = int(lib().csa_attend_backward_workspace(BF16, BF16, B, Tq, H, D, N_cap, m, k, W, q_pos0))
        if ws is None:
            ws = _workspace(need, q)
        _check(lib().csa_attend_backward(_stream(stream), BF16, BF16, B, Tq, H, D, N_cap, m, k, W, q_pos0, _p(q),
                                         _p(kv), _p(idx), _p(win), _p(sink), scale, flags, rope_base, rope_dims,
                                         _p(out), _p(lse), _p(dout), _p(dq), _p(dkv), _p(dwin), _p(dsink), _p(ws),
                                         ws.numel() * ws.element_size()))
    else:
        need = int(lib().hca_attend_backward_workspace(BF16, BF16, B, Tq, H, D, N_cap, m, W, q_pos0))
        if ws is None:
            ws = _workspace(need, q)
        _check(lib().hca_attend_backward(_stream(stream), BF16, BF16, B, Tq, H, D, N_cap, m, W, q_pos0, _p(q),
                                         _p(kv), _p(win), _p(sink), scale, flags, rope_base, rope_dims, _p(out),
                                         _p(lse), _p(dout), _p(dq), _p(dkv), _p(dwin), _p(dsink), _p(ws),
                                         ws.numel() * ws.element_size()))
    return dq, dkv, dwin, dsink


def lca_grouped_out_proj(o, w_g, w_o, out, *, mid=None, stream=None):
    """Grouped output projection: o [T, n_h, c], w_g [g, d_g, (n_h/g)*c],
    w_o [d_model, g*d_g] (bf16) -> out [T, d_model]; see include/lca.h.
    mid [T, g*d_g] is allocated when not given; returns it."""
    T, n_h, c = o.shape
    g, d_g, _ = w_g.shape
    d_model = w_o.shape[0]
    if mid is None:
        mid = torch.empty((T, g * d_g), dtype=torch.bfloat16, device=o.device)
    _check(lib().lca_grouped_out_proj(_stream(stream), T, n_h, c, g, d_g, d_model, _p(o), _p(w_g), _p(w_o),
                                      _p(mid), _p(out)))
    return mid


def lca_version():
    return int(lib().lca_version())


def lca_profile_enable(on: bool):
    _check(lib().lca_profile_enable(1 if on else 0))


def lca_profile_collect(max_entries: int = 64):
    """Per-kernel {name: (launches, total_ms)} of the launches since the last collect."""
    arr = (KernelStat * max_entries)()
    n = lib().lca_profile_collect(arr, max_entries)
    if n < 0:
        _check(n)
    return {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms)) for i in range(n)}
