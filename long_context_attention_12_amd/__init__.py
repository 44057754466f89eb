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
    "csa_compress", "csa_compress_backward", "lca_quantize_rows",
    "csa_index_topk", "csa_index_topk_workspace",
    "csa_attend", "csa_attend_workspace", "csa_attend_noalloc",
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
    L.csa_compress_backward_workspace.argtypes = [i32, i32, i32, i32, u32]
    L.csa_compress_backward_workspace.restype = sz
    L.csa_compress_backward.argtypes = [vp, i32, i32, i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp,
                                        u32, vp, f32, f32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz]
    L.csa_compress_backward.restype = i32
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
    L.csa_attend_noalloc.argtypes = [vp, i32, i32, i32, i32, i32, i32, i64, i32, i32, i32, i64, vp, vp, vp, vp,
                                     vp, vp, vp, f32, u32, f32, i32, vp, vp]
    L.csa_attend_noalloc.restype = i32
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
# Argument checks. The C library trusts that every pointer spans the sizes it
# is given; a tensor smaller than the call's dimensions would be read or
# written out of bounds on the device. Each wrapper therefore checks dtype,
# contiguity, shape and device of every tensor before it passes a pointer, and
# raises ValueError (TypeError for a non-tensor) on a mismatch.
# ---------------------------------------------------------------------------

_U8 = (torch.uint8, torch.int8)
_ELEM = {F32: (torch.float32,), BF16: (torch.bfloat16,), KV_MIXED: _U8, MXFP4: _U8}
_F32 = (torch.float32,)
_I32 = (torch.int32,)


def _row_bytes(dt, D, rope_dims):
    """Bytes of one stored row of D channels in element format dt."""
    if dt == F32:
        return 4 * D
    if dt == BF16:
        return 2 * D
    if dt == KV_MIXED:
        return D + rope_dims            # (D - R) e4m3 bytes + R bf16 values
    if dt == MXFP4:
        return D // 2                   # two e2m1 codes per byte
    raise ValueError(f"unknown element format {dt}")


def _nbytes(t):
    return t.numel() * t.element_size()


class _Args:
    """Collects the tensors of one call, checking each as it is added."""

    def __init__(self, fn):
        self.fn = fn
        self.seen = []

    def _fail(self, msg):
        raise ValueError(f"{self.fn}: {msg}")

    def t(self, x, name, *, dtypes=None, shape=None, numel=None, min_numel=None, optional=False):
        if x is None:
            if optional:
                return None
            self._fail(f"{name} is required")
        if not isinstance(x, torch.Tensor):
            raise TypeError(f"{self.fn}: {name} must be a torch.Tensor, not {type(x).__name__}")
        if dtypes is not None and x.dtype not in dtypes:
            self._fail(f"{name} has dtype {x.dtype}; the call needs {' or '.join(map(str, dtypes))}")
        if not x.is_contiguous():
            self._fail(f"{name} must be contiguous")
        if shape is not None and tuple(x.shape) != tuple(shape):
            self._fail(f"{name} has shape {tuple(x.shape)}; the call needs {tuple(shape)}")
        if numel is not None and x.numel() != numel:
            self._fail(f"{name} has {x.numel()} elements; the call needs {numel}")
        if min_numel is not None and x.numel() < min_numel:
            self._fail(f"{name} has {x.numel()} elements; the call needs at least {min_numel}")
        self.seen.append((name, x))
        return x

    def rows(self, x, name, B, row_bytes, dtypes, *, rows=None, optional=False):
        """x holds B sequences of equally many rows of row_bytes bytes each
        ([B, rows, ...] or [B, rows * row]); returns the rows per sequence,
        which must equal ``rows`` when that is given."""
        if self.t(x, name, dtypes=dtypes, optional=optional) is None:
            return None
        if x.dim() < 2 or x.shape[0] != B:
            self._fail(f"{name} has shape {tuple(x.shape)}; the call needs {B} sequences in dim 0")
        if x.dim() >= 3:
            per_row = x.element_size()
            for n in x.shape[2:]:
                per_row *= n
            if per_row != row_bytes:
                self._fail(f"{name} rows hold {per_row} bytes; the call needs {row_bytes}")
            n_rows = x.shape[1]
        else:
            if _nbytes(x) % (B * row_bytes):
                self._fail(f"{name} holds {_nbytes(x)} bytes: not {B} sequences of whole {row_bytes}-byte rows")
            n_rows = _nbytes(x) // (B * row_bytes)
        if rows is not None and n_rows != rows:
            self._fail(f"{name} holds {n_rows} rows per sequence; the call needs {rows}")
        return n_rows

    def min_bytes(self, x, name, nbytes, dtypes=None, *, optional=False):
        if self.t(x, name, dtypes=dtypes, optional=optional) is None:
            return None
        if _nbytes(x) < nbytes:
            self._fail(f"{name} holds {_nbytes(x)} bytes; the call writes or reads {nbytes}")
        return x

    def span(self, x, name, nbytes, dtypes=None, *, optional=False):
        """An output the call writes at strided rows inside a larger buffer
        (out_rows): x may be a view, but the bytes from its first element to
        the end of its storage must cover what the call writes."""
        if x is None:
            if optional:
                return None
            self._fail(f"{name} is required")
        if not isinstance(x, torch.Tensor):
            raise TypeError(f"{self.fn}: {name} must be a torch.Tensor, not {type(x).__name__}")
        if dtypes is not None and x.dtype not in dtypes:
            self._fail(f"{name} has dtype {x.dtype}; the call needs {' or '.join(map(str, dtypes))}")
        if x.dim() and x.stride(-1) != 1:
            self._fail(f"{name} must have unit stride in its last dimension")
        room = x.untyped_storage().nbytes() - x.storage_offset() * x.element_size()
        if room < nbytes:
            self._fail(f"{name} leaves {room} bytes from its first element; the call writes {nbytes}")
        self.seen.append((name, x))
        return x

    def ptr(self, x):
        return None if x is None else x.data_ptr()

    def done(self):
        """Every tensor of the call must sit on one GPU."""
        dev = None
        for name, x in self.seen:
            if x.device.type != "cuda":
                self._fail(f"{name} is on {x.device}; the library reads and writes device memory only")
            if dev is None:
                dev = x.device
            elif x.device != dev:
                self._fail(f"{name} is on {x.device}, other tensors on {dev}")


def _ws_arg(a, ws, need, like):
    if ws is None:
        ws = _workspace(need, like)
    a.t(ws, "ws")
    return ws, _nbytes(ws)


# ---------------------------------------------------------------------------

def csa_compress(dt_in, dt_out, cb, zb, m, *, ca=None, za=None, prev_ca=None, prev_za=None,
                 overlap=True, pos0=0, flags=0, norm_w=None, eps=1e-6, rope_base=10000.0,
                 rope_dims=0, out=None, out_scale=None, out_rows=0, stream=None):
    """Token compressor; see csa_compress in include/lca.h. cb: [B, T, D]."""
    a = _Args("csa_compress")
    a.t(cb, "cb", dtypes=_ELEM.get(dt_in))
    if cb.dim() != 3:
        a._fail(f"cb must be [B, T, D], not {tuple(cb.shape)}")
    B, T, D = cb.shape
    if m < 1:
        a._fail("m must be >= 1")
    a.t(zb, "zb", dtypes=_F32, numel=B * T)
    a.t(ca, "ca", dtypes=_ELEM.get(dt_in), shape=cb.shape, optional=not overlap)
    a.t(za, "za", dtypes=_F32, numel=B * T, optional=not overlap)
    a.t(prev_ca, "prev_ca", dtypes=_ELEM.get(dt_in), numel=B * m * D, optional=True)
    a.t(prev_za, "prev_za", dtypes=_F32, numel=B * m, optional=True)
    a.t(norm_w, "norm_w", dtypes=_F32, numel=D, optional=not (flags & NORM))
    rows = out_rows if out_rows else T // m
    last = (B - 1) * rows + T // m          # rows written from out's first row on
    a.span(out, "out", last * _row_bytes(dt_out, D, rope_dims), _ELEM.get(dt_out))
    if dt_out == KV_MIXED:
        a.span(out_scale, "out_scale", last * 4, _F32)
    elif dt_out == MXFP4:
        a.span(out_scale, "out_scale", last * (D // 32), _U8)
    a.done()
    st = lib().csa_compress(_stream(stream), dt_in, dt_out, B, T, D, m, 1 if overlap else 0, pos0,
                            _p(ca), _p(za), _p(cb), _p(zb), _p(prev_ca), _p(prev_za), flags,
                            _p(norm_w), eps, rope_base, rope_dims, _p(out), _p(out_scale), out_rows)
    _check(st)


def csa_compress_backward(dt_in, cb, zb, m, dout, dcb, dzb, *, ca=None, za=None, prev_ca=None, prev_za=None,
                          overlap=True, pos0=0, flags=0, norm_w=None, eps=1e-6, rope_base=10000.0, rope_dims=0,
                          dca=None, dza=None, dprev_ca=None, dprev_za=None, dnorm_w=None, ws=None, stream=None):
    """Gradients of the compressor's entries with respect to its inputs; see
    csa_compress_backward in include/lca.h. cb: [B, T, D]; dout: [B, T/m, D]."""
    a = _Args("csa_compress_backward")
    a.t(cb, "cb", dtypes=_ELEM.get(dt_in))
    if cb.dim() != 3:
        a._fail(f"cb must be [B, T, D], not {tuple(cb.shape)}")
    B, T, D = cb.shape
    if m < 1:
        a._fail("m must be >= 1")
    a.t(zb, "zb", dtypes=_F32, numel=B * T)
    a.t(ca, "ca", dtypes=_ELEM.get(dt_in), shape=cb.shape, optional=not overlap)
    a.t(za, "za", dtypes=_F32, numel=B * T, optional=not overlap)
    a.t(prev_ca, "prev_ca", dtypes=_ELEM.get(dt_in), numel=B * m * D, optional=True)
    a.t(prev_za, "prev_za", dtypes=_F32, numel=B * m, optional=True)
    a.t(norm_w, "norm_w", dtypes=_F32, numel=D, optional=not (flags & NORM))
    a.t(dout, "dout", dtypes=_F32, numel=B * (T // m) * D)
    a.t(dcb, "dcb", dtypes=_F32, numel=B * T * D)
    a.t(dzb, "dzb", dtypes=_F32, numel=B * T)
    a.t(dca, "dca", dtypes=_F32, numel=B * T * D, optional=not overlap)
    a.t(dza, "dza", dtypes=_F32, numel=B * T, optional=not overlap)
    a.t(dprev_ca, "dprev_ca", dtypes=_F32, numel=B * m * D, optional=True)
    a.t(dprev_za, "dprev_za", dtypes=_F32, numel=B * m, optional=True)
    a.t(dnorm_w, "dnorm_w", dtypes=_F32, numel=D, optional=not (flags & NORM))
    need = int(lib().csa_compress_backward_workspace(B, T, D, m, flags))
    if ws is None and (flags & NORM):
        ws = torch.empty(need, dtype=torch.uint8, device=cb.device)
    a.t(ws, "ws", optional=True)
    a.done()
    st = lib().csa_compress_backward(_stream(stream), dt_in, B, T, D, m, 1 if overlap else 0, pos0,
                                     _p(ca), _p(za), _p(cb), _p(zb), _p(prev_ca), _p(prev_za), flags,
                                     _p(norm_w), eps, rope_base, rope_dims, _p(dout), _p(dca), _p(dza),
                                     _p(dcb), _p(dzb), _p(dprev_ca), _p(dprev_za), _p(dnorm_w), _p(ws),
                                     _nbytes(ws) if ws is not None else 0)
    _check(st)


def lca_quantize_rows(dt_out, src, out, out_scale, *, rope_dims=64, stream=None):
    """Quantise float32 rows [n, D] to KV_MIXED or MXFP4; see include/lca.h."""
    a = _Args("lca_quantize_rows")
    a.t(src, "src", dtypes=_F32)
    if src.dim() < 1:
        a._fail("src must hold rows of D channels")
    D = src.shape[-1]
    n = src.numel() // D if D else 0
    a.min_bytes(out, "out", n * _row_bytes(dt_out, D, rope_dims), _U8)
    if dt_out == KV_MIXED:
        a.t(out_scale, "out_scale", dtypes=_F32, min_numel=n)
    else:
        a.min_bytes(out_scale, "out_scale", n * (D // 32), _U8)
    a.done()
    _check(lib().lca_quantize_rows(_stream(stream), dt_out, n, D, rope_dims, _p(src), _p(out),
                                   _p(out_scale)))


def csa_compress_state_bytes(dt_in, B, D, m, overlap=True):
    return int(lib().csa_compress_state_bytes(dt_in, B, D, m, 1 if overlap else 0))


def _check_append_compress(a, dt_in, dt_out, cb, zb, m, state, out, ca, za, overlap, flags, norm_w,
                           rope_dims, out_scale, out_rows):
    a.t(cb, "cb", dtypes=_ELEM.get(dt_in))
    if cb.dim() != 2:
        a._fail(f"cb must be [B, D], not {tuple(cb.shape)}")
    B, D = cb.shape
    a.t(zb, "zb", dtypes=_F32, numel=B)
    a.t(ca, "ca", dtypes=_ELEM.get(dt_in), shape=cb.shape, optional=not overlap)
    a.t(za, "za", dtypes=_F32, numel=B, optional=not overlap)
    a.t(norm_w, "norm_w", dtypes=_F32, numel=D, optional=not (flags & NORM))
    a.min_bytes(state, "state", csa_compress_state_bytes(dt_in, B, D, m, overlap))
    if not isinstance(out, torch.Tensor) or out.dim() < 2 or out.shape[0] != B:
        a._fail(f"out must be a tensor with {B} sequences in dim 0")
    rows = out.shape[1] if out_rows is None else out_rows
    # the kernel writes any row below out_rows of a sequence (entry j of a
    # position up to pos_max); the cache must span all of them
    a.span(out, "out", B * rows * _row_bytes(dt_out, D, rope_dims), _ELEM.get(dt_out))
    if dt_out == KV_MIXED:
        a.span(out_scale, "out_scale", B * rows * 4, _F32)
    elif dt_out == MXFP4:
        a.span(out_scale, "out_scale", B * rows * (D // 32), _U8)
    return B, D, rows


def csa_compress_append(dt_in, dt_out, cb, zb, m, pos, state, out, *, pos_max, ca=None, za=None,
                        overlap=True, flags=0, norm_w=None, eps=1e-6, rope_base=10000.0, rope_dims=0,
                        out_scale=None, out_rows=None, stream=None):
    """Append one token per sequence (cb [B, D], zb [B]) at positions pos (int64
    device tensor [B]); see csa_compress_append in include/lca.h. out holds
    out_rows entries per sequence (default: out.shape[1])."""
    a = _Args("csa_compress_append")
    B, D, out_rows = _check_append_compress(a, dt_in, dt_out, cb, zb, m, state, out, ca, za, overlap, flags,
                                            norm_w, rope_dims, out_scale, out_rows)
    qp = _q_pos(pos, B, a)
    a.done()
    _check(lib().csa_compress_append(_stream(stream), dt_in, dt_out, B, D, m, 1 if overlap else 0, pos_max,
                                     qp, _p(ca), _p(za), _p(cb), _p(zb), _p(state),
                                     _nbytes(state), flags, _p(norm_w), eps,
                                     rope_base, rope_dims, _p(out), _p(out_scale), out_rows))


def _check_window(a, dt_in, dt_out, src, win, win_scale, rope_dims):
    a.t(src, "src", dtypes=_ELEM.get(dt_in))
    if src.dim() != 2:
        a._fail(f"src must be [B, D], not {tuple(src.shape)}")
    B, D = src.shape
    ring = a.rows(win, "win", B, _row_bytes(dt_out, D, rope_dims), _ELEM.get(dt_out))
    a.t(win_scale, "win_scale", dtypes=_F32, numel=B * ring, optional=dt_out != KV_MIXED)
    return B, D, ring


def lca_window_append(dt_in, dt_out, src, pos, win, *, pos_max, win_scale=None, rope_dims=64, stream=None):
    """Store each sequence's token row src [B, D] into ring row pos[b] mod
    win.shape[1] of win; see lca_window_append in include/lca.h."""
    a = _Args("lca_window_append")
    B, D, ring = _check_window(a, dt_in, dt_out, src, win, win_scale, rope_dims)
    qp = _q_pos(pos, B, a)
    a.done()
    _check(lib().lca_window_append(_stream(stream), dt_in, dt_out, B, D, rope_dims, ring, pos_max,
                                   qp, _p(src), _p(win), _p(win_scale)))


def append_job_compress(dt_in, dt_out, cb, zb, m, state, out, *, ca=None, za=None, overlap=True, flags=0,
                        norm_w=None, eps=1e-6, rope_base=10000.0, rope_dims=0, out_scale=None, out_rows=None):
    """A compressor job for lca_decode_append (the tensors must outlive the call)."""
    a = _Args("append_job_compress")
    B, D, rows = _check_append_compress(a, dt_in, dt_out, cb, zb, m, state, out, ca, za, overlap, flags,
                                        norm_w, rope_dims, out_scale, out_rows)
    a.done()
    job = AppendJob(APPEND_COMPRESS, dt_in, dt_out, D, m, 1 if overlap else 0, flags, rope_dims, eps,
                    rope_base, _p(ca), _p(za), _p(cb), _p(zb), _p(norm_w), _p(state),
                    _nbytes(state), _p(out), _p(out_scale), rows)
    job.batch = B
    return job


def append_job_window(dt_in, dt_out, src, win, *, win_scale=None, rope_dims=64):
    """A window-ring job for lca_decode_append: src [B, D] into ring win [B, rows, ...]."""
    a = _Args("append_job_window")
    B, D, ring = _check_window(a, dt_in, dt_out, src, win, win_scale, rope_dims)
    a.done()
    job = AppendJob(APPEND_WINDOW, dt_in, dt_out, D, 0, 0, 0, rope_dims, 0.0, 0.0, None, None,
                    _p(src), None, None, None, 0, _p(win), _p(win_scale), ring)
    job.batch = B
    return job


def lca_decode_append(jobs, pos, *, pos_max, stream=None):
    """Run every append job of a decode step in one launch; see include/lca.h."""
    a = _Args("lca_decode_append")
    B = pos.numel() if isinstance(pos, torch.Tensor) else -1
    for i, j in enumerate(jobs):
        if getattr(j, "batch", None) != B:
            a._fail(f"job {i} was made for {getattr(j, 'batch', '?')} sequences; pos holds {B}")
    qp = _q_pos(pos, B, a)
    a.done()
    arr = (AppendJob * len(jobs))(*jobs)
    _check(lib().lca_decode_append(_stream(stream), B, pos_max, qp, arr, len(jobs)))


def csa_index_topk_workspace(dt, B, Tq, H_I, d_I, N_cap, m, k, q_pos0, flags=0):
    return int(lib().csa_index_topk_workspace(dt, B, Tq, H_I, d_I, N_cap, m, k, q_pos0, flags))


def _q_pos(q_pos, B, a=None):
    a = a or _Args("q_pos")
    a.t(q_pos, "q_pos", dtypes=(torch.int64,), numel=B)
    return q_pos.data_ptr()


def csa_index_topk(dt, qI, w, kI, idx_out, *, m, k, q_pos0, d_I=None, qI_scale=None, kI_scale=None,
                   flags=0, score_out=None, ws=None, stream=None, q_pos=None):
    """Indexer scores + top-k. qI [B, Tq, H_I, d_I(/2)], kI [B, N_cap, d_I(/2)].

    q_pos: optional int64 device tensor [B] of per-sequence positions (a ragged
    batch, csa_index_topk_ragged); q_pos0 is then their bound."""
    a = _Args("csa_index_topk")
    a.t(qI, "qI", dtypes=_ELEM.get(dt))
    if qI.dim() != 4:
        a._fail(f"qI must be [B, Tq, H_I, d_I], not {tuple(qI.shape)}")
    B, Tq, H_I = qI.shape[0], qI.shape[1], qI.shape[2]
    if d_I is None:
        d_I = qI.shape[3] * (2 if dt == MXFP4 else 1)
    rb = _row_bytes(dt, d_I, 0)
    if qI.shape[3] * qI.element_size() != rb:
        a._fail(f"qI rows hold {qI.shape[3] * qI.element_size()} bytes; d_I = {d_I} needs {rb}")
    a.t(w, "w", dtypes=_F32, numel=B * Tq * H_I)
    N_cap = a.rows(kI, "kI", B, rb, _ELEM.get(dt))
    if dt == MXFP4:
        a.t(qI_scale, "qI_scale", dtypes=_U8, numel=B * Tq * H_I * (d_I // 32))
        a.t(kI_scale, "kI_scale", dtypes=_U8, numel=B * N_cap * (d_I // 32))
    a.t(idx_out, "idx_out", dtypes=_I32, numel=B * Tq * k)
    a.t(score_out, "score_out", dtypes=_F32, numel=B * Tq * k, optional=True)
    qp = _q_pos(q_pos, B, a) if q_pos is not None else None
    need = csa_index_topk_workspace(dt, B, Tq, H_I, d_I, N_cap, m, k, q_pos0, flags)
    ws, ws_bytes = _ws_arg(a, ws, need, kI)
    a.done()
    if qp is not None:
        _check(lib().csa_index_topk_ragged(_stream(stream), dt, B, Tq, H_I, d_I, N_cap, m, k, q_pos0,
                                           qp, _p(qI), _p(qI_scale), _p(w), _p(kI),
                                           _p(kI_scale), flags, _p(idx_out), _p(score_out), _p(ws), ws_bytes))
        return
    _check(lib().csa_index_topk(_stream(stream), dt, B, Tq, H_I, d_I, N_cap, m, k, q_pos0, _p(qI),
                                _p(qI_scale), _p(w), _p(kI), _p(kI_scale), flags, _p(idx_out),
                                _p(score_out), _p(ws), ws_bytes))


def csa_attend_workspace(dt_q, dt_kv, B, Tq, H, D, N_cap, m, k, W, q_pos0):
    return int(lib().csa_attend_workspace(dt_q, dt_kv, B, Tq, H, D, N_cap, m, k, W, q_pos0))


def hca_attend_workspace(dt_q, dt_kv, B, Tq, H, D, N_cap, m, W, q_pos0):
    return int(lib().hca_attend_workspace(dt_q, dt_kv, B, Tq, H, D, N_cap, m, W, q_pos0))


def _check_attend(a, dt_q, dt_kv, q, kv, win, sink, out, W, N_cap, kv_scale, win_scale, rope_dims, lse_out):
    """Checks shared by the attention calls; returns (B, Tq, H, D, N_cap)."""
    a.t(q, "q", dtypes=_ELEM.get(dt_q))
    if q.dim() != 4:
        a._fail(f"q must be [B, Tq, H, D], not {tuple(q.shape)}")
    B, Tq, H, D = q.shape
    rb = _row_bytes(dt_kv, D, rope_dims)
    N_cap = a.rows(kv, "kv", B, rb, _ELEM.get(dt_kv), rows=N_cap)
    a.rows(win, "win", B, rb, _ELEM.get(dt_kv), rows=W - 1 + Tq)
    mixed = dt_kv == KV_MIXED
    a.t(kv_scale, "kv_scale", dtypes=_F32, numel=B * N_cap, optional=not mixed)
    a.t(win_scale, "win_scale", dtypes=_F32, numel=B * (W - 1 + Tq), optional=not mixed)
    a.t(sink, "sink", dtypes=_F32, numel=H)
    a.t(out, "out", dtypes=_ELEM.get(dt_q), numel=B * Tq * H * D)
    a.t(lse_out, "lse_out", dtypes=_F32, numel=B * Tq * H, optional=True)
    return B, Tq, H, D, N_cap


def csa_attend(dt_q, dt_kv, q, kv, idx, win, sink, out, *, m, W, q_pos0, scale, N_cap=None,
               kv_scale=None, win_scale=None, flags=0, rope_base=10000.0, rope_dims=0, lse_out=None,
               ws=None, stream=None, q_pos=None):
    """CSA core attention; q [B, Tq, H, D], kv [B, N_cap, ...], idx [B, Tq, k].

    q_pos: optional int64 device tensor [B] (csa_attend_ragged); q_pos0 is its bound."""
    a = _Args("csa_attend")
    B, Tq, H, D, N_cap = _check_attend(a, dt_q, dt_kv, q, kv, win, sink, out, W, N_cap, kv_scale, win_scale,
                                       rope_dims, lse_out)
    a.t(idx, "idx", dtypes=_I32)
    if idx.dim() != 3 or idx.shape[0] != B or idx.shape[1] != Tq:
        a._fail(f"idx must be [{B}, {Tq}, k], not {tuple(idx.shape)}")
    k = idx.shape[2]
    qp = _q_pos(q_pos, B, a) if q_pos is not None else None
    need = csa_attend_workspace(dt_q, dt_kv, B, Tq, H, D, N_cap, m, k, W, q_pos0)
    ws, ws_bytes = _ws_arg(a, ws, need, q)
    a.done()
    if qp is not None:
        _check(lib().csa_attend_ragged(_stream(stream), dt_q, dt_kv, B, Tq, H, D, N_cap, m, k, W, q_pos0,
                                       qp, _p(q), _p(kv), _p(kv_scale), _p(idx), _p(win),
                                       _p(win_scale), _p(sink), scale, flags, rope_base, rope_dims,
                                       _p(out), _p(lse_out), _p(ws), ws_bytes))
        return
    _check(lib().csa_attend(_stream(stream), dt_q, dt_kv, B, Tq, H, D, N_cap, m, k, W, q_pos0,
                            _p(q), _p(kv), _p(kv_scale), _p(idx), _p(win), _p(win_scale), _p(sink),
                            scale, flags, rope_base, rope_dims, _p(out), _p(lse_out), _p(ws), ws_bytes))


NOALLOC_SCRATCH_BYTES = 64 << 20


def csa_attend_noalloc(dt_q, dt_kv, q, kv, idx, win, sink, out, *, m, W, q_pos0, scale, N_cap=None,
                       kv_scale=None, win_scale=None, flags=0, rope_base=10000.0, rope_dims=0, lse_out=None,
                       stream=None):
    """csa_attend with its scratch in the library's static device array (no
    workspace, nothing allocated); see csa_attend_noalloc in include/lca.h."""
    a = _Args("csa_attend_noalloc")
    B, Tq, H, D, N_cap = _check_attend(a, dt_q, dt_kv, q, kv, win, sink, out, W, N_cap, kv_scale, win_scale,
                                       rope_dims, lse_out)
    a.t(idx, "idx", dtypes=_I32)
    if idx.dim() != 3 or idx.shape[0] != B or idx.shape[1] != Tq:
        a._fail(f"idx must be [{B}, {Tq}, k], not {tuple(idx.shape)}")
    a.done()
    _check(lib().csa_attend_noalloc(_stream(stream), dt_q, dt_kv, B, Tq, H, D, N_cap, m, idx.shape[2], W, q_pos0,
                                    _p(q), _p(kv), _p(kv_scale), _p(idx), _p(win), _p(win_scale), _p(sink),
                                    scale, flags, rope_base, rope_dims, _p(out), _p(lse_out)))


def hca_attend(dt_q, dt_kv, q, kv, win, sink, out, *, m, W, q_pos0, scale, N_cap=None, kv_scale=None,
               win_scale=None, flags=0, rope_base=10000.0, rope_dims=0, lse_out=None, ws=None,
               stream=None, q_pos=None):
    """HCA dense attention over every visible entry; arguments as csa_attend without idx."""
    a = _Args("hca_attend")
    B, Tq, H, D, N_cap = _check_attend(a, dt_q, dt_kv, q, kv, win, sink, out, W, N_cap, kv_scale, win_scale,
                                       rope_dims, lse_out)
    qp = _q_pos(q_pos, B, a) if q_pos is not None else None
    need = hca_attend_workspace(dt_q, dt_kv, B, Tq, H, D, N_cap, m, W, q_pos0)
    ws, ws_bytes = _ws_arg(a, ws, need, q)
    a.done()
    if qp is not None:
        _check(lib().hca_attend_ragged(_stream(stream), dt_q, dt_kv, B, Tq, H, D, N_cap, m, W, q_pos0,
                                       qp, _p(q), _p(kv), _p(kv_scale), _p(win),
                                       _p(win_scale), _p(sink), scale, flags, rope_base, rope_dims,
                                       _p(out), _p(lse_out), _p(ws), ws_bytes))
        return
    _check(lib().hca_attend(_stream(stream), dt_q, dt_kv, B, Tq, H, D, N_cap, m, W, q_pos0, _p(q),
                            _p(kv), _p(kv_scale), _p(win), _p(win_scale), _p(sink), scale, flags,
                            rope_base, rope_dims, _p(out), _p(lse_out), _p(ws), ws_bytes))


def attend_backward(kind, q, kv, win, sink, out, lse, dout, *, m, W, q_pos0, scale, idx=None, N_cap=None,
                    flags=0, rope_base=10000.0, rope_dims=0, ws=None, stream=None):
    """Gradients of csa_attend (kind "csa", idx given) or hca_attend: returns
    (dq [B,Tq,H,D], dkv [B,N_cap,D], dwin [B,W-1+Tq,D], dsink [H]), all fp32;
    see csa_attend_backward in include/lca.h."""
    a = _Args(f"{kind}_attend_backward")
    if kind not in ("csa", "hca"):
        a._fail("kind must be 'csa' or 'hca'")
    a.t(lse, "lse", dtypes=_F32)
    B, Tq, H, D, N_cap = _check_attend(a, BF16, BF16, q, kv, win, sink, out, W, N_cap, None, None,
                                       rope_dims, lse)
    a.t(dout, "dout", dtypes=_ELEM[BF16], numel=B * Tq * H * D)
    if kind == "csa":
        a.t(idx, "idx", dtypes=_I32)
        if idx.dim() != 3 or idx.shape[0] != B or idx.shape[1] != Tq:
            a._fail(f"idx must be [{B}, {Tq}, k], not {tuple(idx.shape)}")
    dev = q.device
    a.done()
    dq = torch.empty((B, Tq, H, D), dtype=torch.float32, device=dev)
    dkv = torch.empty((B, N_cap, D), dtype=torch.float32, device=dev)
    dwin = torch.empty((B, W - 1 + Tq, D), dtype=torch.float32, device=dev)
    dsink = torch.empty((H,), dtype=torch.float32, device=dev)
    if kind == "csa":
        k = idx.shape[2]
        need = int(lib().csa_attend_backward_workspace(BF16, BF16, B, Tq, H, D, N_cap, m, k, W, q_pos0))
        ws, ws_bytes = _ws_arg(a, ws, need, q)
        a.done()
        _check(lib().csa_attend_backward(_stream(stream), BF16, BF16, B, Tq, H, D, N_cap, m, k, W, q_pos0, _p(q),
                                         _p(kv), _p(idx), _p(win), _p(sink), scale, flags, rope_base, rope_dims,
                                         _p(out), _p(lse), _p(dout), _p(dq), _p(dkv), _p(dwin), _p(dsink), _p(ws),
                                         ws_bytes))
    else:
        need = int(lib().hca_attend_backward_workspace(BF16, BF16, B, Tq, H, D, N_cap, m, W, q_pos0))
        ws, ws_bytes = _ws_arg(a, ws, need, q)
        a.done()
        _check(lib().hca_attend_backward(_stream(stream), BF16, BF16, B, Tq, H, D, N_cap, m, W, q_pos0, _p(q),
                                         _p(kv), _p(win), _p(sink), scale, flags, rope_base, rope_dims, _p(out),
                                         _p(lse), _p(dout), _p(dq), _p(dkv), _p(dwin), _p(dsink), _p(ws),
                                         ws_bytes))
    return dq, dkv, dwin, dsink


def lca_grouped_out_proj(o, w_g, w_o, out, *, mid=None, stream=None):
    """Grouped output projection: o [T, n_h, c], w_g [g, d_g, (n_h/g)*c],
    w_o [d_model, g*d_g] (bf16) -> out [T, d_model]; see include/lca.h.
    mid [T, g*d_g] is allocated when not given; returns it."""
    a = _Args("lca_grouped_out_proj")
    bf = _ELEM[BF16]
    a.t(o, "o", dtypes=bf)
    a.t(w_g, "w_g", dtypes=bf)
    a.t(w_o, "w_o", dtypes=bf)
    if o.dim() != 3 or w_g.dim() != 3 or w_o.dim() != 2:
        a._fail("o must be [T, n_h, c], w_g [g, d_g, (n_h/g)*c] and w_o [d_model, g*d_g]")
    T, n_h, c = o.shape
    g, d_g, kg = w_g.shape
    d_model = w_o.shape[0]
    if g < 1 or n_h % g or kg != (n_h // g) * c:
        a._fail(f"w_g has shape {tuple(w_g.shape)}; {n_h} heads of {c} channels in {g} groups need "
                f"[{g}, d_g, {(n_h // g) * c if g and n_h % g == 0 else '?'}]")
    if w_o.shape[1] != g * d_g:
        a._fail(f"w_o has shape {tuple(w_o.shape)}; the call needs [d_model, {g * d_g}]")
    if mid is None:
        mid = torch.empty((T, g * d_g), dtype=torch.bfloat16, device=o.device)
    a.t(mid, "mid", dtypes=bf, numel=T * g * d_g)
    a.t(out, "out", dtypes=bf, numel=T * d_model)
    a.done()
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
