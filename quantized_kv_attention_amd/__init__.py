"""Quantized cross-loop decode attention for looped Transformers on MI355X (gfx950).

Thin ctypes binding over ``libqkvattn.so`` (C ABI in ``include/qkv_attn.h``).  The
functions below carry the ABI's names and only marshal arguments: every step of the
computation runs in the HIP kernels.  PyTorch provides device memory and streams.
If the library is missing, every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqkvattn.so")

MAX_LOOPS = 32
GROUP = 64
TAIL_SLOTS = 128

QKV_OK, QKV_EINVAL, QKV_EUNSUPPORTED, QKV_ECAPACITY, QKV_ELAUNCH, QKV_EWORKSPACE = 0, -1, -2, -3, -4, -5

EXPORTED = ("qkv_strerror", "qkv_block_bytes", "qkv_body_len", "qkv_workspace_bytes", "kv_encode_loop",
            "kv_append_tail", "attn_decode_dense", "select_columns", "attn_decode_sparse", "qkv_stream_read")
STREAM_READ_GROUPS = 2048


class QkvError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status} ({strerror(status)})")
        self.status = status


class QkvPlane(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("n_blocks", ctypes.c_int32), ("dense", ctypes.c_int32),
                ("rowmap", ctypes.c_void_p), ("rowpos", ctypes.c_void_p), ("rowstart", ctypes.c_void_p)]


class QkvCache(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_loops", ctypes.c_int32), ("cap_ctx", ctypes.c_int32), ("n_ctx", ctypes.c_int32),
                ("plane", QkvPlane * MAX_LOOPS), ("tail_k", ctypes.c_void_p * MAX_LOOPS),
                ("tail_v", ctypes.c_void_p * MAX_LOOPS), ("stored_loops", ctypes.c_void_p)]


_lib = None


def lib():
    """Loads libqkvattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first (__graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    cp = ctypes.POINTER(QkvCache)
    L.qkv_strerror.argtypes = [i32]
    L.qkv_strerror.restype = ctypes.c_char_p
    L.qkv_block_bytes.argtypes = [i32]
    L.qkv_block_bytes.restype = sz
    L.qkv_body_len.argtypes = [i32]
    L.qkv_body_len.restype = i32
    L.qkv_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.qkv_workspace_bytes.restype = sz
    L.kv_encode_loop.argtypes = [cp, i32, i32, i32, vp, vp, i32, vp, vp, i32, vp]
    L.kv_encode_loop.restype = i32
    L.kv_append_tail.argtypes = [cp, i32, i32, i32, vp, vp, vp]
    L.kv_append_tail.restype = i32
    L.attn_decode_dense.argtypes = [cp, i32, vp, vp, vp, f32, vp, vp, vp, i32, vp, vp, sz, vp]
    L.attn_decode_dense.restype = i32
    L.select_columns.argtypes = [vp, i32, vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.select_columns.restype = i32
    L.qkv_stream_read.argtypes = [vp, sz, vp, vp]
    L.qkv_stream_read.restype = i32
    L.attn_decode_sparse.argtypes = [cp, i32, vp, vp, vp, f32, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    L.attn_decode_sparse.restype = i32
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().qkv_strerror(int(status)).decode()


def block_bytes(head_dim: int) -> int:
    return int(lib().qkv_block_bytes(head_dim))


def body_len(n_ctx: int) -> int:
    return int(lib().qkv_body_len(n_ctx))


def workspace_bytes(batch, heads, head_dim, max_ctx, max_k) -> int:
    return int(lib().qkv_workspace_bytes(batch, heads, head_dim, max_ctx, max_k))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, st):
    if st != QKV_OK:
        raise QkvError(fn, st)


def kv_encode_loop(cache, loop, pos0, n_pos, act_pos=None, n_act=None, k_src=None, v_src=None, stream=None):
    """Residual-quantize encode of `loop` for positions [pos0, pos0+n_pos).

    act_pos int32 [B, ld] / n_act int32 [B] (sparse planes; None for dense planes);
    k_src, v_src bf16 [B, H, ld_src, d] (None: read the rows from the loop's BF16 tail)."""
    ld_act = 0 if act_pos is None else act_pos.shape[-1]
    ld_src = 0 if k_src is None else k_src.shape[2]
    st = lib().kv_encode_loop(ctypes.byref(cache.desc), loop, pos0, n_pos, _ptr(act_pos), _ptr(n_act), ld_act,
                              _ptr(k_src), _ptr(v_src), ld_src, _stream(stream))
    _check("kv_encode_loop", st)


def kv_append_tail(cache, loop, pos0, k, v, stream=None):
    """Writes bf16 rows k, v [B, H, n_rows, d] at positions pos0.. of `loop`'s BF16 tail
    (loop 0: every loop, k, v [R, B, H, n_rows, d])."""
    st = lib().kv_append_tail(ctypes.byref(cache.desc), loop, pos0, k.shape[-2], _ptr(k), _ptr(v), _stream(stream))
    _check("kv_append_tail", st)


def attn_decode_dense(cache, loop, q, sm_scale, o, o_f32, scores, lse, ws, stream=None, k_new=None, v_new=None):
    """k_new / v_new: this loop's row of the newest position n_ctx - 1 ([B, H, d] bf16), stored
    in the loop's tail by the same call; None when the tail already holds it."""
    st = lib().attn_decode_dense(ctypes.byref(cache.desc), loop, _ptr(q), _ptr(k_new), _ptr(v_new), float(sm_scale),
                                 _ptr(o), _ptr(o_f32),
                                 _ptr(scores), 0 if scores is None else scores.shape[-1], _ptr(lse), _ptr(ws),
                                 ws.numel() * ws.element_size(),
                                 _stream(stream))
    _check("attn_decode_dense", st)


def select_columns(scores, lse, n, k, idx, p_sel, mass, ws=None, stream=None):
    B, H = scores.shape[0], scores.shape[1]
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().select_columns(_ptr(scores), scores.shape[-1], _ptr(lse), B, H, n, k, _ptr(idx), _ptr(p_sel),
                              _ptr(mass), _ptr(ws), wsb, _stream(stream))
    _check("select_columns", st)


def attn_decode_sparse(cache, loop, q, sm_scale, idx, p_sel, mass, k, o_prev, lse, scores, o, o_f32, ws,
                       stream=None, k_new=None, v_new=None):
    """k_new / v_new as for attn_decode_dense."""
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().attn_decode_sparse(ctypes.byref(cache.desc), loop, _ptr(q), _ptr(k_new), _ptr(v_new), float(sm_scale),
                                  _ptr(idx), _ptr(p_sel),
                                  _ptr(mass), k, _ptr(o_prev), _ptr(lse), _ptr(scores),
                                  0 if scores is None else scores.shape[-1], _ptr(o),
                                  _ptr(o_f32), _ptr(ws), wsb, _stream(stream))
    _check("attn_decode_sparse", st)


from .cache import LayerCache, DecodeBuffers  # noqa: E402


def stream_read(src, sink, stream=None):
    """Bandwidth reference (not part of the attention path): reads every byte of the device
    tensor `src` with a plain streaming kernel; `sink` is a device int32 tensor of
    STREAM_READ_GROUPS words (each workgroup's XOR of the 32-bit words it read)."""
    assert src.is_cuda and sink.is_cuda and sink.numel() >= STREAM_READ_GROUPS and sink.element_size() == 4
    _check("qkv_stream_read", lib().qkv_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                                   _stream(stream)))
