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
            "kv_append_tail", "attn_decode_dense", "attn_decode_dense_noalloc", "select_columns",
            "attn_decode_sparse", "select_tokens", "qkv_token_workspace_bytes", "kv_gather_rows",
            "attn_prefill_sparse", "qkv_export_plane", "qkv_stream_read")
NOALLOC_SCRATCH_BYTES = 4 << 20
FLAG_PLANE_FULL = 1
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
                ("tail_v", ctypes.c_void_p * MAX_LOOPS), ("stored_loops", ctypes.c_void_p),
                ("residual_bits", ctypes.c_int32), ("full_state", ctypes.c_int32),
                ("error_flags", ctypes.c_void_p)]


class QkvFlush(ctypes.Structure):
    _fields_ = [("pos0", ctypes.c_int32), ("ld_act", ctypes.c_int32), ("act_pos", ctypes.c_void_p),
                ("n_act", ctypes.c_void_p)]


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
    L.qkv_block_bytes.argtypes = [i32, i32]
    L.qkv_block_bytes.restype = sz
    L.qkv_body_len.argtypes = [i32]
    L.qkv_body_len.restype = i32
    L.qkv_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.qkv_workspace_bytes.restype = sz
    L.kv_encode_loop.argtypes = [cp, i32, i32, i32, vp, vp, i32, vp, vp, i32, vp]
    L.kv_encode_loop.restype = i32
    L.kv_append_tail.argtypes = [cp, i32, i32, i32, vp, vp, vp]
    L.kv_append_tail.restype = i32
    fp = ctypes.POINTER(QkvFlush)
    L.attn_decode_dense.argtypes = [cp, i32, vp, vp, vp, f32, vp, vp, vp, i32, vp, fp, vp, sz, vp]
    L.attn_decode_dense.restype = i32
    L.attn_decode_dense_noalloc.argtypes = [cp, i32, vp, vp, vp, f32, vp, vp, vp, i32, vp, vp]
    L.attn_decode_dense_noalloc.restype = i32
    L.select_columns.argtypes = [vp, i32, vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.select_columns.restype = i32
    L.select_tokens.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.select_tokens.restype = i32
    L.qkv_token_workspace_bytes.argtypes = [i32, i32]
    L.qkv_token_workspace_bytes.restype = sz
    L.kv_gather_rows.argtypes = [vp, i32, i32, i32, i32, vp, i32, i32, i32, vp, vp]
    L.kv_gather_rows.restype = i32
    L.attn_prefill_sparse.argtypes = [i32, i32, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp,
                                      vp]
    L.attn_prefill_sparse.restype = i32
    L.qkv_export_plane.argtypes = [cp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.qkv_export_plane.restype = i32
    L.qkv_stream_read.argtypes = [vp, sz, vp, vp]
    L.qkv_stream_read.restype = i32
    L.attn_decode_sparse.argtypes = [cp, i32, vp, vp, vp, f32, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp, fp, vp, sz,
                                     vp]
    L.attn_decode_sparse.restype = i32
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().qkv_strerror(int(status)).decode()


def block_bytes(head_dim: int, bits: int = 4) -> int:
    return int(lib().qkv_block_bytes(head_dim, bits))


def body_len(n_ctx: int) -> int:
    return int(lib().qkv_body_len(n_ctx))


def workspace_bytes(batch, heads, head_dim, max_ctx, max_k) -> int:
    return int(lib().qkv_workspace_bytes(batch, heads, head_dim, max_ctx, max_k))


def _ptr(t):
    """A tensor's device address, or an address given as an int, or None (a NULL argument);
    the entry points' argtypes turn ints into pointers."""
    if t is None or isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


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


def _flush_ref(flush):
    return None if flush is None else ctypes.byref(flush)


def attn_decode_dense(cache, loop, q, sm_scale, o, o_f32, scores, lse, ws, stream=None, k_new=None, v_new=None,
                      flush=None):
    """k_new / v_new: this loop's row of the newest position n_ctx - 1 ([B, H, d] bf16), stored
    in the loop's tail by the same call; None when the tail already holds it.  flush: a
    QkvFlush (this loop's part of the next step's tail flush, encoded by the same launch)."""
    st = lib().attn_decode_dense(ctypes.byref(cache.desc), loop, _ptr(q), _ptr(k_new), _ptr(v_new), float(sm_scale),
                                 _ptr(o), _ptr(o_f32),
                                 _ptr(scores), 0 if scores is None else scores.shape[-1], _ptr(lse),
                                 _flush_ref(flush), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream))
    _check("attn_decode_dense", st)


def attn_decode_dense_noalloc(cache, loop, q, sm_scale, o, o_f32, scores, lse, stream=None, k_new=None, v_new=None):
    """attn_decode_dense with the split partials in the library's fixed device scratch
    (NOALLOC_SCRATCH_BYTES per GPU) instead of a workspace: allocates nothing."""
    st = lib().attn_decode_dense_noalloc(ctypes.byref(cache.desc), loop, _ptr(q), _ptr(k_new), _ptr(v_new),
                                         float(sm_scale), _ptr(o), _ptr(o_f32), _ptr(scores),
                                         0 if scores is None else scores.shape[-1], _ptr(lse), _stream(stream))
    _check("attn_decode_dense_noalloc", st)


def select_columns(scores, lse, n, k, idx, p_sel, mass, ws=None, stream=None):
    B, H = scores.shape[0], scores.shape[1]
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().select_columns(_ptr(scores), scores.shape[-1], _ptr(lse), B, H, n, k, _ptr(idx), _ptr(p_sel),
                              _ptr(mass), _ptr(ws), wsb, _stream(stream))
    _check("select_columns", st)


def attn_decode_sparse(cache, loop, q, sm_scale, idx, p_sel, mass, k, o_prev, lse, scores, o, o_f32, ws,
                       stream=None, k_new=None, v_new=None, flush=None):
    """k_new / v_new and flush as for attn_decode_dense."""
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().attn_decode_sparse(ctypes.byref(cache.desc), loop, _ptr(q), _ptr(k_new), _ptr(v_new), float(sm_scale),
                                  _ptr(idx), _ptr(p_sel),
                                  _ptr(mass), k, _ptr(o_prev), _ptr(lse), _ptr(scores),
                                  0 if scores is None else scores.shape[-1], _ptr(o),
                                  _ptr(o_f32), _flush_ref(flush), _ptr(ws), wsb, _stream(stream))
    _check("attn_decode_sparse", st)


def token_workspace_bytes(batch, k) -> int:
    return int(lib().qkv_token_workspace_bytes(batch, k))


def select_tokens(h_cur, h_prev, n, k, score, act_out, n_act_out, ws, act_prev=None, n_act_prev=None, split=0,
                  n_before=None, stream=None):
    """The next loop's active tokens from hidden states h_cur, h_prev (bf16 [B, ld_tok, dm]):
    top-k normalized change among act_prev (int32 [B, ld_act], n_act_prev [B]; None = every
    token).  Writes score [B, n] fp32, act_out [B, k] int32 (ascending, n_act_out[b] valid),
    n_act_out [B] and, if given, n_before [B] (entries below `split`)."""
    B, ld_tok, dm = h_cur.shape
    ld_act = 0 if act_prev is None else act_prev.shape[-1]
    st = lib().select_tokens(_ptr(h_cur), _ptr(h_prev), ld_tok, B, n, dm, _ptr(act_prev), _ptr(n_act_prev), ld_act,
                             k, split, _ptr(score), _ptr(act_out), _ptr(n_act_out), _ptr(n_before), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream))
    _check("select_tokens", st)


def gather_rows(src, idx, transpose=False, stream=None):
    """Compact rows of src (bf16 [B, H, ld_src, d]) at idx (int32 [B, n] shared by the heads, or
    [B, H, n]): [B, H, n, d], or transposed [B, H, d, ld_t] with ld_t = n rounded up to 32."""
    import torch
    B, H, ld, d = src.shape
    per_head = 1 if idx.dim() == 3 else 0
    n = idx.shape[-1]
    ldt = ((n + 31) // 32) * 32
    dst = torch.empty((B, H, d, ldt) if transpose else (B, H, n, d), dtype=src.dtype, device=src.device)
    st = lib().kv_gather_rows(_ptr(src), B, H, ld, d, _ptr(idx), n, per_head, 1 if transpose else 0, _ptr(dst),
                              _stream(stream))
    _check("kv_gather_rows", st)
    return dst


def attn_prefill_sparse(q, q_prev, q_pos, lse_prev, o_prev, k, k_prev, v_t, v_prev_t, c_pos, sm_scale, o_f32, o=None,
                        mass=None, stream=None):
    """Prefill-side sparse loop over compact buffers (see include/qkv_attn.h)."""
    B, H, n_q, d = q.shape
    n_c = k.shape[2]
    st = lib().attn_prefill_sparse(B, H, d, _ptr(q), _ptr(q_prev), _ptr(q_pos), n_q, _ptr(lse_prev), _ptr(o_prev),
                                   _ptr(k), _ptr(k_prev), _ptr(v_t), _ptr(v_prev_t), _ptr(c_pos), n_c,
                                   float(sm_scale), _ptr(o_f32), _ptr(o), _ptr(mass), _stream(stream))
    _check("attn_prefill_sparse", st)


def export_plane(cache, loop, b, h, n_slots, stream=None):
    """Slots [0, n_slots) of loop `loop`'s plane for (b, h), unpacked by the library:
    dict of device tensors kc, vc (uint8 [n_slots, d]), ks, kz (fp32 [ceil(n_slots/64), d]),
    vs, vz (fp32 [n_slots, d/64])."""
    import torch
    d = cache.d
    dev = cache.planes[loop - 1].device
    out = dict(kc=torch.empty((n_slots, d), dtype=torch.uint8, device=dev),
               vc=torch.empty((n_slots, d), dtype=torch.uint8, device=dev),
               ks=torch.empty(((n_slots + 63) // 64, d), dtype=torch.float32, device=dev),
               kz=torch.empty(((n_slots + 63) // 64, d), dtype=torch.float32, device=dev),
               vs=torch.empty((n_slots, d // 64), dtype=torch.float32, device=dev),
               vz=torch.empty((n_slots, d // 64), dtype=torch.float32, device=dev))
    st = lib().qkv_export_plane(ctypes.byref(cache.desc), loop, b, h, n_slots, _ptr(out["kc"]), _ptr(out["vc"]),
                                _ptr(out["ks"]), _ptr(out["kz"]), _ptr(out["vs"]), _ptr(out["vz"]), _stream(stream))
    _check("qkv_export_plane", st)
    return out


from .cache import LayerCache, DecodeBuffers  # noqa: E402


def stream_read(src, sink, stream=None):
    """Bandwidth reference (not part of the attention path): reads every byte of the device
    tensor `src` with a plain streaming kernel; `sink` is a device int32 tensor of
    STREAM_READ_GROUPS words (each workgroup's XOR of the 32-bit words it read)."""
    assert src.is_cuda and sink.is_cuda and sink.numel() >= STREAM_READ_GROUPS and sink.element_size() == 4
    _check("qkv_stream_read", lib().qkv_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                                   _stream(stream)))
