"""The C ABI library loads without a GPU, exports every declared entry point, and rejects
bad arguments on the host before queueing any work."""
import ctypes
import os
import re

import pytest

import quantized_kv_attention_amd as qkv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qkv_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_exports_every_declared_symbol():
    L = qkv.lib()
    names = declared_functions()
    assert set(names) == set(qkv.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_sizes():
    assert qkv.block_bytes(128) == 10240 and qkv.block_bytes(64) == 5120 and qkv.block_bytes(96) == 0
    # 2-bit planes: codes take half the bytes, metadata the same
    assert qkv.block_bytes(128, 2) == 6144 and qkv.block_bytes(64, 2) == 3072 and qkv.block_bytes(128, 3) == 0
    assert qkv.body_len(0) == 0 and qkv.body_len(127) == 0 and qkv.body_len(256) == 192
    assert qkv.body_len(32768) == 32704
    assert qkv.workspace_bytes(1, 16, 128, 32768, 3277) > 16 * (512 + 1) * 130 * 4 * 0
    assert qkv.workspace_bytes(1, 16, 96, 32768, 3277) == 0
    assert qkv.strerror(qkv.QKV_EINVAL) == "invalid argument"


def _desc(**kw):
    d = qkv.QkvCache()
    d.batch, d.heads, d.head_dim, d.n_loops, d.cap_ctx, d.n_ctx = 1, 1, 128, 2, 256, 256
    for r in range(2):
        d.plane[r].data = 4096 * (r + 1)
        d.plane[r].n_blocks = 4
        d.plane[r].dense = 1
        d.tail_k[r] = 65536 * (r + 1)
        d.tail_v[r] = 65536 * (r + 3)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


class _C:
    def __init__(self, desc):
        self.desc = desc


@pytest.mark.parametrize("mut,expect", [
    (dict(head_dim=96), qkv.QKV_EUNSUPPORTED),
    (dict(n_loops=33), qkv.QKV_EUNSUPPORTED),
    (dict(cap_ctx=100), qkv.QKV_EINVAL),
    (dict(n_ctx=300), qkv.QKV_ECAPACITY),
    (dict(batch=0), qkv.QKV_EINVAL),
])
def test_descriptor_validation(mut, expect):
    L = qkv.lib()
    d = _desc(**mut)
    vp = ctypes.c_void_p
    st = L.attn_decode_dense(ctypes.byref(d), 1, vp(16), None, None, 1.0, None, vp(16), vp(16), 256, vp(16), None, vp(16), 1 << 20, None)
    assert st == expect


def test_argument_validation():
    L = qkv.lib()
    vp = ctypes.c_void_p
    d = _desc()
    # loop out of range, null query, misaligned pointer, short workspace
    assert L.attn_decode_dense(ctypes.byref(d), 3, vp(16), None, None, 1.0, None, vp(16), vp(16), 256, vp(16), None, vp(16), 1 << 20, None) == qkv.QKV_EINVAL
    assert L.attn_decode_dense(ctypes.byref(d), 1, None, None, None, 1.0, None, vp(16), vp(16), 256, vp(16), None, vp(16), 1 << 20, None) == qkv.QKV_EINVAL
    assert L.attn_decode_dense(ctypes.byref(d), 1, vp(18), None, None, 1.0, None, vp(16), vp(16), 256, vp(16), None, vp(16), 1 << 20, None) == qkv.QKV_EINVAL
    assert L.attn_decode_dense(ctypes.byref(d), 1, vp(16), None, None, 1.0, None, vp(16), vp(16), 100, vp(16), None, vp(16), 1 << 20, None) == qkv.QKV_EINVAL
    assert L.attn_decode_dense(ctypes.byref(d), 1, vp(16), None, None, 1.0, None, vp(16), vp(16), 256, vp(16), None, vp(16), 16, None) == qkv.QKV_EWORKSPACE
    # the newest position's row: both pointers or neither, 16-byte aligned
    assert L.attn_decode_dense(ctypes.byref(d), 1, vp(16), vp(16), None, 1.0, None, vp(16), vp(16), 256, vp(16), None, vp(16), 1 << 20, None) == qkv.QKV_EINVAL
    assert L.attn_decode_dense(ctypes.byref(d), 1, vp(16), vp(16), vp(20), 1.0, None, vp(16), vp(16), 256, vp(16), None, vp(16), 1 << 20, None) == qkv.QKV_EINVAL
    assert L.attn_decode_sparse(ctypes.byref(d), 2, vp(16), None, vp(16), 1.0, vp(16), vp(16), vp(16), 4, vp(16), vp(16), vp(16), 256, None, vp(16), None, vp(16), 1 << 20, None) == qkv.QKV_EINVAL
    # sparse loop 1 is not allowed; k beyond the context is not allowed
    assert L.attn_decode_sparse(ctypes.byref(d), 1, vp(16), None, None, 1.0, vp(16), vp(16), vp(16), 4, vp(16), vp(16), vp(16), 256, None, vp(16), None, vp(16), 1 << 20, None) == qkv.QKV_EINVAL
    assert L.attn_decode_sparse(ctypes.byref(d), 2, vp(16), None, None, 1.0, vp(16), vp(16), vp(16), 300, vp(16), vp(16), vp(16), 256, None, vp(16), None, vp(16), 1 << 20, None) == qkv.QKV_EINVAL
    # encode: unaligned range, dense plane with an active list, beyond capacity, tail rows not in the tail
    assert L.kv_encode_loop(ctypes.byref(d), 1, 32, 64, None, None, 0, vp(16), vp(16), 64, None) == qkv.QKV_EINVAL
    assert L.kv_encode_loop(ctypes.byref(d), 1, 0, 64, vp(16), vp(16), 64, vp(16), vp(16), 64, None) == qkv.QKV_EINVAL
    assert L.kv_encode_loop(ctypes.byref(d), 1, 256, 64, None, None, 0, vp(16), vp(16), 64, None) == qkv.QKV_ECAPACITY
    assert L.kv_encode_loop(ctypes.byref(d), 1, 0, 64, None, None, 0, None, None, 0, None) == qkv.QKV_EINVAL
    # a sparse base plane is rejected
    d2 = _desc()
    d2.plane[0].dense = 0
    assert L.kv_encode_loop(ctypes.byref(d2), 1, 0, 64, None, None, 0, vp(16), vp(16), 64, None) == qkv.QKV_EINVAL
    # select: k above n
    assert L.select_columns(vp(16), 256, vp(16), 1, 1, 256, 257, vp(16), vp(16), vp(16), None, 0, None) == qkv.QKV_EINVAL
    assert L.kv_append_tail(ctypes.byref(d), 1, 0, 129, vp(16), vp(16), None) == qkv.QKV_EINVAL
    # stream read: null source, empty, ragged length, misaligned source or sink
    assert L.qkv_stream_read(None, 64, vp(16), None) == qkv.QKV_EINVAL
    assert L.qkv_stream_read(vp(16), 0, vp(16), None) == qkv.QKV_EINVAL
    assert L.qkv_stream_read(vp(16), 40, vp(16), None) == qkv.QKV_EINVAL
    assert L.qkv_stream_read(vp(24), 64, vp(16), None) == qkv.QKV_EINVAL
    assert L.qkv_stream_read(vp(16), 64, vp(20), None) == qkv.QKV_EINVAL
    # token selection: dm not a multiple of 8, k out of range, a list without its counts,
    # a list longer than the context, misaligned states, short workspace
    ws_t = qkv.token_workspace_bytes(1, 8)
    assert ws_t >= (2 + 8) * 4
    args = lambda **kw: dict(dict(hc=vp(16), hp=vp(16), ld=64, B=1, n=64, dm=64, ap=None, npv=None, lda=0, k=8,
                                  ws=ws_t), **kw)
    def tok(a):
        return L.select_tokens(a["hc"], a["hp"], a["ld"], a["B"], a["n"], a["dm"], a["ap"], a["npv"], a["lda"],
                               a["k"], 0, vp(16), vp(16), vp(16), None, vp(16), a["ws"], None)
    assert tok(args(dm=60)) == qkv.QKV_EINVAL
    assert tok(args(k=0)) == qkv.QKV_EINVAL and tok(args(k=65)) == qkv.QKV_EINVAL
    assert tok(args(ap=vp(16))) == qkv.QKV_EINVAL
    assert tok(args(ap=vp(16), npv=vp(16), lda=65)) == qkv.QKV_EINVAL
    assert tok(args(hc=vp(24))) == qkv.QKV_EINVAL
    assert tok(args(ld=32)) == qkv.QKV_EINVAL
    assert tok(args(ws=16)) == qkv.QKV_EWORKSPACE
    # tail flush carried by an attention call: the group must be the tail's oldest 64 rows,
    # must not hold the newest position, and a dense plane takes no active list
    fd = _desc(cap_ctx=320, n_ctx=300)
    for r in range(2):
        fd.plane[r].n_blocks = 5
    def dflush(f):
        return L.attn_decode_dense(ctypes.byref(fd), 1, vp(16), None, None, 1.0, None, vp(16), vp(16), 320, vp(16),
                                   ctypes.byref(f), vp(16), 1 << 20, None)
    assert dflush(qkv.QkvFlush(128, 0, None, None)) == qkv.QKV_EINVAL       # not the body length
    assert dflush(qkv.QkvFlush(192, 64, 16, 16)) == qkv.QKV_EINVAL          # a dense plane with a list
    fd.n_ctx = 256                                                            # the group holds n_ctx - 1
    assert dflush(qkv.QkvFlush(192, 0, None, None)) == qkv.QKV_EINVAL
    # plane export: loop, sequence or head out of range, more slots than the plane holds
    assert L.qkv_export_plane(ctypes.byref(d), 3, 0, 0, 64, *[vp(16)] * 6, None) == qkv.QKV_EINVAL
    assert L.qkv_export_plane(ctypes.byref(d), 1, 1, 0, 64, *[vp(16)] * 6, None) == qkv.QKV_EINVAL
    assert L.qkv_export_plane(ctypes.byref(d), 1, 0, 1, 64, *[vp(16)] * 6, None) == qkv.QKV_EINVAL
    assert L.qkv_export_plane(ctypes.byref(d), 1, 0, 0, 257, *[vp(16)] * 6, None) == qkv.QKV_EINVAL
    # codec fields: 3-bit residuals are unsupported; the full-state codec is 4-bit only
    assert L.attn_decode_dense(ctypes.byref(_desc(residual_bits=3)), 1, vp(16), None, None, 1.0, None, vp(16), vp(16), 256, vp(16), None, vp(16), 1 << 20, None) == qkv.QKV_EUNSUPPORTED
    assert L.attn_decode_dense(ctypes.byref(_desc(residual_bits=2, full_state=1)), 1, vp(16), None, None, 1.0, None, vp(16), vp(16), 256, vp(16), None, vp(16), 1 << 20, None) == qkv.QKV_EUNSUPPORTED
    assert L.attn_decode_dense(ctypes.byref(_desc(full_state=2)), 1, vp(16), None, None, 1.0, None, vp(16), vp(16), 256, vp(16), None, vp(16), 1 << 20, None) == qkv.QKV_EINVAL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(qkv, "_lib", None)
    monkeypatch.setattr(qkv, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError):
        qkv.lib()


def test_host_buffers_and_descriptor_cpu():
    # allocation and descriptor bookkeeping run without a GPU (host memory stands in)
    from quantized_kv_attention_amd import cache as qcache
    c = qcache.LayerCache(2, 3, 128, 4, 512, device="cpu")
    assert c.dense == [True, True, False, False]
    assert c.desc.plane[0].n_blocks == 8 and c.desc.plane[2].dense == 0
    assert c.desc.plane[2].rowmap == c.rowmap[2].data_ptr()
    assert c.planes[0].numel() == 2 * 3 * 8 * qkv.block_bytes(128)
    # 2-bit residual planes: the base keeps 4-bit blocks, later planes take 2-bit ones
    c2 = qcache.LayerCache(1, 2, 128, 4, 256, device="cpu", residual_bits=2)
    assert c2.desc.residual_bits == 2 and c2.bits == [4, 2, 2, 2]
    assert c2.planes[0].numel() == 2 * 4 * 10240 and c2.planes[1].numel() == 2 * 4 * 6144
    c3 = qcache.LayerCache(1, 2, 64, 4, 256, device="cpu", full_state=True)
    assert c3.desc.full_state == 1 and c3.bits == [4, 4, 4, 4]
    b = qcache.DecodeBuffers(c, max_k=50, device="cpu")
    idx, ps, m = b.selection(3, 50)
    assert idx.shape == (2, 3, 50) and ps.shape == (2, 3, 50) and m.shape == (2, 3)
    assert b.ws.numel() >= qkv.workspace_bytes(2, 3, 128, 512, 50)
    a, n = c._active_lists(2, 0, 64)
    assert a.shape == (2, 64) and n.shape == (2,)


def test_layer_stack_layout_cpu():
    # layer l of a stack owns rows l*B..(l+1)*B of the stacked scores / lse / mass and the
    # l-th run of B*H*k entries of each loop's selection: one select_columns call over the
    # stack (batch L*B) writes exactly the per-layer views
    import torch
    from quantized_kv_attention_amd import cache as qcache
    cs = [qcache.LayerCache(2, 3, 128, 4, 512, device="cpu") for _ in range(3)]
    st = qcache.LayerStack(cs, max_k=40, device="cpu")
    assert st.scores.shape == (6, 3, 512) and st.mass.shape == (4, 6, 3)
    k = 17
    for l, b in enumerate(st.layers):
        assert b.scores.data_ptr() == st.scores[2 * l].data_ptr() and b.scores.shape == (2, 3, 512)
        assert b.lse.data_ptr() == st.lse[2 * l].data_ptr()
        idx, ps, m = b.selection(3, k)
        assert idx.shape == (2, 3, k) and m.shape == (2, 3)
        assert idx.data_ptr() == st.idx[2, l * 2 * 3 * k:].data_ptr()
        assert ps.data_ptr() == st.p_sel[2, l * 2 * 3 * k:].data_ptr()
        assert m.data_ptr() == st.mass[2, 2 * l].data_ptr()
        assert b.ws.data_ptr() == st.ws.data_ptr()
    # the stacked selection, viewed as [L*B, H, k], is the layers' selections in order
    st.idx[2, :6 * 3 * k] = torch.arange(6 * 3 * k, dtype=torch.int32)
    whole = st.idx[2, :6 * 3 * k].view(6, 3, k)
    for l, b in enumerate(st.layers):
        assert torch.equal(b.selection(3, k)[0], whole[2 * l:2 * l + 2])


def test_call_addresses_follow_the_current_tensors_cpu():
    # the decode calls pass addresses as integers (DecodeBuffers.out_ptrs / selection_ptrs):
    # they must equal those of the views they stand for, for a standalone layer and for every
    # layer of a stack, and follow a tensor that replaced an attribute (an address kept from
    # the replaced tensor would point at freed memory)
    import torch
    from quantized_kv_attention_amd import cache as qcache
    c = qcache.LayerCache(2, 3, 128, 4, 512, device="cpu")
    cs = [qcache.LayerCache(2, 3, 128, 4, 512, device="cpu") for _ in range(3)]
    st = qcache.LayerStack(cs, max_k=40, device="cpu")
    for b in [qcache.DecodeBuffers(c, max_k=50, device="cpu")] + st.layers:
        for loop in range(1, 5):
            o, o32 = b.out_ptrs(loop)
            assert (o, o32) == (b.o[loop - 1].data_ptr(), b.o_f32[loop - 1].data_ptr())
        for loop in (3, 4):
            for k in (0, 1, 17, 40):
                assert b.selection_ptrs(loop, k) == tuple(t.data_ptr() for t in b.selection(loop, k))
    b = st.layers[1]
    b.o_f32 = torch.zeros_like(b.o_f32)
    b.idx = torch.zeros_like(b.idx)
    assert b.out_ptrs(2)[1] == b.o_f32[1].data_ptr()
    assert b.selection_ptrs(3, 17)[0] == b.selection(3, 17)[0].data_ptr()
