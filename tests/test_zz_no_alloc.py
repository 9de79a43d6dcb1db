"""attn_decode_dense_noalloc (split partials in the library's fixed device scratch) against
attn_decode_dense (caller workspace), through the C ABI: two calls in a row on one GPU, the
second on a smaller cache, each bit-identical to the workspace entry point's outputs; and a
shape whose partials exceed the scratch is refused before anything is queued."""
import ctypes
import dataclasses

import pytest
import torch

import quantized_kv_attention_amd as qkv
from gpu_helpers import Pair, say, to_dev_bf16
from quantized_kv_attention_amd import synth

pytestmark = pytest.mark.gpu


def _call_noalloc(cache, loop, q, o, o_f32, scores, lse):
    L = qkv.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return L.attn_decode_dense_noalloc(ctypes.byref(cache.desc), loop, ctypes.c_void_p(q.data_ptr()), None, None,
                                       1.0, ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(o_f32.data_ptr()),
                                       ctypes.c_void_p(scores.data_ptr()), scores.shape[-1],
                                       ctypes.c_void_p(lse.data_ptr()), stream)


def _compare(p: Pair, loop: int, label: str):
    c, b = p.gpu, p.bufs
    q = to_dev_bf16(p.queries(0)[loop - 1])
    o1, o1f = torch.zeros_like(b.o[0]), torch.zeros_like(b.o_f32[0])
    s1, l1 = torch.full_like(b.scores, 7.0), torch.zeros_like(b.lse)
    qkv.attn_decode_dense(c, loop, q, 1.0, o1, o1f, s1, l1, b.ws)
    o2, o2f = torch.zeros_like(o1), torch.zeros_like(o1f)
    s2, l2 = torch.full_like(s1, 7.0), torch.zeros_like(l1)
    st = _call_noalloc(c, loop, q, o2, o2f, s2, l2)
    assert st == qkv.QKV_OK, qkv.strerror(st)
    torch.cuda.synchronize()
    n = c.n_ctx
    for name, x, y in (("o", o1, o2), ("o_f32", o1f, o2f), ("scores", s1[..., :n], s2[..., :n]), ("lse", l1, l2)):
        assert torch.equal(x, y), f"{label}: {name} differs"
    assert torch.equal(s2[..., n:], s1[..., n:]), f"{label}: scores past n_ctx written"
    say(f"  {label}: no-alloc outputs equal the workspace entry point's")


def test_noalloc_matches_workspace_entry_point_twice():
    w = synth.WORKLOADS["ctx4k"]
    say("no-alloc: 16 heads x 128, n = 4000, loop 2")
    _compare(Pair(w, n=4000, extra=8, oracle_heads=[0]), 2, "first call (16 x 128, 4000, loop 2)")
    w2 = dataclasses.replace(synth.WORKLOADS["tiny"], H=3)
    say("no-alloc: 3 heads x 64, n = 1000, loop 4 read densely through its chain")
    _compare(Pair(w2, n=1000, extra=8, oracle_heads=[0]), 4, "second call (3 x 64, 1000, loop 4)")


def test_noalloc_refuses_partials_beyond_scratch():
    # 64 sequences x 64 heads at 3.7K context need ~8.5 MB of partials: refused on the host
    # (the descriptor's pointers are never dereferenced)
    d = qkv.QkvCache()
    d.batch, d.heads, d.head_dim, d.n_loops, d.cap_ctx, d.n_ctx = 64, 64, 128, 1, 3712, 3700
    d.plane[0].data, d.plane[0].n_blocks, d.plane[0].dense = 4096, 58, 1
    d.tail_k[0], d.tail_v[0] = 65536, 131072

    class C:
        desc = d

    t16 = torch.zeros(8, dtype=torch.float32, device="cuda")
    st = _call_noalloc(C, 1, t16, t16, t16, torch.zeros((1, 3712), device="cuda"), t16)
    assert st == qkv.QKV_EWORKSPACE
