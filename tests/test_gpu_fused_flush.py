"""The 64-row tail flush encoded by the attention calls of the step before the body
boundary moves (each loop's call encodes its loop's rows in extra workgroups of its own
kernel) gives the results of the separate kv_encode_loop flush, bit for bit: outputs,
scores and lse of every step, planes and maps after every flush, across two flushes, at
head_dim 128 and 64, for the default codec and both variants."""
import dataclasses

import pytest
import torch

from gpu_helpers import Pair, check_step, compare_planes, say, to_dev_bf16
from quantized_kv_attention_amd import cache as qcache
from quantized_kv_attention_amd import synth

pytestmark = pytest.mark.gpu


def _layer(w, n, cap, seed, **codec):
    K, V, act = synth.gen_layer_torch(w, seed, n=n)
    c = qcache.LayerCache(w.B, w.H, w.d, w.R, cap, dense=[w.rho[r] >= 1.0 for r in range(w.R)], **codec)
    c.prefill(K, V, act)
    return c


def _maps_equal(a, b, r):
    if a.dense[r]:
        return True
    return (torch.equal(a.rowmap[r], b.rowmap[r]) and torch.equal(a.rowpos[r], b.rowpos[r])
            and torch.equal(a.rowstart[r], b.rowstart[r]))


@pytest.mark.parametrize("codec", [{}, dict(residual_bits=2), dict(full_state=True)],
                         ids=["int4-residual", "int2-residual", "full-state"])
@pytest.mark.parametrize("wname,H,n0", [("ctx4k", 3, 1000), ("tiny", None, 256)])
def test_fused_flush_equals_separate_flush(wname, H, n0, codec):
    w = synth.WORKLOADS[wname]
    if H is not None:
        w = dataclasses.replace(w, H=H)
    steps = 135                     # two boundary moves
    cap = 64 * ((n0 + steps + 64 + 63) // 64)
    a, b = _layer(w, n0, cap, 5, **codec), _layer(w, n0, cap, 5, **codec)
    max_k = w.k_cols(n0 + steps)
    ba, bb = qcache.DecodeBuffers(a, max_k=max_k), qcache.DecodeBuffers(b, max_k=max_k)
    flushes = fused = 0
    for step in range(steps):
        kn, vn = synth.gen_new_token(w, step)
        kn = [to_dev_bf16(x) for x in kn]
        vn = [to_dev_bf16(x) for x in vn]
        q = [to_dev_bf16(x) for x in synth.gen_queries(w, step)]
        nb0 = qcache.body_len(a.n_ctx)
        a.advance_token()
        b.advance_token()
        flushes += qcache.body_len(a.n_ctx) > nb0
        k = w.k_cols(a.n_ctx)
        fused += b.tail_full()
        qcache.decode_step(a, ba, q, w.n_dense, k, k_new=kn, v_new=vn)
        qcache.decode_step(b, bb, q, w.n_dense, k, k_new=kn, v_new=vn, fused_flush=True)
        torch.cuda.synchronize()
        n = a.n_ctx
        assert torch.equal(ba.o_f32, bb.o_f32), f"step {step}: outputs"
        assert torch.equal(ba.lse, bb.lse), f"step {step}: lse"
        assert torch.equal(ba.scores[:, :, :n], bb.scores[:, :, :n]), f"step {step}: scores"
        if b.preflushed <= qcache.body_len(a.n_ctx):   # both have encoded every group so far
            for r in range(w.R):
                assert torch.equal(a.planes[r], b.planes[r]), f"step {step}: plane {r + 1}"
                assert _maps_equal(a, b, r), f"step {step}: maps of loop {r + 1}"
            assert torch.equal(a.stored_loops, b.stored_loops), f"step {step}: stored-loops words"
    assert flushes == 2 and fused == 2
    say(f"  {wname} {codec}: {steps} steps, {flushes} flushes encoded inside the attention calls, equal")


def test_fused_flush_against_the_oracle():
    # the same path end to end against the oracle after a fused flush (4 loops, d 128)
    w = dataclasses.replace(synth.WORKLOADS["ctx4k"], H=2)
    p = Pair(w, n=900, extra=140)
    for step in range(70):
        k, v = synth.gen_new_token(w, step, heads=p.heads)
        p.gpu.advance_token()
        kn = [to_dev_bf16(x) for x in k]
        vn = [to_dev_bf16(x) for x in v]
        q = [to_dev_bf16(x) for x in p.queries(step)]
        qcache.decode_step(p.gpu, p.bufs, q, w.n_dense, w.k_cols(p.gpu.n_ctx), k_new=kn, v_new=vn, fused_flush=True)
        p.orc.append(k, v)
    torch.cuda.synchronize()
    assert p.gpu.preflushed > 0
    compare_planes(p.gpu, p.orc, range(2), range(2))
    check_step(p, p.queries(77), w.n_dense, w.k_cols(p.gpu.n_ctx), "after a fused flush")
