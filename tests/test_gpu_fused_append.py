"""The newest position's rows stored by the attention calls themselves (k_new / v_new)
give the results of a separate kv_append_tail, bit for bit, across a tail flush."""
import dataclasses

import pytest
import torch

from gpu_helpers import say, to_dev_bf16
from quantized_kv_attention_amd import cache as qcache
from quantized_kv_attention_amd import synth

pytestmark = pytest.mark.gpu


def _layer(w, n, cap, seed):
    K, V, act = synth.gen_layer_torch(w, seed, n=n)
    c = qcache.LayerCache(w.B, w.H, w.d, w.R, cap, dense=[w.rho[r] >= 1.0 for r in range(w.R)])
    c.prefill(K, V, act)
    return c


@pytest.mark.parametrize("wname,H", [("ctx4k", 3), ("tiny", None)])
def test_fused_append_equals_separate_append(wname, H):
    w = synth.WORKLOADS[wname]
    if H is not None:
        w = dataclasses.replace(w, H=H)
    n0 = min(w.n, 1000)
    steps = 70                      # crosses at least one 64-row flush
    cap = 64 * ((n0 + steps + 64 + 63) // 64)
    a, b = _layer(w, n0, cap, 3), _layer(w, n0, cap, 3)
    max_k = w.k_cols(n0 + steps)
    ba, bb = qcache.DecodeBuffers(a, max_k=max_k), qcache.DecodeBuffers(b, max_k=max_k)
    flushes = 0
    for step in range(steps):
        kn, vn = synth.gen_new_token(w, step)
        kn = [to_dev_bf16(x) for x in kn]
        vn = [to_dev_bf16(x) for x in vn]
        q = [to_dev_bf16(x) for x in synth.gen_queries(w, step)]
        nb0 = qcache.body_len(a.n_ctx)
        a.append_token(kn, vn)
        b.advance_token()
        flushes += qcache.body_len(a.n_ctx) > nb0
        k = w.k_cols(a.n_ctx)
        qcache.decode_step(a, ba, q, w.n_dense, k)
        qcache.decode_step(b, bb, q, w.n_dense, k, k_new=kn, v_new=vn)
        torch.cuda.synchronize()
        n = a.n_ctx
        assert torch.equal(ba.o_f32, bb.o_f32), f"step {step}: outputs"
        assert torch.equal(ba.lse, bb.lse), f"step {step}: lse"
        assert torch.equal(ba.scores[:, :, :n], bb.scores[:, :, :n]), f"step {step}: scores"
        if step % 16 == 15 or step == steps - 1:
            for r in range(w.R):
                assert torch.equal(a.tail_k[r], b.tail_k[r]) and torch.equal(a.tail_v[r], b.tail_v[r]), \
                    f"step {step}: tail of loop {r + 1}"
                assert torch.equal(a.planes[r], b.planes[r]), f"step {step}: plane {r + 1}"
    assert flushes >= 1
    say(f"  {wname}: {steps} steps with {flushes} flush(es), fused append equals kv_append_tail")
