"""Decode steps captured in a HIP graph give the eager results on every replay."""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_helpers import Pair, say, to_dev_bf16
from quantized_kv_attention_amd import cache as qcache
from quantized_kv_attention_amd import synth

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    w = dataclasses.replace(synth.WORKLOADS["ctx4k"], H=2)
    p = Pair(w, n=1500, extra=8)
    k = w.k_cols(1500)
    qs = [[to_dev_bf16(x) for x in p.queries(s)] for s in range(2)]
    q_static = [torch.empty_like(x) for x in qs[0]]

    def step():
        qcache.decode_step(p.gpu, p.bufs, q_static, w.n_dense, k)

    eager = []
    for s in range(2):
        for dst, src in zip(q_static, qs[s]):
            dst.copy_(src)
        step()
        torch.cuda.synchronize()
        eager.append(p.bufs.o_f32.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        s = rep % 2
        for dst, src in zip(q_static, qs[s]):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(p.bufs.o_f32, eager[s]), f"replay {rep} differs from eager"
        # eager work between replays
        step()
        torch.cuda.synchronize()
        assert torch.equal(p.bufs.o_f32, eager[s])
    say("  graph replays equal eager results")


def test_layer_stack_matches_per_layer_steps():
    """Loop-major steps of a three-layer stack, with one selection call per sparse loop for
    all layers, equal each layer's own step bit for bit (eager and replayed from a graph)."""
    w = dataclasses.replace(synth.WORKLOADS["ctx4k"], H=3)
    n = 2100
    k = w.k_cols(n)
    cap = 64 * ((n + 8 + 64 + 63) // 64)
    caches, qs = [], []
    for l in range(3):
        K, V, act = synth.gen_layer_torch(w, 7 + l, n=n)
        c = qcache.LayerCache(w.B, w.H, w.d, w.R, cap, dense=[w.rho[r] >= 1.0 for r in range(w.R)])
        c.prefill(K, V, act)
        caches.append(c)
        qs.append([to_dev_bf16(x) for x in synth.gen_queries(w, 30 + l)])
    ref = []
    for c, q in zip(caches, qs):
        b = qcache.DecodeBuffers(c, max_k=k)
        qcache.decode_step(c, b, q, w.n_dense, k)
        torch.cuda.synchronize()
        sel = [[t.clone() for t in b.selection(loop, k)] for loop in range(w.n_dense + 1, w.R + 1)]
        ref.append((b.o_f32.clone(), b.scores.clone(), b.lse.clone(), sel))
    stack = qcache.LayerStack(caches, max_k=k)

    def check(what):
        for l, b in enumerate(stack.layers):
            o, sc, lse, sel = ref[l]
            assert torch.equal(b.o_f32, o), f"{what}: layer {l} outputs"
            assert torch.equal(b.scores, sc) and torch.equal(b.lse, lse), f"{what}: layer {l} scores"
            for loop, tr in zip(range(w.n_dense + 1, w.R + 1), sel):
                for t, u in zip(b.selection(loop, k), tr):
                    assert torch.equal(t, u), f"{what}: layer {l} loop {loop} selection"

    qcache.decode_step_stack(stack, qs, w.n_dense, k)
    torch.cuda.synchronize()
    check("eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qcache.decode_step_stack(stack, qs, w.n_dense, k)
    for rep in range(3):
        stack.idx.zero_()
        for b in stack.layers:
            b.o_f32.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(f"replay {rep}")
        qcache.decode_step_stack(stack, qs, w.n_dense, k)   # eager work between replays
        torch.cuda.synchronize()
    say("  stacked loop-major steps equal per-layer steps")
