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


def test_side_stream_selection_matches_inline():
    """Selections issued on the side stream (eager and inside a graph) give the results of
    the inline schedule bit for bit."""
    w = dataclasses.replace(synth.WORKLOADS["ctx4k"], H=3)
    p = Pair(w, n=2100, extra=8)
    k = w.k_cols(2100)
    q = [to_dev_bf16(x) for x in p.queries(5)]
    qcache.decode_step(p.gpu, p.bufs, q, w.n_dense, k)
    torch.cuda.synchronize()
    ref_o, ref_idx, ref_s = p.bufs.o_f32.clone(), p.bufs.idx.clone(), p.bufs.scores.clone()
    side = qcache.SideSelect()
    p.bufs.o_f32.zero_()
    p.bufs.idx.zero_()
    qcache.decode_step(p.gpu, p.bufs, q, w.n_dense, k, side=side)
    torch.cuda.synchronize()
    assert torch.equal(p.bufs.o_f32, ref_o) and torch.equal(p.bufs.idx, ref_idx)
    assert torch.equal(p.bufs.scores, ref_s)
    assert not p.bufs.pending
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qcache.decode_step(p.gpu, p.bufs, q, w.n_dense, k, side=side)
    for rep in range(3):
        p.bufs.o_f32.zero_()
        p.bufs.idx.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(p.bufs.o_f32, ref_o), f"replay {rep}"
        assert torch.equal(p.bufs.idx, ref_idx), f"replay {rep}"
        qcache.decode_step(p.gpu, p.bufs, q, w.n_dense, k)   # eager work between replays
        torch.cuda.synchronize()
    say("  side-stream selections equal the inline schedule")
