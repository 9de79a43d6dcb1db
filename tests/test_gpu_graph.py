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
