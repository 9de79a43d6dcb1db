"""GPU parity: the HIP path against the oracle on the same seeded inputs.

Bit-exact: INT4 codes, fp32 scales/zeros, storage maps and the top-k index sets (the
selection compared on identical fp32 scores).  Tolerance: bf16 outputs within rel-L2
2e-3 and max-abs 1e-2 of the oracle rounded to bf16.
"""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_helpers import Pair, assert_out, check_step, compare_planes, say, to_dev_bf16
from quantized_kv_attention_amd import cache as qcache
from quantized_kv_attention_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def test_tiny_codes_and_step():
    w = W["tiny"]
    say(f"tiny: {w}")
    p = Pair(w, extra=80)
    compare_planes(p.gpu, p.orc, [0], [0])
    check_step(p, p.queries(0), w.n_dense, w.k_cols(p.n), "tiny")
    # the untaught selections of both sparse loops sit on gapped scores here, and are
    # asserted identical to the oracle's
    assert p.gapped == 2


def test_tiny_decode_with_flush():
    w = W["tiny"]
    p = Pair(w, extra=80)
    for step in range(64):
        p.append(step)
        if step in (0, 62):
            check_step(p, p.queries(step + 1), w.n_dense, w.k_cols(p.gpu.n_ctx), f"tiny step {step}")
    assert p.gpu.n_ctx == w.n + 64 and p.orc.nb == w.n - 64 + 64
    compare_planes(p.gpu, p.orc, [0], [0])
    check_step(p, p.queries(99), w.n_dense, w.k_cols(p.gpu.n_ctx), "tiny after flush")


@pytest.mark.parametrize("n", [1, 37, 64, 100, 128, 191])
def test_short_contexts(n):
    w = W["tiny"]
    p = Pair(w, n=n, extra=8)
    compare_planes(p.gpu, p.orc, [0], [0])
    check_step(p, p.queries(1), w.n_dense, w.k_cols(n), f"n={n}")


def test_ragged_d128_multihead():
    # 16x128 shape at a ragged length: body 896 + tail 104, several splits and chunks
    w = dataclasses.replace(W["ctx4k"], H=3)
    p = Pair(w, n=1000, extra=70)
    compare_planes(p.gpu, p.orc, range(3), range(3))
    check_step(p, p.queries(0), w.n_dense, w.k_cols(1000), "n=1000 d=128")
    for step in range(25):
        p.append(step)
    compare_planes(p.gpu, p.orc, range(3), range(3))
    check_step(p, p.queries(30), w.n_dense, w.k_cols(p.gpu.n_ctx), "n=1025 d=128 after flush")


def test_ragged_d64_several_splits_and_chunks():
    # head_dim 64 at a ragged length: 12 dense splits and 4 sparse chunks per (b, h), so
    # both merges combine several records with half-wave rows
    w = dataclasses.replace(W["tiny"], H=2)
    p = Pair(w, n=3000, extra=70)
    compare_planes(p.gpu, p.orc, range(2), range(2))
    check_step(p, p.queries(0), w.n_dense, w.k_cols(3000), "n=3000 d=64")
    for step in range(40):
        p.append(step)
    check_step(p, p.queries(41), w.n_dense, w.k_cols(p.gpu.n_ctx), "n=3040 d=64 after flush")


def test_batch_with_different_masks():
    w = dataclasses.replace(W["batch8"], B=3, H=2)
    p = Pair(w, n=700, extra=8)
    a = p.act[2]
    assert not np.array_equal(a[0], a[1])
    compare_planes(p.gpu, p.orc, range(2), range(2))
    check_step(p, p.queries(0), w.n_dense, w.k_cols(700), "batch 3")


def test_deep_recurrence_32_loops():
    w = dataclasses.replace(W["deep32"], H=2)
    p = Pair(w, n=900, extra=8)
    compare_planes(p.gpu, p.orc, range(2), range(2))
    check_step(p, p.queries(0), w.n_dense, w.k_cols(900), "R=32")


@pytest.mark.parametrize("codec", [{}, {"full_state": True}, {"residual_bits": 2}], ids=["int4", "full", "int2"])
def test_deep_recurrence_head_dim_64(codec):
    # d = 64: the deep-chain gather's long columns then spread over eight lane groups of 8
    # lanes (rather than four of 16), with a step across the 64-row tail flush
    w = dataclasses.replace(W["deep32"], H=2, d=64)
    p = Pair(w, n=900, extra=70, **codec)
    compare_planes(p.gpu, p.orc, range(2), range(2), loops=[0, 1, 2, 31])
    check_step(p, p.queries(0), w.n_dense, w.k_cols(900), f"R=32 d=64 {codec}")
    for step in range(66):
        p.append(step)
    check_step(p, p.queries(1), w.n_dense, w.k_cols(p.gpu.n_ctx), f"R=32 d=64 {codec} after a flush")


def test_deep_chain_stored_loops_mask():
    # the per-position mask of the loops whose sparse planes store a position matches the
    # planes' contents, and the deep-chain gather gives the same bits with and without it
    w = dataclasses.replace(W["deep32"], H=2)
    p = Pair(w, n=900, extra=70)
    c = p.gpu
    mask = c.stored_loops.cpu().numpy().view(np.uint32)
    for b in range(w.B):
        for r in range(w.R):
            if c.dense[r]:
                continue
            pos = p.orc.planes[b][0][r].pos
            stored = np.zeros(c.cap, bool)
            stored[pos[pos >= 0]] = True
            assert np.array_equal((mask[b] >> r) & 1 == 1, stored), f"loop {r + 1} mask"
    q = [to_dev_bf16(x) for x in p.queries(0)]
    k = w.k_cols(900)

    def run():
        qcache.decode_step(c, p.bufs, q, w.n_dense, k)
        torch.cuda.synchronize()
        return p.bufs.o_f32.clone(), p.bufs.scores[:, :, :c.n_ctx].clone(), p.bufs.lse.clone()

    with_mask = run()
    keep = c.desc.stored_loops
    c.desc.stored_loops = None
    try:
        without = run()
    finally:
        c.desc.stored_loops = keep
    for a_, b_ in zip(with_mask, without):
        assert torch.equal(a_, b_)


def test_all_columns_is_dense_on_gpu():
    w = dataclasses.replace(W["ctx4k"], H=2)
    p = Pair(w, n=777, extra=8)
    q = p.queries(3)
    dense = p.run_gpu_loopwise(q, w.R, 0)
    full = p.run_gpu_loopwise(q, w.n_dense, 777)
    for r in range(w.R):
        rel = np.linalg.norm(full[r]["o_f32"] - dense[r]["o_f32"]) / np.linalg.norm(dense[r]["o_f32"])
        say(f"  k=n loop {r + 1}: rel-L2 vs dense {rel:.2e}")
        assert rel < 1e-5


@pytest.mark.parametrize("d,n,k", [(128, 4000, 60), (64, 3000, 110)])
def test_selection_spread_over_many_key_groups(d, n, k):
    # a few columns over a long context: a chunk's columns fall in more distinct key groups
    # than a workgroup stages, so the columns past them read their own group metadata
    w = dataclasses.replace(W["ctx4k"] if d == 128 else W["tiny"], H=2)
    p = Pair(w, n=n, extra=8)
    check_step(p, p.queries(5), w.n_dense, k, f"n={n} k={k} d={d}")


def test_no_columns_keeps_previous_output():
    w = W["tiny"]
    p = Pair(w, extra=8)
    s = p.run_gpu_loopwise(p.queries(2), w.n_dense, 0)
    for r in range(w.n_dense, w.R):
        assert np.array_equal(s[r]["o_f32"], s[r - 1]["o_f32"])


def test_special_values_codes():
    # constant channel groups, constant rows, a tiny-magnitude (denormal-range) group, -0
    w = dataclasses.replace(W["tiny"], rho=[1, 1, 1, 1])
    p = Pair(w, extra=8)
    import oracle as orc
    K, V, act = synth.gen_layer(w)
    K = [k.copy() for k in K]
    V = [v.copy() for v in V]
    K[0][0, 0, :64, 5] = synth.bf16_round_bits(np.full(64, 1.5, np.float32))
    V[0][0, 0, 3, :64] = synth.bf16_round_bits(np.full(64, -2.25, np.float32))
    K[0][0, 0, 64:128, 7] = synth.bf16_round_bits(np.linspace(-1e-38, 1e-38, 64).astype(np.float32))
    K[0][0, 0, 128:192, 9] = np.uint16(0x8000)
    cap = 256 + 64
    g = qcache.LayerCache(1, 1, w.d, w.R, cap, dense=[True] * 4)
    g.prefill([to_dev_bf16(k) for k in K], [to_dev_bf16(v) for v in V], act)
    o = orc.OracleCache(1, 1, w.d, w.R, cap)
    o.prefill(K, V, act)
    torch.cuda.synchronize()
    compare_planes(g, o, [0], [0])


def test_dense_loop_without_scores():
    # a dense call given no score buffer: the same o, o_f32 and lse bit for bit, and the
    # score buffer left as it was; the step that skips loop 1's scores ends equal too
    w = dataclasses.replace(W["ctx4k"], H=3)
    p = Pair(w, n=1500, extra=8)
    q = [to_dev_bf16(x) for x in p.queries(2)]
    c, b = p.gpu, p.bufs
    qcache.decode_loop(c, b, 1, q[0], w.n_dense, 0)
    torch.cuda.synchronize()
    ref = [b.o[0].clone(), b.o_f32[0].clone(), b.lse.clone()]
    b.scores.fill_(7.0)
    b.o_f32[0].zero_()
    qcache.decode_loop(c, b, 1, q[0], w.n_dense, 0, need_scores=False)
    torch.cuda.synchronize()
    assert torch.equal(b.o[0], ref[0]) and torch.equal(b.o_f32[0], ref[1]) and torch.equal(b.lse, ref[2])
    assert bool((b.scores == 7.0).all())
    k = w.k_cols(c.n_ctx)
    outs = []
    for skip in (False, True):
        for loop in range(1, w.R + 1):
            qcache.decode_loop(c, b, loop, q[loop - 1], w.n_dense, k,
                               need_scores=(loop >= w.n_dense) if skip else True)
        torch.cuda.synchronize()
        outs.append([b.o_f32[r].clone() for r in range(w.R)] + [b.scores.clone(), b.lse.clone()])
    for x, y in zip(*outs):
        assert torch.equal(x, y)


def test_sparse_loop_without_scores():
    # a sparse call given no score buffer: the same o and o_f32 bit for bit, scores untouched
    w = dataclasses.replace(W["ctx4k"], H=3)
    p = Pair(w, n=1500, extra=8)
    q = [to_dev_bf16(x) for x in p.queries(4)]
    c, b = p.gpu, p.bufs
    k = w.k_cols(c.n_ctx)
    for loop in range(1, w.n_dense + 2):
        qcache.decode_loop(c, b, loop, q[loop - 1], w.n_dense, k)
    torch.cuda.synchronize()
    r = w.n_dense  # the sparse loop just run, 0-based
    ref = [b.o[r].clone(), b.o_f32[r].clone()]
    saved = b.scores.clone()
    qcache.decode_loop(c, b, w.n_dense + 1, q[w.n_dense], w.n_dense, k, selected=True, need_scores=False)
    torch.cuda.synchronize()
    assert torch.equal(b.o[r], ref[0]) and torch.equal(b.o_f32[r], ref[1])
    assert torch.equal(b.scores, saved)


def test_full_sparse_plane_is_reported():
    # loop 3 keeps 25% of 1000 positions (4 groups of rows) but its plane holds 2 blocks: the
    # encoder stores what fits and sets the error word; a plane with room leaves it 0
    import math

    import quantized_kv_attention_amd as qkv
    w = dataclasses.replace(W["ctx4k"], H=2)
    K, V, act = synth.gen_layer(w, n=1000)
    for blocks, expect in ((2, qkv.FLAG_PLANE_FULL), (6, 0)):
        c = qcache.LayerCache(w.B, w.H, w.d, w.R, 1088, sparse_blocks=[0, 0, blocks, blocks])
        c.prefill([to_dev_bf16(k) for k in K], [to_dev_bf16(v) for v in V], act)
        assert c.errors() == expect, (blocks, c.errors())
