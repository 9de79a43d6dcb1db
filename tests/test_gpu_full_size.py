"""Parity at the workloads' full sizes, in the launch configurations the bench uses: the GPU
runs every head (and every sequence); the oracle models a sample of heads (inputs are drawn
per (sequence, head), so the sampled heads' inputs are identical on both sides)."""
import pytest

from gpu_helpers import Pair, check_step, compare_planes, say
from quantized_kv_attention_amd import synth

pytestmark = pytest.mark.gpu


def test_ctx32k_sampled_heads():
    """16 heads x 128, 32K context, 4 loops."""
    w = synth.WORKLOADS["ctx32k"]
    say("ctx32k: generating inputs and encoding")
    p = Pair(w, extra=64, oracle_heads=[0, 11])
    say("ctx32k: comparing planes of heads 0 and 11")
    compare_planes(p.gpu, p.orc, [0, 11], [0, 1])
    say("ctx32k: decode step")
    check_step(p, p.queries(0), w.n_dense, w.k_cols(w.n), "ctx32k")
    say("ctx32k: every loop read densely through its full chain (the bench's comparison row)")
    check_step(p, p.queries(0), w.R, 0, "ctx32k full chain")


def test_ctx4k_64_decode_steps_with_flush():
    """16 heads x 128, 4K context, 64 decode steps (the last one flushes 64 tail rows)."""
    w = synth.WORKLOADS["ctx4k"]
    say("ctx4k: generating inputs and encoding")
    p = Pair(w, extra=80, oracle_heads=[3, 12])
    check_step(p, p.queries(0), w.n_dense, w.k_cols(p.gpu.n_ctx), "ctx4k step 0")
    for step in range(64):
        p.append(step)
    assert p.gpu.n_ctx == w.n + 64
    say("ctx4k: planes after the flush")
    compare_planes(p.gpu, p.orc, [3, 12], [0, 1])
    check_step(p, p.queries(64), w.n_dense, w.k_cols(p.gpu.n_ctx), "ctx4k after 64 steps")


@pytest.mark.timeout(300)
def test_deep32_sampled_heads():
    """40 heads x 128, 8K context, 32 loops (30 sparse loops over the full residual chain)."""
    w = synth.WORKLOADS["deep32"]
    say("deep32: generating inputs and encoding")
    p = Pair(w, extra=64, oracle_heads=[0, 27])
    say("deep32: comparing planes of heads 0 and 27, all 32 loops")
    compare_planes(p.gpu, p.orc, [0, 27], [0, 1])
    say("deep32: decode step")
    check_step(p, p.queries(0), w.n_dense, w.k_cols(w.n), "deep32")


@pytest.mark.timeout(300)
def test_batch8_sampled_heads():
    """8 sequences x 16 heads x 128, 16K context each, per-sequence masks and selections."""
    w = synth.WORKLOADS["batch8"]
    say("batch8: generating inputs and encoding")
    p = Pair(w, extra=64, oracle_heads=[5])
    say("batch8: comparing planes of head 5 in all 8 sequences")
    compare_planes(p.gpu, p.orc, [5], [0])
    say("batch8: decode step")
    check_step(p, p.queries(0), w.n_dense, w.k_cols(w.n), "batch8")
    say("batch8: 64 generated tokens (the last flushes 64 tail rows of every sequence)")
    for step in range(64):
        p.append(step)
    compare_planes(p.gpu, p.orc, [5], [0])
    check_step(p, p.queries(64), w.n_dense, w.k_cols(p.gpu.n_ctx), "batch8 after 64 steps")
