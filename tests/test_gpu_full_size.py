"""Parity at the 32K long-context size, in the launch configuration the bench times: the GPU
runs all 16 heads; the oracle models a sample of heads (inputs are drawn per head, so the
sampled heads' inputs are identical on both sides)."""
import pytest

from gpu_helpers import Pair, check_step, compare_planes, say
from quantized_kv_attention_amd import synth

pytestmark = pytest.mark.gpu


def test_ctx32k_sampled_heads():
    w = synth.WORKLOADS["ctx32k"]
    say("ctx32k: generating inputs and encoding")
    p = Pair(w, extra=64, oracle_heads=[0, 11])
    say("ctx32k: comparing planes of heads 0 and 11")
    compare_planes(p.gpu, p.orc, [0, 11], [0, 1])
    say("ctx32k: decode step")
    check_step(p, p.queries(0), w.n_dense, w.k_cols(w.n), "ctx32k")
