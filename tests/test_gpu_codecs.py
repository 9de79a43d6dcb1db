"""GPU parity of the codec variants (project page, "Main Results": KV residual quantization
precision; explainer section 4, the "Per-loop KIVI4" ablation, and section 5, the 2-bit
setting): 2-bit residual planes and per-loop full-state INT4, against the oracle run with
the same codec.  Bit-exact codes and fp32 scales/zeros; bf16 outputs within rel-L2 2e-3 and
max-abs 1e-2; selections exact on identical fp32 scores, as for the default codec."""
import dataclasses

import pytest

from gpu_helpers import Pair, check_step, compare_planes, say
from quantized_kv_attention_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
CODECS = [dict(residual_bits=2), dict(full_state=True)]
NAMES = ["int2-residual", "full-state-int4"]


@pytest.mark.parametrize("codec", CODECS, ids=NAMES)
def test_tiny_codec_step_and_flush(codec):
    w = W["tiny"]
    p = Pair(w, extra=80, **codec)
    compare_planes(p.gpu, p.orc, [0], [0])
    check_step(p, p.queries(0), w.n_dense, w.k_cols(p.n), f"tiny {codec}")
    for step in range(64):
        p.append(step)
    compare_planes(p.gpu, p.orc, [0], [0])
    check_step(p, p.queries(99), w.n_dense, w.k_cols(p.gpu.n_ctx), f"tiny {codec} after flush")
    # every loop read densely through its chain, and k = 0 (o = o_prev)
    check_step(p, p.queries(7), w.R, 0, f"tiny {codec} dense chain")
    check_step(p, p.queries(8), w.n_dense, 0, f"tiny {codec} k=0")


@pytest.mark.parametrize("codec", CODECS, ids=NAMES)
@pytest.mark.parametrize("d,n", [(128, 1000), (64, 3000)])
def test_ragged_codec_multihead(codec, d, n):
    base = W["ctx4k"] if d == 128 else W["tiny"]
    w = dataclasses.replace(base, H=3)
    p = Pair(w, n=n, extra=70, **codec)
    compare_planes(p.gpu, p.orc, range(3), range(3))
    check_step(p, p.queries(0), w.n_dense, w.k_cols(n), f"n={n} d={d} {codec}")
    for step in range(40):
        p.append(step)
    compare_planes(p.gpu, p.orc, range(3), range(3))
    check_step(p, p.queries(41), w.n_dense, w.k_cols(p.gpu.n_ctx), f"n={n}+40 d={d} {codec}")


@pytest.mark.parametrize("codec", CODECS, ids=NAMES)
def test_deep_chain_codec(codec):
    # 32 loops: the full-state read takes the last plane storing a column, the 2-bit chain
    # sums 31 2-bit residual planes over the base
    w = dataclasses.replace(W["deep32"], H=2)
    p = Pair(w, n=900, extra=8, **codec)
    compare_planes(p.gpu, p.orc, range(2), range(2), loops=[0, 1, 2, 15, 31])
    check_step(p, p.queries(0), w.n_dense, w.k_cols(900), f"R=32 {codec}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("codec", CODECS, ids=NAMES)
def test_ctx32k_codec_sampled_heads(codec):
    """16 heads x 128, 32K context, 4 loops, with the codec variant."""
    w = W["ctx32k"]
    say(f"ctx32k {codec}: generating inputs and encoding")
    p = Pair(w, extra=64, oracle_heads=[2, 13], **codec)
    compare_planes(p.gpu, p.orc, [2, 13], [0, 1])
    check_step(p, p.queries(0), w.n_dense, w.k_cols(w.n), f"ctx32k {codec}")
    check_step(p, p.queries(0), w.R, 0, f"ctx32k {codec} full chain")
