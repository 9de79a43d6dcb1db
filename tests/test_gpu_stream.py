"""The bandwidth reference read: every 16-byte word is read once, by the workgroup the
header names, checked through the XOR each workgroup stores."""
import numpy as np
import pytest
import torch

import quantized_kv_attention_amd as qkv
from gpu_helpers import say


@pytest.mark.gpu
@pytest.mark.parametrize("n16", [2048 * 3 + 123, qkv.STREAM_READ_GROUPS * 2048 + 2048 * 5 + 77])
def test_stream_read_xor_per_workgroup(n16):
    G = qkv.STREAM_READ_GROUPS
    say(f"  stream read of {n16} 16-byte words")
    words = np.random.default_rng(n16).integers(0, 1 << 32, size=(n16, 4), dtype=np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((G,), -1, dtype=torch.int32, device="cuda")
    qkv.stream_read(src, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    exp = np.zeros(G, np.uint32)
    np.bitwise_xor.at(exp, (np.arange(n16) // 2048) % G, np.bitwise_xor.reduce(words, axis=1))
    assert np.array_equal(got, exp)
