"""The bytes model against the numbers the flozi.net explainer prints (Cell 1, Cell 3)."""
import json
import os

from quantized_kv_attention_amd import bytes_model as bm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bytes_per_token_loop_cell1():
    g = json.load(open(os.path.join(GOLDEN, "cell1_bytes_per_token_loop.json")))
    # 16 heads x 128 x 48 layers, BF16 K and V: the Ouro-2.6B-shaped geometry of the cache
    per = bm.cache_payload_bytes(1, 128, 16, 48, [1.0], tail_tokens=0, metadata=False)["baseline"]
    assert per == g["printed_bytes_per_token_loop"]
    total = bm.cache_payload_bytes(g["context"], 128, 16, 48, [1.0] * g["loops"], 0, False)["baseline"]
    assert total == g["kv_gib"] * 1024 ** 3


def test_ideal_payload_cell3():
    g = json.load(open(os.path.join(GOLDEN, "cell3_ideal_payload.json")))
    r = bm.cache_payload_bytes(g["context"], 128, 16, 48, g["retained"], g["tail_tokens"], metadata=False)
    gib = 1024 ** 3
    dp = g["printed_decimals"]
    assert round(r["packed"] / gib, dp) == g["printed"]["packed_gib"]
    # the page charges the tail once over all loops' BF16 payload: 48 GiB * 64/32768 * 3/4
    tail = r["tail_extra"] / gib
    assert round(tail, dp) == g["printed"]["tail_extra_gib"]
    assert round(r["total"] / gib, dp) == g["printed"]["total_gib"]
    assert round(r["reduction"], dp) == g["printed"]["reduction"]


def test_plane_bytes():
    # 64 rows x d=128: 8 KiB codes + 1 KiB key metadata + 1 KiB value metadata = one block
    assert bm.plane_bytes(64, 128) == 10240
    assert bm.plane_bytes(65, 128) == 65 * 128 + 2 * 1024 + 65 * 16


def test_plane_bytes_two_bit_and_prefill_flops():
    # 2-bit codes take half the code bytes, the metadata stays
    assert bm.plane_bytes(64, 128, 2) == 64 * 128 // 2 + 1024 + 1024
    # one row at position 10 sees the columns at 3 and 10, not 11: 2 pairs x 4 products x 2 d
    assert bm.prefill_sparse_flops([10], [3, 10, 11], 64) == 2 * 4 * 2 * 64
    # the full-state encode re-reads no chain
    assert bm.encode_bytes(64, 128, 3, full_state=True) == 64 * 128 * 4 + 10240
    assert bm.encode_bytes(64, 128, 3) == 64 * 128 * 4 + 3 * 10240
