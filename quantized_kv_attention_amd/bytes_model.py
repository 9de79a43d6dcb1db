"""Algorithmic byte counts of the decode path and of the stored cache.

Bytes are counted from what each step must touch at least once: INT4 codes (half a byte
per element), fp32 scale/zero pairs (8 bytes per group), BF16 tail rows, query, scores
and outputs.  Sparse loops are counted from the actual selection: the codes and value
metadata of every selected column in every plane that stores it, and the key metadata
of every distinct (plane, key group) the selection touches.
"""
from __future__ import annotations

import numpy as np

GROUP = 64


def plane_bytes(rows: int, d: int, bits: int = 4) -> int:
    """One stored plane of `rows` slots with `bits`-bit codes: K+V codes, K metadata per
    64-slot group, V metadata per slot."""
    groups = (rows + GROUP - 1) // GROUP
    return rows * d * bits // 4 + groups * d * 8 + rows * (d // GROUP) * 8


def dense_loop_bytes(rows_per_plane, tail_rows: int, n: int, d: int, scores: bool = True, bits_per_plane=None) -> int:
    """Dense loop r for one (sequence, head): the planes it reads (1..r; in the full-state
    codec from the last dense one on), the loop's BF16 tail, q, scores (unless the loop does
    not store them), o."""
    bits_per_plane = [4] * len(rows_per_plane) if bits_per_plane is None else bits_per_plane
    b = sum(plane_bytes(r, d, bt) for r, bt in zip(rows_per_plane, bits_per_plane))
    b += tail_rows * d * 2 * 2          # BF16 K and V rows of the tail
    b += d * 2                          # query
    b += n * 4 if scores else 0         # raw scores written for the next selection
    b += d * (2 + 4) + 4                # o (bf16 + fp32) and lse
    return b


def encode_bytes(rows: int, d: int, loop: int, bits_per_plane=None, full_state: bool = False) -> int:
    """Encoding `rows` stored rows of loop `loop` for one (sequence, head): BF16 K and V rows
    in, the rows' chain through planes 1..loop-1 re-read to form the residual (none in the
    full-state codec), the new plane rows written."""
    bits_per_plane = [4] * loop if bits_per_plane is None else bits_per_plane
    chain = [] if full_state else range(loop - 1)
    return rows * d * 2 * 2 + sum(plane_bytes(rows, d, bits_per_plane[p]) for p in chain) + \
        plane_bytes(rows, d, bits_per_plane[loop - 1])


def select_bytes(n: int, k: int) -> int:
    return n * 4 + 4 + k * 8 + 4        # scores + lse in; idx + p_sel + mass out


def sparse_loop_bytes(idx: np.ndarray, slots_per_plane, n_body: int, d: int, scores: bool = True,
                      bits_per_plane=None) -> int:
    """Sparse loop r for one (sequence, head).

    idx: selected columns (ascending).  slots_per_plane[p]: int array over body positions
    giving the slot of each position in plane p (-1 if not stored), for the planes the loop
    reads (1..r; in the full-state codec from the last dense one on).
    """
    idx = np.asarray(idx)
    body = idx[idx < n_body]
    ntail = int((idx >= n_body).sum())
    bits_per_plane = [4] * len(slots_per_plane) if bits_per_plane is None else bits_per_plane
    b = 0
    for slots, bt in zip(slots_per_plane, bits_per_plane):
        s = slots[body]
        s = s[s >= 0]
        b += s.size * (d * bt // 4 + (d // GROUP) * 8)  # K+V codes + V metadata of each stored column
        b += np.unique(s // GROUP).size * d * 8      # K metadata of each touched key group
    b += ntail * d * 2 * 3                          # tail K^(r), V^(r), V^(r-1)
    b += idx.size * (4 + 4)                         # idx, p_sel
    b += idx.size * (4 + 4) if scores else 0        # score written, then shifted in place
    b += d * 2 + d * 4 + d * (2 + 4) + 4 + 4       # q, o_prev, o (bf16 + fp32), mass, lse
    return b


def cache_payload_bytes(n: int, d: int, heads: int, layers: int, retained, tail_tokens: int = 64,
                        metadata: bool = True) -> dict:
    """Stored bytes of a cross-loop cache at context n.

    retained[r]: fraction of tokens stored by loop r+1.  Without metadata, INT4 is one
    quarter of BF16; the most recent `tail_tokens` tokens of every loop stay BF16.
    """
    bf16_per_loop = 2 * 2 * heads * d * layers * n               # K and V, 2 bytes each
    packed = sum(bf16_per_loop / 4 * r for r in retained)
    if metadata:
        for r in retained:
            rows = r * n
            packed += (np.ceil(rows / GROUP) * d * 8 + rows * (d // GROUP) * 8) * 2 * heads * layers / 2
    tail_extra = 2 * 2 * heads * d * layers * tail_tokens * len(retained) * (1 - 1 / 4)
    baseline = bf16_per_loop * len(retained)
    return dict(baseline=baseline, packed=packed, tail_extra=tail_extra, total=packed + tail_extra,
                reduction=baseline / (packed + tail_extra))


def token_select_bytes(n_prev: int, n: int, dm: int, k: int) -> int:
    """select_tokens for one sequence: the two hidden states of the n_prev tokens of the
    preceding set, the score row written and read by the selection, the kept list."""
    return n_prev * dm * 2 * 2 + n * 4 * 2 + k * 4 * 2 + 8


def prefill_sparse_bytes(n_q: int, n_c: int, d: int) -> int:
    """attn_prefill_sparse for one (sequence, head): the compact queries (two loops), keys and
    values (two loops), positions, lse and previous output in; output (fp32 + bf16), mass out."""
    return n_q * d * 2 * 2 + n_c * d * 2 * 4 + n_q * 4 + n_c * 4 + n_q * 4 + n_q * d * 4 + n_q * d * 6 + n_q * 4


def prefill_sparse_flops(qpos: np.ndarray, cpos: np.ndarray, d: int) -> int:
    """Useful flops of attn_prefill_sparse for one (sequence, head): four products of length d
    (two logits, two value sums) per visible (row, column) pair, 2 flops per multiply-add."""
    vis = np.searchsorted(np.asarray(cpos), np.asarray(qpos), side="right")
    return int(vis.sum()) * 4 * 2 * d
