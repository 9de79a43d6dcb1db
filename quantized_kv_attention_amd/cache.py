"""One layer's cross-loop cache on the GPU, and the decode-step orchestration over it.

Allocation (torch device memory) and host bookkeeping only; every byte of the path is
produced by the library's kernels.  Loop order within a decode step follows the PyPI
page's configuration: dense loops first, then per sparse loop a top-k selection from the
preceding loop's scores followed by the sparse splice (project page STEP 02).
"""
from __future__ import annotations

import ctypes
import math

import numpy as np
import torch

from . import (GROUP, MAX_LOOPS, TAIL_SLOTS, QkvCache, attn_decode_dense, attn_decode_sparse, block_bytes,
               body_len, kv_append_tail, kv_encode_loop, select_columns, workspace_bytes)


class LayerCache:
    """Planes, maps and BF16 tails of one layer (B sequences x H heads x R loops).

    dense[r]: loop r+1 stores every body position (loop 1 must be dense).
    sparse_blocks[r]: capacity in 64-slot blocks of a sparse plane (default: enough
    for every position).
    """

    def __init__(self, batch, heads, head_dim, n_loops, cap_ctx, dense=None, sparse_blocks=None,
                 device="cuda"):
        assert n_loops <= MAX_LOOPS and cap_ctx % GROUP == 0
        self.B, self.H, self.d, self.R, self.cap = batch, heads, head_dim, n_loops, cap_ctx
        self.device = device
        dense = [True, True] + [False] * (n_loops - 2) if dense is None else list(dense)
        dense = (dense + [dense[-1]] * n_loops)[:n_loops]
        assert dense[0], "loop 1 (the base) stores every position"
        self.dense = dense
        bb = block_bytes(head_dim)
        self.block_bytes = bb
        self.planes, self.rowmap, self.rowpos, self.rowstart = [], [], [], []
        self.tail_k, self.tail_v = [], []
        desc = QkvCache()
        desc.batch, desc.heads, desc.head_dim, desc.n_loops = batch, heads, head_dim, n_loops
        desc.cap_ctx, desc.n_ctx = cap_ctx, 0
        for r in range(n_loops):
            nblk = cap_ctx // GROUP
            if not dense[r] and sparse_blocks is not None:
                nblk = int(sparse_blocks[r])
            data = torch.zeros(batch * heads * nblk * bb, dtype=torch.uint8, device=device)
            self.planes.append(data)
            desc.plane[r].data = data.data_ptr()
            desc.plane[r].n_blocks = nblk
            desc.plane[r].dense = 1 if dense[r] else 0
            if dense[r]:
                self.rowmap.append(None)
                self.rowpos.append(None)
                self.rowstart.append(None)
            else:
                rm = torch.full((batch, cap_ctx), -1, dtype=torch.int32, device=device)
                rp = torch.full((batch, nblk * GROUP), -1, dtype=torch.int32, device=device)
                rs = torch.zeros((batch, cap_ctx // GROUP + 1), dtype=torch.int32, device=device)
                self.rowmap.append(rm)
                self.rowpos.append(rp)
                self.rowstart.append(rs)
                desc.plane[r].rowmap = rm.data_ptr()
                desc.plane[r].rowpos = rp.data_ptr()
                desc.plane[r].rowstart = rs.data_ptr()
            tk = torch.zeros((batch, heads, TAIL_SLOTS, head_dim), dtype=torch.bfloat16, device=device)
            tv = torch.zeros_like(tk)
            self.tail_k.append(tk)
            self.tail_v.append(tv)
            desc.tail_k[r] = tk.data_ptr()
            desc.tail_v[r] = tv.data_ptr()
        self.desc = desc
        # host copy of each loop's activity for positions still in the tail
        self.act = np.zeros((n_loops, batch, cap_ctx), bool)

    @property
    def n_ctx(self) -> int:
        return int(self.desc.n_ctx)

    @n_ctx.setter
    def n_ctx(self, n: int):
        assert 0 <= n <= self.cap
        self.desc.n_ctx = int(n)

    def nbytes(self) -> int:
        t = sum(p.numel() for p in self.planes)
        t += sum(x.numel() * 2 for x in self.tail_k + self.tail_v)
        return t

    # ------------------------------------------------------------------ prefill ----
    def prefill(self, K, V, act, stream=None):
        """Encodes a prompt of n positions.

        K[r], V[r]: bf16 device tensors [B, H, n, d] (loop r+1's keys/values; inactive
        tokens carry the previous loop's value); act[r]: bool array [B, n].
        """
        n = K[0].shape[2]
        nb = body_len(n)
        for r in range(self.R):
            self.act[r, :, :n] = np.asarray(act[r])
        for r in range(self.R):
            if nb > 0:
                self._encode_rows(r, 0, nb, K[r], V[r], src_offset=0, stream=stream)
            if n > nb:
                kv_append_tail(self, r + 1, nb, K[r][:, :, nb:n].contiguous(), V[r][:, :, nb:n].contiguous(),
                               stream=stream)
        self.n_ctx = n

    def _encode_rows(self, r, p0, n_pos, Kr, Vr, src_offset, stream=None):
        """Encodes loop r+1 for body positions [p0, p0+n_pos) from rows of Kr/Vr [B,H,*,d]
        indexed by position - src_offset."""
        if self.dense[r]:
            ks = Kr[:, :, p0 - src_offset:p0 - src_offset + n_pos].contiguous()
            vs = Vr[:, :, p0 - src_offset:p0 - src_offset + n_pos].contiguous()
            kv_encode_loop(self, r + 1, p0, n_pos, k_src=ks, v_src=vs, stream=stream)
            return
        act_pos, n_act = self._active_lists(r, p0, p0 + n_pos)
        ks = torch.zeros((self.B, self.H, n_pos, self.d), dtype=torch.bfloat16, device=self.device)
        vs = torch.zeros_like(ks)
        for b in range(self.B):
            c = int(n_act[b])
            if c:
                rows = torch.from_numpy(act_pos[b, :c].astype(np.int64) - src_offset).to(self.device)
                ks[b, :, :c] = Kr[b].index_select(1, rows)
                vs[b, :, :c] = Vr[b].index_select(1, rows)
        kv_encode_loop(self, r + 1, p0, n_pos, torch.from_numpy(act_pos).to(self.device),
                       torch.from_numpy(n_act).to(self.device), ks, vs, stream=stream)

    def _active_lists(self, r, p0, p1):
        act_pos = np.zeros((self.B, p1 - p0), np.int32)
        n_act = np.zeros(self.B, np.int32)
        for b in range(self.B):
            pos = p0 + np.nonzero(self.act[r, b, p0:p1])[0]
            act_pos[b, :pos.size] = pos
            n_act[b] = pos.size
        return act_pos, n_act

    # ------------------------------------------------------------------ decode -----
    def append_token(self, k_new, v_new, stream=None):
        """Adds the generated token (active in every loop) at position n_ctx.

        k_new[r], v_new[r]: bf16 [B, H, d].  If the tail would reach 128 tokens, its oldest
        64 positions are first encoded into every loop's plane, loops in order.
        """
        t = self.n_ctx
        nb_old, nb_new = body_len(t), body_len(t + 1)
        if nb_new > nb_old:
            for r in range(self.R):
                if self.dense[r]:
                    kv_encode_loop(self, r + 1, nb_old, GROUP, stream=stream)
                else:
                    act_pos, n_act = self._active_lists(r, nb_old, nb_old + GROUP)
                    kv_encode_loop(self, r + 1, nb_old, GROUP, torch.from_numpy(act_pos).to(self.device),
                                   torch.from_numpy(n_act).to(self.device), stream=stream)
        self.act[:, :, t] = True
        if torch.is_tensor(k_new) and k_new.dim() == 5:
            kv_append_tail(self, 0, t, k_new, v_new, stream=stream)  # [R, B, H, 1, d], one launch
        else:
            ks = torch.stack([x.reshape(self.B, self.H, 1, self.d) for x in k_new])
            vs = torch.stack([x.reshape(self.B, self.H, 1, self.d) for x in v_new])
            kv_append_tail(self, 0, t, ks, vs, stream=stream)
        self.n_ctx = t + 1


class DecodeBuffers:
    """Per-layer outputs of a decode step: o / o_f32 per loop, scores, lse, selection, workspace."""

    def __init__(self, cache: LayerCache, max_k: int, device="cuda"):
        B, H, d, R = cache.B, cache.H, cache.d, cache.R
        self.o = torch.zeros((R, B, H, d), dtype=torch.bfloat16, device=device)
        self.o_f32 = torch.zeros((R, B, H, d), dtype=torch.float32, device=device)
        self.scores = torch.zeros((B, H, cache.cap), dtype=torch.float32, device=device)
        self.lse = torch.zeros((B, H), dtype=torch.float32, device=device)
        self.max_k = max(1, max_k)
        # one selection per loop: idx/p_sel [R, B*H*k used as B x H x k], mass [R, B, H]
        self.idx = torch.zeros((R, B * H * self.max_k), dtype=torch.int32, device=device)
        self.p_sel = torch.zeros((R, B * H * self.max_k), dtype=torch.float32, device=device)
        self.mass = torch.zeros((R, B, H), dtype=torch.float32, device=device)
        self.B, self.H = B, H
        nbytes = workspace_bytes(B, H, d, cache.cap, self.max_k)
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.pending = {}   # loop -> (k, event) of a selection issued on a side stream

    def selection(self, loop: int, k: int):
        """Views (idx, p_sel, mass) of loop `loop`'s selection of k columns."""
        r = loop - 1
        kk = max(k, 1)
        n = self.B * self.H * kk
        return (self.idx[r, :n].view(self.B, self.H, kk), self.p_sel[r, :n].view(self.B, self.H, kk),
                self.mass[r])


def k_columns(frac: float, n: int) -> int:
    return min(n, int(math.ceil(frac * n)))


class SideSelect:
    """Second stream (default priority) for the column selections of sparse loops.

    Loop r+1's selection reads only loop r's scores and lse, so it can start as soon as
    loop r of the same layer is done, beside whatever the main stream runs next (in a
    looped model: loop r of the following layers).  The sparse loop waits for it."""

    def __init__(self):
        self.stream = torch.cuda.Stream()

    def issue(self, cache, bufs, loop, k, main):
        ev = torch.cuda.Event()
        ev.record(main)
        self.stream.wait_event(ev)
        idx, ps, mass = bufs.selection(loop, k)
        select_columns(bufs.scores, bufs.lse, cache.n_ctx, k, idx, ps, mass, None, self.stream)
        done = torch.cuda.Event()
        done.record(self.stream)
        bufs.pending[loop] = (k, done)


def decode_loop(cache: LayerCache, bufs: DecodeBuffers, loop: int, q, n_dense: int, k: int, sm: float = 1.0,
                stream=None, side: SideSelect | None = None):
    """Attention of loop `loop` (1-based) for query q [B, H, d] bf16.

    With `side`, the selection of the next loop is issued on the side stream as soon as
    this loop's scores are written, and a sparse loop consumes the selection issued for it."""
    r = loop - 1
    main = torch.cuda.current_stream() if stream is None else stream
    if loop <= n_dense:
        attn_decode_dense(cache, loop, q, sm, bufs.o[r], bufs.o_f32[r], bufs.scores, bufs.lse, bufs.ws, main)
    else:
        n = cache.n_ctx
        assert k <= bufs.max_k
        idx, ps, mass = bufs.selection(loop, k)
        pend = bufs.pending.pop(loop, None)
        if pend is not None and pend[0] == k:
            main.wait_event(pend[1])
        else:
            if pend is not None:
                main.wait_event(pend[1])   # a stale selection must finish before it is overwritten
            select_columns(bufs.scores, bufs.lse, n, k, idx, ps, mass, None, main)
        attn_decode_sparse(cache, loop, q, sm, idx, ps, mass, k, bufs.o_f32[r - 1], bufs.lse, bufs.scores,
                           bufs.o[r], bufs.o_f32[r], bufs.ws, main)
    if side is not None and n_dense <= loop < cache.R:
        side.issue(cache, bufs, loop + 1, k, main)


def decode_step(cache: LayerCache, bufs: DecodeBuffers, q, n_dense: int, k: int, sm: float = 1.0, stream=None,
                side: SideSelect | None = None):
    """All loops of one decode step of one layer; q[r] bf16 [B, H, d]."""
    for loop in range(1, cache.R + 1):
        decode_loop(cache, bufs, loop, q[loop - 1], n_dense, k, sm, stream, side)
