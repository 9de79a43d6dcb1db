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

from . import (GROUP, MAX_LOOPS, TAIL_SLOTS, QkvCache, QkvFlush, attn_decode_dense, attn_decode_sparse, block_bytes,
               body_len, kv_append_tail, kv_encode_loop, select_columns, workspace_bytes)


class LayerCache:
    """Planes, maps and BF16 tails of one layer (B sequences x H heads x R loops).

    dense[r]: loop r+1 stores every body position (loop 1 must be dense).
    sparse_blocks[r]: capacity in 64-slot blocks of a sparse plane (default: enough
    for every position).
    residual_bits: code width of the planes of loops >= 2 (4 or 2; the base is 4-bit).
    full_state: every loop stores its own K/V with 4-bit codes instead of a residual.
    """

    def __init__(self, batch, heads, head_dim, n_loops, cap_ctx, dense=None, sparse_blocks=None,
                 device="cuda", residual_bits=4, full_state=False):
        assert n_loops <= MAX_LOOPS and cap_ctx % GROUP == 0
        assert residual_bits in (2, 4) and not (full_state and residual_bits != 4)
        self.B, self.H, self.d, self.R, self.cap = batch, heads, head_dim, n_loops, cap_ctx
        self.device = device
        self.residual_bits, self.full_state = residual_bits, bool(full_state)
        dense = [True, True] + [False] * (n_loops - 2) if dense is None else list(dense)
        dense = (dense + [dense[-1]] * n_loops)[:n_loops]
        assert dense[0], "loop 1 (the base) stores every position"
        self.dense = dense
        self.bits = [4 if (r == 0 or full_state) else residual_bits for r in range(n_loops)]
        self.block_bytes_of = [block_bytes(head_dim, b) for b in self.bits]
        self.block_bytes = self.block_bytes_of[0]
        self.planes, self.rowmap, self.rowpos, self.rowstart = [], [], [], []
        self.tail_k, self.tail_v = [], []
        desc = QkvCache()
        desc.batch, desc.heads, desc.head_dim, desc.n_loops = batch, heads, head_dim, n_loops
        desc.cap_ctx, desc.n_ctx = cap_ctx, 0
        desc.residual_bits, desc.full_state = residual_bits, 1 if full_state else 0
        for r in range(n_loops):
            bb = self.block_bytes_of[r]
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
        # which loops' sparse planes store each position (kept by the encoder; lets a gather
        # over a deep chain skip the planes that do not store a column)
        self.stored_loops = torch.zeros((batch, cap_ctx), dtype=torch.int32, device=device)
        desc.stored_loops = self.stored_loops.data_ptr()
        # error word of the encoder (a sparse plane without room for a group of active rows)
        self.error_flags = torch.zeros(1, dtype=torch.int32, device=device)
        desc.error_flags = self.error_flags.data_ptr()
        self.desc = desc
        # host copy of each loop's activity for positions still in the tail
        self.act = np.zeros((n_loops, batch, cap_ctx), bool)
        # end of the last 64-row group already encoded by attention calls (flush_args)
        self.preflushed = 0
        self._flush_lists = []

    def errors(self) -> int:
        """The encoder's error word (FLAG_PLANE_FULL: rows of a full sparse plane were not
        stored); synchronizes with the device."""
        return int(self.error_flags.item())

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
        self._flush_before(t, stream)
        self.act[:, :, t] = True
        if torch.is_tensor(k_new) and k_new.dim() == 5:
            kv_append_tail(self, 0, t, k_new, v_new, stream=stream)  # [R, B, H, 1, d], one launch
        else:
            ks = torch.stack([x.reshape(self.B, self.H, 1, self.d) for x in k_new])
            vs = torch.stack([x.reshape(self.B, self.H, 1, self.d) for x in v_new])
            kv_append_tail(self, 0, t, ks, vs, stream=stream)
        self.n_ctx = t + 1

    def advance_token(self, stream=None):
        """Counts the generated token at position n_ctx without writing its rows: each loop's
        attention call of the step stores its own row (k_new / v_new of decode_loop).
        Flushes the tail first if it is full, as append_token does."""
        t = self.n_ctx
        self._flush_before(t, stream)
        self.act[:, :, t] = True
        self.n_ctx = t + 1

    def tail_full(self) -> bool:
        """Whether the next position moves the body boundary (a 64-row flush is due)."""
        n = self.n_ctx
        return body_len(n + 1) > body_len(n)

    def flush_args(self):
        """Per loop, the QkvFlush of the tail's 64 oldest positions, for the attention calls
        of the current step (each call encodes its loop's rows of the group in the same
        launch); the next advance then does not flush them again.  Call when tail_full()."""
        nb = body_len(self.n_ctx)
        out, keep = [], []
        for r in range(self.R):
            if self.dense[r]:
                out.append(QkvFlush(nb, 0, None, None))
            else:
                act_pos, n_act = self._active_lists(r, nb, nb + GROUP)
                ap = torch.from_numpy(act_pos).to(self.device)
                na = torch.from_numpy(n_act).to(self.device)
                keep += [ap, na]
                out.append(QkvFlush(nb, GROUP, ap.data_ptr(), na.data_ptr()))
        self._flush_lists = keep   # the lists must outlive the calls that read them
        self.preflushed = nb + GROUP
        return out

    def _flush_before(self, t, stream):
        """If adding position t moves the body boundary, encodes the tail's 64 oldest
        positions into every loop's plane, loops in order (unless the attention calls of
        the previous step have encoded them already: flush_args)."""
        nb_old, nb_new = body_len(t), body_len(t + 1)
        if nb_new > nb_old and self.preflushed >= nb_new:
            return
        if nb_new > nb_old:
            for r in range(self.R):
                if self.dense[r]:
                    kv_encode_loop(self, r + 1, nb_old, GROUP, stream=stream)
                else:
                    act_pos, n_act = self._active_lists(r, nb_old, nb_old + GROUP)
                    kv_encode_loop(self, r + 1, nb_old, GROUP, torch.from_numpy(act_pos).to(self.device),
                                   torch.from_numpy(n_act).to(self.device), stream=stream)


class DecodeBuffers:
    """Per-layer outputs of a decode step: o / o_f32 per loop, scores, lse, selection, workspace.

    A layer of a LayerStack keeps scores, lse and its selections inside the stack's
    allocations (its rows of a batch of L*B sequences) and shares the stack's workspace."""

    def __init__(self, cache: LayerCache, max_k: int, device="cuda", stack: "LayerStack | None" = None,
                 layer: int = 0):
        B, H, d, R = cache.B, cache.H, cache.d, cache.R
        self.o = torch.zeros((R, B, H, d), dtype=torch.bfloat16, device=device)
        self.o_f32 = torch.zeros((R, B, H, d), dtype=torch.float32, device=device)
        self.max_k = max(1, max_k)
        self.B, self.H = B, H
        if stack is None:
            self.scores = torch.zeros((B, H, cache.cap), dtype=torch.float32, device=device)
            self.lse = torch.zeros((B, H), dtype=torch.float32, device=device)
            # one selection per loop: idx/p_sel [R, B*H*k used as B x H x k], mass [R, B, H]
            self.idx = torch.zeros((R, B * H * self.max_k), dtype=torch.int32, device=device)
            self.p_sel = torch.zeros((R, B * H * self.max_k), dtype=torch.float32, device=device)
            self.mass = torch.zeros((R, B, H), dtype=torch.float32, device=device)
            nbytes = workspace_bytes(B, H, d, cache.cap, self.max_k)
            self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            self.layer = 0
        else:
            self.scores = stack.scores[layer * B:(layer + 1) * B]
            self.lse = stack.lse[layer * B:(layer + 1) * B]
            self.idx, self.p_sel, self.mass, self.ws = stack.idx, stack.p_sel, stack.mass, stack.ws
            self.layer = layer

    def out_ptrs(self, loop: int):
        """Device addresses of o[loop - 1] and o_f32[loop - 1], taken from the current tensors
        at each call (no views built; the attributes may be replaced)."""
        r = loop - 1
        return (self.o.data_ptr() + r * self.o.stride(0) * self.o.element_size(),
                self.o_f32.data_ptr() + r * self.o_f32.stride(0) * self.o_f32.element_size())

    def selection_ptrs(self, loop: int, k: int):
        """Device addresses of the (idx, p_sel, mass) that selection(loop, k) views, taken from
        the current tensors at each call."""
        r = loop - 1
        off = self.layer * self.B * self.H * max(k, 1)
        return (self.idx.data_ptr() + 4 * (r * self.idx.stride(0) + off),
                self.p_sel.data_ptr() + 4 * (r * self.p_sel.stride(0) + off),
                self.mass.data_ptr() + 4 * (r * self.mass.stride(0) + self.layer * self.B * self.mass.stride(1)))

    def selection(self, loop: int, k: int):
        """Views (idx, p_sel, mass) of loop `loop`'s selection of k columns."""
        r = loop - 1
        kk = max(k, 1)
        n = self.B * self.H * kk
        off = self.layer * n
        return (self.idx[r, off:off + n].view(self.B, self.H, kk),
                self.p_sel[r, off:off + n].view(self.B, self.H, kk),
                self.mass[r, self.layer * self.B:(self.layer + 1) * self.B])


class LayerStack:
    """Decode buffers of L layers of one model, laid out as one batch of L*B sequences.

    A looped model runs loop r through every layer before loop r+1 begins, and the
    selection of loop r+1 reads only loop r's scores and lse.  So once loop r has passed
    the last layer, one select_columns call over the stacked scores makes the selections
    of every layer; select_columns treats the L layers as L*B independent sequences.
    Layer l's k selected columns of loop r sit at idx[r, l*B*H*k : (l+1)*B*H*k]."""

    def __init__(self, caches: list, max_k: int, device="cuda"):
        c0 = caches[0]
        for c in caches:
            assert (c.B, c.H, c.d, c.R, c.cap) == (c0.B, c0.H, c0.d, c0.R, c0.cap), "layers differ in shape"
        L, B, H, R = len(caches), c0.B, c0.H, c0.R
        self.caches, self.L, self.B, self.H = list(caches), L, B, H
        self.max_k = max(1, max_k)
        self.scores = torch.zeros((L * B, H, c0.cap), dtype=torch.float32, device=device)
        self.lse = torch.zeros((L * B, H), dtype=torch.float32, device=device)
        self.idx = torch.zeros((R, L * B * H * self.max_k), dtype=torch.int32, device=device)
        self.p_sel = torch.zeros((R, L * B * H * self.max_k), dtype=torch.float32, device=device)
        self.mass = torch.zeros((R, L * B, H), dtype=torch.float32, device=device)
        self.ws = torch.zeros(workspace_bytes(B, H, c0.d, c0.cap, self.max_k), dtype=torch.uint8, device=device)
        self.layers = [DecodeBuffers(c, max_k, device, stack=self, layer=l) for l, c in enumerate(caches)]

    def select(self, loop: int, k: int, stream=None):
        """Selections of loop `loop` for every layer, in one call."""
        r = loop - 1
        kk = max(k, 1)
        n = self.L * self.B * self.H * kk
        select_columns(self.scores, self.lse, self.caches[0].n_ctx, k, self.idx[r, :n], self.p_sel[r, :n],
                       self.mass[r], None, stream)


def k_columns(frac: float, n: int) -> int:
    return min(n, int(math.ceil(frac * n)))


def decode_loop(cache: LayerCache, bufs: DecodeBuffers, loop: int, q, n_dense: int, k: int, sm: float = 1.0,
                stream=None, selected: bool = False, k_new=None, v_new=None, need_scores: bool = True, flush=None):
    """Attention of loop `loop` (1-based) for query q [B, H, d] bf16.

    A sparse loop first selects its k columns from the previous loop's scores, unless
    `selected` says that the selection is already in place (LayerStack.select).
    k_new / v_new ([B, H, d] bf16): this loop's row of the newest position, stored in the
    loop's tail by the attention call itself (after LayerCache.advance_token).
    need_scores=False: the loop stores no scores (a dense loop whose next loop is dense too
    and overwrites them; the last loop, whose scores no selection reads).
    flush: this loop's QkvFlush (LayerCache.flush_args), encoded by the same call."""
    r = loop - 1
    main = torch.cuda.current_stream() if stream is None else stream
    o, o32 = bufs.out_ptrs(loop)
    if loop <= n_dense:
        attn_decode_dense(cache, loop, q, sm, o, o32, bufs.scores if need_scores else None,
                          bufs.lse, bufs.ws, main, k_new=k_new, v_new=v_new, flush=flush)
    else:
        assert k <= bufs.max_k
        if not selected:
            idx, ps, mass = bufs.selection(loop, k)
            select_columns(bufs.scores, bufs.lse, cache.n_ctx, k, idx, ps, mass, None, main)
        idx, ps, mass = bufs.selection_ptrs(loop, k)
        o32_prev = bufs.out_ptrs(loop - 1)[1]
        attn_decode_sparse(cache, loop, q, sm, idx, ps, mass, k, o32_prev, bufs.lse,
                           bufs.scores if need_scores else None, o, o32, bufs.ws, main,
                           k_new=k_new, v_new=v_new, flush=flush)


def scores_read_after(loop: int, n_dense: int, n_loops: int) -> bool:
    """Whether a selection reads loop `loop`'s scores: those of the next loop, if it is sparse."""
    return n_dense <= loop < n_loops


def decode_step(cache: LayerCache, bufs: DecodeBuffers, q, n_dense: int, k: int, sm: float = 1.0, stream=None,
                k_new=None, v_new=None, fused_flush: bool = False):
    """All loops of one decode step of one layer; q[r] bf16 [B, H, d].  With k_new / v_new
    (per loop, [B, H, d] bf16) each loop's call stores its row of the newest position.  A loop
    stores scores only when the next loop selects from them.  fused_flush: when the next
    position moves the body boundary, each loop's call also encodes its rows of the tail's
    64 oldest positions (instead of kv_encode_loop launches at the next advance)."""
    fl = cache.flush_args() if fused_flush and cache.tail_full() else None
    for loop in range(1, cache.R + 1):
        kn = None if k_new is None else k_new[loop - 1]
        vn = None if v_new is None else v_new[loop - 1]
        decode_loop(cache, bufs, loop, q[loop - 1], n_dense, k, sm, stream, k_new=kn, v_new=vn,
                    need_scores=scores_read_after(loop, n_dense, cache.R), flush=None if fl is None else fl[loop - 1])


def decode_step_stack(stack: LayerStack, qs, n_dense: int, k: int, sm: float = 1.0, stream=None,
                      k_new=None, v_new=None, fused_flush: bool = False):
    """One decode step of every layer of a stack, loop-major (loop r through all layers,
    then loop r+1); qs[l][r] is layer l's loop-(r+1) query.  Each sparse loop starts with
    one selection call for all layers.  k_new[l][r] / v_new[l][r] and fused_flush: as for
    decode_step."""
    main = torch.cuda.current_stream() if stream is None else stream
    fls = [c.flush_args() if fused_flush and c.tail_full() else None for c in stack.caches]
    for loop in range(1, stack.caches[0].R + 1):
        if loop > n_dense:
            stack.select(loop, k, main)
        for l, (c, b) in enumerate(zip(stack.caches, stack.layers)):
            kn = None if k_new is None else k_new[l][loop - 1]
            vn = None if v_new is None else v_new[l][loop - 1]
            decode_loop(c, b, loop, qs[l][loop - 1], n_dense, k, sm, main, selected=True, k_new=kn, v_new=vn,
                        need_scores=scores_read_after(loop, n_dense, stack.caches[0].R),
                        flush=None if fls[l] is None else fls[l][loop - 1])
