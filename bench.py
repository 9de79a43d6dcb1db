#!/usr/bin/env python3
"""Decode-attention bench: quantized cross-loop KV cache, 32K context, 4 loops, one MI355X.

Headline step = one decode step of every rotated layer, run loop-major as a looped model
does (loop r over all layers before loop r+1): dense attention in loops 1-2, top-k
selection and the sparse splice in loops 3-4, each loop's call storing the new token's K/V
row of that loop in its BF16 tail, and, once every 64 steps, the 64-row tail flush, which
the attention calls of the step before the boundary moves encode in their own launches.
A selection reads only the previous loop's scores, so each sparse loop begins with one
select_columns call over all layers.  Eight distinct layer caches rotate so that no loop
finds its planes in the 256 MB last-level cache.  Steps are replayed from two captured HIP
graphs (with and without the fused flush); the context stays at n+1 columns.

Prints one JSON line.  `value` is microseconds per decode step of one layer (lower is
better), the flush charged at one step in 64.  `roofline` reports the kernel with the
largest share of the step, `rooflines` every kernel of the step, each against the 8 TB/s
HBM peak with counter traffic from the committed profiles; `extra` holds the other
workloads (4K context with appends and flushes, 32 loops, batch 8 with its bulk encode),
the codec variants, the token selection and the prefill-side sparse loop; `cpu_baseline`
times the fp64 oracle on a sample of the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak of the MI355X
COPY_BYTES = 1 << 30             # the calibration copy reads and writes this many bytes per launch
COPY_REPS = 8
CSRC = os.path.join(ROOT, "quantized_kv_attention_amd", "csrc")

# kernels whose counter traffic is committed under profiles/: key -> (file, kernel names, sources)
TRAFFIC = {
    "dense1": ("dense_reader_loop1_ctx32k_traffic.txt", ("dense_split_kernel", "dense_combine_kernel"),
               ("dense.hip", "common.h", "encode_group.h", "launch.h")),
    "dense2": ("dense_reader_loop2_ctx32k_traffic.txt", ("dense_split_kernel", "dense_combine_kernel"),
               ("dense.hip", "common.h", "encode_group.h", "launch.h")),
    "sparse3": ("sparse_gather_loop3_ctx32k_traffic.txt", ("sparse_chunk_kernel", "sparse_combine_kernel"),
                ("sparse.hip", "common.h", "encode_group.h", "launch.h")),
    "sparse4": ("sparse_gather_loop4_ctx32k_traffic.txt", ("sparse_chunk_kernel", "sparse_combine_kernel"),
                ("sparse.hip", "common.h", "encode_group.h", "launch.h")),
    "select": ("select_columns_ctx32k_traffic.txt", ("select_kernel",), ("select.hip", "common.h")),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="each oracle baseline (all cores, one core) runs decode steps for this long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the per-entry-point measurements")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads and components")
    ap.add_argument("--only", choices=["headline", "c1", "c3", "c4", "codecs", "tokens", "prefill", "shard"],
                    help="run one section only (for kernel traces)")
    ap.add_argument("--profile", choices=sorted(TRAFFIC), help="only launch one kernel family (counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain elementwise copy of 1 GiB (reference for the byte counters)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write a per-kernel table of the rocprofv3 kernel trace under DIR to --out")
    ap.add_argument("--summarize-inflight", nargs=2, metavar=("KEY", "DIR"),
                    help="from a rocprofv3 --pmc TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_RDREQ_sum GRBM_GUI_ACTIVE run of "
                         "--profile KEY: write the mean reads in flight and their latency to --out")
    ap.add_argument("--summarize-traffic", nargs=5, metavar=("KEY", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of --profile KEY and of "
                         "--copy-calibration): write the calibrated HBM bytes of that kernel family to --out")
    ap.add_argument("--out", help="output file of the summaries")
    ap.add_argument("--cmd", default="", help="command line recorded in a summary")
    return ap.parse_args()


def say(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------ setup ----
def dev_bf16(u16):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


class Rotation:
    """L distinct layer caches of one workload at context n + 1 (the decode position), with
    per-layer queries, new-token rows and the fused-flush arguments of the 64 oldest tail rows."""

    def __init__(self, w, L, codec=None, sparse_tight=False, seed=0):
        import numpy as np
        import torch

        import quantized_kv_attention_amd as qkv
        from quantized_kv_attention_amd import cache as qcache
        from quantized_kv_attention_amd import synth
        codec = codec or {}
        self.w, self.L, self.codec = w, L, codec
        n = w.n
        self.n_step = n + 1
        self.k = w.k_cols(self.n_step)
        self.cap = int(math.ceil((n + 128) / 64) * 64)
        self.nb = qkv.body_len(self.n_step)
        self.dense = [w.rho[r] >= 1.0 for r in range(w.R)]
        sb = None
        if sparse_tight:   # sparse planes sized for their rows (+ the flush group) instead of every position
            sb = [0 if self.dense[r] else int(math.ceil(w.rho[r] * n / 64)) + 3 for r in range(w.R)]
        self.layers = []
        for l in range(L):
            K, V, act = synth.gen_layer_torch(w, seed + l)
            c = qcache.LayerCache(w.B, w.H, w.d, w.R, self.cap, dense=self.dense, sparse_blocks=sb, **codec)
            c.prefill(K, V, act)
            del K, V
            qs = [dev_bf16(x) for x in synth.gen_queries(w, 1000 + l)]
            kn, vn = synth.gen_new_token(w, 1000 + l)
            kn = [dev_bf16(x) for x in kn]
            vn = [dev_bf16(x) for x in vn]
            c.act[:, :, n] = True
            flush, keep = [], []
            for r in range(w.R):
                if self.dense[r]:
                    flush.append(qkv.QkvFlush(self.nb, 0, None, None))
                else:
                    ap, na = c._active_lists(r, self.nb, self.nb + 64)
                    apd, nad = torch.from_numpy(ap).cuda(), torch.from_numpy(na).cuda()
                    keep += [apd, nad]
                    flush.append(qkv.QkvFlush(self.nb, 64, apd.data_ptr(), nad.data_ptr()))
            c.n_ctx = self.n_step
            self.layers.append(dict(c=c, q=qs, kn=kn, vn=vn, flush=flush, keep=keep, act=act))
            torch.cuda.synchronize()
        self.stack = qcache.LayerStack([ly["c"] for ly in self.layers], max_k=self.k)
        for ly, b in zip(self.layers, self.stack.layers):
            ly["b"] = b
        torch.cuda.empty_cache()

    def step(self, with_flush=False, stream=None):
        from quantized_kv_attention_amd import cache as qcache
        w = self.w
        for loop in range(1, w.R + 1):
            if loop > w.n_dense:
                self.stack.select(loop, self.k, stream)   # loop `loop`'s selections of every layer
            for ly in self.layers:
                qcache.decode_loop(ly["c"], ly["b"], loop, ly["q"][loop - 1], w.n_dense, self.k, stream=stream,
                                   selected=loop > w.n_dense, k_new=ly["kn"][loop - 1], v_new=ly["vn"][loop - 1],
                                   need_scores=qcache.scores_read_after(loop, w.n_dense, w.R),
                                   flush=ly["flush"][loop - 1] if with_flush else None)

    def bits(self):
        return self.layers[0]["c"].bits

    def step_bytes(self):
        """Algorithmic bytes of one layer-step (layer 0's masks and last selections), per loop,
        and of the fused 64-row flush of every loop."""
        import numpy as np
        from quantized_kv_attention_amd import bytes_model as bm
        from quantized_kv_attention_amd import cache as qcache
        w = self.w
        c0, b0, act0 = self.layers[0]["c"], self.layers[0]["b"], self.layers[0]["act"]
        nb, n_step, B, H, d = self.nb, self.n_step, w.B, w.H, w.d
        T = n_step - nb
        full = self.codec.get("full_state", False)
        bits = self.bits()
        rows, slots = [], []
        for r in range(w.R):
            per_b, sl = [], []
            for b in range(B):
                if self.dense[r]:
                    per_b.append(nb)
                    sl.append(np.arange(nb))
                else:
                    a = np.asarray(act0[r][b, :nb])
                    s = np.full(nb, -1, np.int64)
                    s[a] = np.arange(int(a.sum()))
                    per_b.append(int(a.sum()))
                    sl.append(s)
            rows.append(per_b)
            slots.append(sl)

        def planes_of(r):  # the planes loop r reads: 0..r, or from the last dense one (full state)
            first = max(p for p in range(r + 1) if self.dense[p]) if full else 0
            return list(range(first, r + 1))

        loop_bytes = []
        for r in range(w.R):
            lb = 0
            ps = planes_of(r)
            if r < w.n_dense:
                for b in range(B):
                    lb += H * bm.dense_loop_bytes([rows[p][b] for p in ps], T, n_step, d,
                                                  scores=qcache.scores_read_after(r + 1, w.n_dense, w.R),
                                                  bits_per_plane=[bits[p] for p in ps])
            else:
                idx_all = b0.selection(r + 1, self.k)[0].cpu().numpy()
                lb += B * H * bm.select_bytes(n_step, self.k)
                pv = sorted(set(planes_of(r)) | set(planes_of(r - 1)))
                for b in range(B):
                    for h in range(H):
                        lb += bm.sparse_loop_bytes(idx_all[b, h], [slots[p][b] for p in pv], nb, d,
                                                   scores=qcache.scores_read_after(r + 1, w.n_dense, w.R),
                                                   bits_per_plane=[bits[p] for p in pv])
            loop_bytes.append(lb)
        flush_loop = []
        for r in range(w.R):
            fb = 0
            for b in range(B):
                stored = 64 if self.dense[r] else int(np.asarray(act0[r][b, nb:nb + 64]).sum())
                fb += H * bm.encode_bytes(stored, d, r + 1, bits_per_plane=bits, full_state=full)
            flush_loop.append(fb)
        append = w.R * B * H * d * 2 * 2 * 2     # the new token's K/V rows read and stored in the tails
        full_chain = sum(H * bm.dense_loop_bytes([rows[p][b] for p in planes_of(w.R - 1)], T, n_step, d,
                                                 bits_per_plane=[bits[p] for p in planes_of(w.R - 1)])
                         for b in range(B))
        return loop_bytes, flush_loop, append, full_chain


def timed(fn, reps, stream=None):
    """Mean microseconds of fn() over reps back-to-back calls (HIP events on the stream)."""
    import torch
    s = stream or torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / reps


def row(us, nbytes, bound="hbm", **kw):
    gbps = nbytes / (us * 1e-6) / 1e9 if us > 0 else 0.0
    out = {"us": round(us, 2), "bytes": int(nbytes), "GBps": round(gbps, 1),
           "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "bound": bound}
    out.update(kw)
    return out


# ------------------------------------------------------------------------- headline ----
def headline(args, w):
    import numpy as np
    import torch

    t0 = time.time()
    rot = Rotation(w, args.layers)
    L = rot.L
    say(f"{L} layer caches of {rot.layers[0]['c'].nbytes() / 1e6:.1f} MB ready in {time.time() - t0:.1f}s "
        f"(n={rot.n_step}, k={rot.k})")
    if args.profile:
        profile_run(args, rot)
        return None
    # eager warm-up, then the two step variants as graphs
    rot.step(True)
    rot.step(False)
    torch.cuda.synchronize()
    g_plain, g_flush = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_plain):
        rot.step(False)
    with torch.cuda.graph(g_flush):
        rot.step(True)
    for _ in range(args.warmup):
        g_plain.replay()
    torch.cuda.synchronize()
    b0 = rot.layers[0]["b"]
    ref_o = b0.o_f32.clone()
    rot.step(False)
    torch.cuda.synchronize()
    eager_o = b0.o_f32.clone()
    g_plain.replay()
    torch.cuda.synchronize()
    assert torch.equal(eager_o, b0.o_f32) and torch.equal(ref_o, eager_o), "graph replay differs"
    g_flush.replay()
    torch.cuda.synchronize()
    assert torch.equal(ref_o, b0.o_f32), "the fused flush changed a result of its step"

    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record()
    for i in range(K):
        (g_flush if (i % 64) == 63 else g_plain).replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = e0.elapsed_time(e1)
    n_flush = sum(1 for i in range(K) if (i % 64) == 63)
    # the flush's surcharge, measured on its own (alternating replays), charged at 1 step in 64
    pf, pp = [], []
    for _ in range(6):
        pf.append(timed(g_flush.replay, 1))
        pp.append(timed(g_plain.replay, 1))
    surcharge_us = max(0.0, float(np.median(pf)) - float(np.median(pp)))
    charged_ms = total_ms + (K / 64.0 - n_flush) * surcharge_us / 1000.0
    us_step_layer = charged_ms * 1000.0 / (K * L)
    say(f"{K} steps x {L} layers: {total_ms:.2f} ms (wall {wall * 1e3:.2f} ms, {n_flush} with the flush); "
        f"flush surcharge {surcharge_us / L:.2f} us per layer-step at 1 in 64 -> {us_step_layer:.2f} us per layer-step")
    Ke = min(K, 16)
    eager_us = timed(lambda: rot.step(False), Ke) / L
    say(f"eager (no graph), {Ke} steps without the flush: {eager_us:.2f} us per layer-step")
    ceiling = read_ceiling()

    loop_bytes, flush_loop, append_bytes, full_chain = rot.step_bytes()
    step_bytes = sum(loop_bytes) + append_bytes + sum(flush_loop) / 64.0
    gbps_step = step_bytes / (us_step_layer * 1e-6) / 1e9

    rows = None if args.no_rows else measure_rows(rot, loop_bytes, flush_loop, append_bytes, full_chain)
    rl, dominant = rooflines(rows, loop_bytes, w, rot)
    out = {
        "value": round(us_step_layer, 3), "steps": K, "ms_per_step": round(charged_ms / K, 4),
        "config": {"workload": f"ctx32k: batch {w.B}, {w.H} heads x {w.d}, context {rot.n_step}, {w.R} loops, "
                               f"token retention {w.rho}, {int(w.k_frac * 100)}% key columns in loops "
                               f"{w.n_dense + 1}-{w.R}, INT4 g64 + fp32 scale/zero, 64-token BF16 tail",
                   "layers_rotated": L, "k_columns": rot.k,
                   "step": "R-loop attention, each loop's call storing the new token's tail row; the 64-row flush "
                           "encoded inside the attention calls of one step in 64 (charged at 1/64 when fewer timed)",
                   "selection": f"one call per sparse loop for all {L} layers",
                   "value_is": "microseconds per decode step of one layer"},
        "flush_surcharge_us_per_layer_step": round(surcharge_us / L, 3),
        "eager_us_per_layer_step": round(eager_us, 3),
        "read_ceiling": ceiling,
        "hbm_GBps_step": round(gbps_step, 1),
        "pct_peak_step": round(100 * gbps_step / HBM_PEAK_GBPS, 2),
        "bytes_per_layer_step": int(step_bytes),
        "bytes_per_loop": [int(x) for x in loop_bytes],
        "roofline": dominant,
        "rooflines": rl,
        "rows": rows,
    }
    del g_plain, g_flush, rot
    torch.cuda.empty_cache()
    return out


def measure_rows(rot, loop_bytes, flush_loop, append_bytes, full_chain):
    """Each entry point of the path timed on its own (events around back-to-back calls over
    the rotated layers), with its algorithmic bytes and the fraction of the HBM peak."""
    import torch

    import quantized_kv_attention_amd as qkv
    from quantized_kv_attention_amd import bytes_model as bm
    from quantized_kv_attention_amd import cache as qcache
    w, layers, stack, k, L = rot.w, rot.layers, rot.stack, rot.k, rot.L
    s = torch.cuda.current_stream()
    n1 = rot.n_step
    out = {}
    sel_b = w.B * w.H * bm.select_bytes(n1, k)

    def call(ly, loop, flush=False, scores=True):
        b = ly["b"]
        fl = ly["flush"][loop - 1] if flush else None
        if loop <= w.n_dense:
            qkv.attn_decode_dense(ly["c"], loop, ly["q"][loop - 1], 1.0, b.o[loop - 1], b.o_f32[loop - 1],
                                  b.scores if scores else None, b.lse, b.ws, s, flush=fl)
        else:
            idx, ps, mass = b.selection(loop, k)
            qkv.attn_decode_sparse(ly["c"], loop, ly["q"][loop - 1], 1.0, idx, ps, mass, k, b.o_f32[loop - 2], b.lse,
                                   b.scores if scores else None, b.o[loop - 1], b.o_f32[loop - 1], b.ws, s, flush=fl)

    rot.step(False)
    torch.cuda.synchronize()
    for loop in range(1, w.R + 1):
        need = qcache.scores_read_after(loop, w.n_dense, w.R)
        if loop <= w.n_dense:
            t = timed(lambda: [call(ly, loop, scores=need) for ly in layers], 5) / L
            out[f"attn_decode_dense loop {loop}"] = row(t, loop_bytes[loop - 1], calls_timed=5 * L)
        else:
            t = timed(lambda: [qkv.select_columns(ly["b"].scores, ly["b"].lse, n1, k,
                                                  *ly["b"].selection(loop, k), None, s) for ly in layers], 4) / L
            out[f"select_columns loop {loop} (one call per layer)"] = row(t, sel_b, "latency")
            t = timed(lambda: stack.select(loop, k, s), 8) / L
            out[f"select_columns loop {loop} ({L} layers per call)"] = row(t, sel_b, "latency")
            t = timed(lambda: [call(ly, loop, scores=need) for ly in layers], 5) / L
            out[f"attn_decode_sparse loop {loop}"] = row(t, loop_bytes[loop - 1] - sel_b, calls_timed=5 * L)
        # the same call carrying its loop's part of the fused 64-row flush
        tf = timed(lambda: [call(ly, loop, flush=True, scores=need) for ly in layers], 3) / L
        base = out[f"attn_decode_{'dense' if loop <= w.n_dense else 'sparse'} loop {loop}"]["us"]
        out[f"fused flush in the loop-{loop} call (surcharge)"] = row(max(0.0, tf - base), flush_loop[loop - 1],
                                                                      "latency")
    R = w.R
    t = timed(lambda: [qkv.attn_decode_dense(ly["c"], R, ly["q"][R - 1], 1.0, ly["b"].o[R - 1], ly["b"].o_f32[R - 1],
                                             ly["b"].scores, ly["b"].lse, ly["b"].ws, s) for ly in layers], 3) / L
    out[f"attn_decode_dense loop {R} (full chain, for comparison)"] = row(t, full_chain)
    rows_kv = [(torch.stack([x.view(w.B, w.H, 1, w.d) for x in ly["kn"]]),
                torch.stack([x.view(w.B, w.H, 1, w.d) for x in ly["vn"]])) for ly in layers]   # built untimed
    t = timed(lambda: [qkv.kv_append_tail(ly["c"], 0, rot.n_step - 1, kv[0], kv[1], s)
                       for ly, kv in zip(layers, rows_kv)], 3) / L
    out["kv_append_tail (all loops; the step stores rows inside the attention calls)"] = row(t, append_bytes, "latency")
    for r in range(w.R):
        def fl(ly, r=r):
            c = ly["c"]
            f = ly["flush"][r]
            if rot.dense[r]:
                qkv.kv_encode_loop(c, r + 1, rot.nb, 64, stream=s)
            else:
                ap, na = ly["keep"][2 * (r - w.n_dense)], ly["keep"][2 * (r - w.n_dense) + 1]
                qkv.kv_encode_loop(c, r + 1, rot.nb, 64, ap, na, stream=s)
        t = timed(lambda: [fl(ly) for ly in layers], 3) / L
        out[f"kv_encode_loop flush loop {r + 1} (separate launch, for comparison)"] = row(t, flush_loop[r], "latency")
    for name, v in out.items():
        say(f"{name:58s} {v['us']:9.2f} us  {v['bytes'] / 1e6:8.2f} MB  {v['GBps']:8.1f} GB/s")
    return out


def rooflines(rows, loop_bytes, w, rot):
    """Per kernel family of the step: bytes per launch, mean launch time, fraction of the HBM
    peak, counter traffic; and the family with the largest share of the step."""
    if rows is None:
        return None, None
    out = []

    def entry(key, name, us, nbytes, share):
        ach = nbytes / (us * 1e-6) / 1e9
        tr = read_traffic(key)
        e = {"bound": "hbm", "kernel": name, "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": tr, "bytes_per_launch": int(nbytes),
             "mean_launch_us": round(us, 3), "share_us_per_layer_step": round(share, 3),
             "timing": "HIP events around 5 x 8 back-to-back calls (one call = both kernels)"}
        if tr:
            e["traffic_over_algorithmic"] = round(tr / nbytes, 3)
        out.append(e)
        return e

    d1 = rows["attn_decode_dense loop 1"]
    d2 = rows["attn_decode_dense loop 2"]
    entry("dense1", "dense_split_kernel<128,1> + dense_combine_kernel<128> (loop 1: base plane)", d1["us"],
          d1["bytes"], d1["us"])
    entry("dense2", "dense_split_kernel<128,2> + dense_combine_kernel<128> (loop 2: base + residual plane)",
          d2["us"], d2["bytes"], d2["us"])
    s3, s4 = rows["attn_decode_sparse loop 3"], rows["attn_decode_sparse loop 4"]
    entry("sparse3", "sparse_chunk_kernel<128> + sparse_combine_kernel<128> (loop 3)", s3["us"], s3["bytes"],
          s3["us"])
    entry("sparse4", "sparse_chunk_kernel<128> + sparse_combine_kernel<128> (loop 4)", s4["us"], s4["bytes"],
          s4["us"])
    sel = [v for k_, v in rows.items() if k_.startswith("select_columns") and "layers per call" in k_]
    if sel:   # one launch selects for every rotated layer
        e = entry("select", f"select_kernel (one launch for {rot.L} layers)", sel[0]["us"] * rot.L,
                  sel[0]["bytes"] * rot.L, sum(v["us"] for v in sel))
        e["bound"] = "latency"
    # the step's largest share: the sparse gather runs twice (loops 3 and 4)
    fams = {"dense_split_kernel<128,2> (loop 2)": (d2["us"], d2["bytes"], "dense2", d2["us"]),
            "dense_split_kernel<128,1> (loop 1)": (d1["us"], d1["bytes"], "dense1", d1["us"]),
            "sparse_chunk_kernel<128> (loops 3 and 4)": ((s3["us"] + s4["us"]) / 2, (s3["bytes"] + s4["bytes"]) / 2,
                                                          None, s3["us"] + s4["us"])}
    name, (us, nbytes, key, share) = max(fams.items(), key=lambda kv: kv[1][3])
    if key is None:
        t3, t4 = read_traffic("sparse3"), read_traffic("sparse4")
        tr = (t3 + t4) / 2 if (t3 and t4) else None
    else:
        tr = read_traffic(key)
    ach = nbytes / (us * 1e-6) / 1e9
    dom = {"bound": "hbm", "kernel": name + " + its combine kernel", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
           "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": int(tr) if tr else None,
           "bytes_per_launch": int(nbytes), "mean_launch_us": round(us, 3),
           "share_us_per_layer_step": round(share, 3),
           "timing": "HIP events around 5 x 8 back-to-back calls on the calls' stream"}
    return out, dom


def read_ceiling():
    """A read-only reference on the same device: the library's plain streaming read of 2 GiB."""
    import torch
    import quantized_kv_attention_amd as qkv
    x = torch.zeros(1 << 31, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(qkv.STREAM_READ_GROUPS, dtype=torch.int32, device="cuda")
    us = timed(lambda: qkv.stream_read(x, sink), 10)
    gbps = x.numel() / (us * 1e-6) / 1e9
    del x, sink
    torch.cuda.empty_cache()
    say(f"read ceiling (plain streaming read of 2 GiB): {gbps:.0f} GB/s")
    return {"GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "how": "qkv_stream_read over 2 GiB, HIP events around 10 calls"}


def profile_run(args, rot):
    """For counter runs: one warm-up step of every loop (the sparse calls need its scores and
    selections), then warmup + steps calls of one kernel family over the layers."""
    import torch
    import quantized_kv_attention_amd as qkv
    w, s = rot.w, torch.cuda.current_stream()
    rot.step(False)
    torch.cuda.synchronize()
    key = args.profile
    for _ in range(args.warmup + args.steps):
        for ly in rot.layers:
            b = ly["b"]
            if key in ("dense1", "dense2"):
                loop = 1 if key == "dense1" else 2
                qkv.attn_decode_dense(ly["c"], loop, ly["q"][loop - 1], 1.0, b.o[loop - 1], b.o_f32[loop - 1],
                                      b.scores if loop == 2 else None, b.lse, b.ws, s)
            elif key in ("sparse3", "sparse4"):
                loop = int(key[-1])
                idx, ps, mass = b.selection(loop, rot.k)
                qkv.attn_decode_sparse(ly["c"], loop, ly["q"][loop - 1], 1.0, idx, ps, mass, rot.k, b.o_f32[loop - 2],
                                       b.lse, b.scores if loop < w.R else None, b.o[loop - 1], b.o_f32[loop - 1],
                                       b.ws, s)
        if key == "select":
            rot.stack.select(3, rot.k, s)
    torch.cuda.synchronize()
    say(f"profiling run of {key} done")


# ----------------------------------------------------------------------- other rows ----
def extra_c1(args):
    """4K context, 64 decode steps with appends and the fused flush (context grows each step,
    so the steps are launched eagerly), 8 rotated layers."""
    import torch

    from quantized_kv_attention_amd import cache as qcache
    from quantized_kv_attention_amd import synth
    w = synth.WORKLOADS["ctx4k"]
    L = 8
    caps = int(math.ceil((w.n + 64 + 128) / 64) * 64)
    caches, kns = [], []
    for l in range(L):
        K, V, act = synth.gen_layer_torch(w, 200 + l)
        c = qcache.LayerCache(w.B, w.H, w.d, w.R, caps)
        c.prefill(K, V, act)
        caches.append(c)
    stack = qcache.LayerStack(caches, max_k=w.k_cols(w.n + 64))
    toks = []
    for step in range(64):
        kn, vn = synth.gen_new_token(w, step)
        q = [dev_bf16(x) for x in synth.gen_queries(w, step)]
        toks.append(([dev_bf16(x) for x in kn], [dev_bf16(x) for x in vn], q))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flushes = 0
    e0.record()
    for step in range(64):
        kn, vn, q = toks[step]
        for c in caches:
            c.advance_token()
        flushes += caches[0].tail_full()
        k = w.k_cols(caches[0].n_ctx)
        qcache.decode_step_stack(stack, [q] * L, w.n_dense, k, k_new=[kn] * L, v_new=[vn] * L, fused_flush=True)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / (64 * L)
    say(f"ctx4k: 64 decode steps x {L} layers with appends and {flushes} fused flush(es): {us:.2f} us per layer-step")
    return {"workload": f"ctx4k: batch 1, 16 heads x 128, context 4096 -> 4160, 4 loops, 64 decode steps, "
                        f"{L} layers, eager launches", "us_per_layer_step": round(us, 2), "flushes": int(flushes)}


def graph_step_row(rot, reps=10):
    import torch
    rot.step(False)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rot.step(False)
    g.replay()
    us = timed(g.replay, reps) / rot.L
    loop_bytes, flush_loop, append_bytes, _ = rot.step_bytes()
    nbytes = sum(loop_bytes) + append_bytes
    del g
    return us, nbytes, loop_bytes


def extra_shard(args):
    """One GPU's share of the 32K step when the 16 heads are sharded over 8 GPUs: 2 heads x 128
    at 32K, 8 rotated layers, graph replay, flush not included.  The kernels are the same; the
    dense plan sizes its splits for the smaller head count."""
    import dataclasses

    from quantized_kv_attention_amd import synth
    w = dataclasses.replace(synth.WORKLOADS["ctx32k"], H=2)
    rot = Rotation(w, 8, seed=600)
    us, nbytes, lb = graph_step_row(rot)
    say(f"shard (2 heads x 32K): {us:.1f} us per layer-step ({nbytes / 1e6:.1f} MB, {nbytes / us / 1e3:.0f} GB/s)")
    loop_bytes, flush_loop, append_bytes, full_chain = rot.step_bytes()
    rows = measure_rows(rot, loop_bytes, flush_loop, append_bytes, full_chain)
    keep = {k_: v for k_, v in rows.items() if k_.startswith("attn_decode_") and "flush" not in k_}
    for k_, v in keep.items():
        say(f"  shard {k_}: {v['us']:.2f} us ({v['GBps']:.0f} GB/s)")
    out = row(us, nbytes, bytes_per_loop=[int(x) for x in lb], calls=keep,
              workload="2 heads x 128 at 32K (one GPU's share of 16 heads over 8 GPUs), 8 rotated layers, "
                       "graph replay, flush not included")
    del rot
    return out


def extra_c3(args):
    """40 heads x 128, 8K context, 32 loops (2 dense + 30 sparse loops over the full chain)."""
    from quantized_kv_attention_amd import synth
    w = synth.WORKLOADS["deep32"]
    rot = Rotation(w, 2, sparse_tight=True, seed=300)
    us, nbytes, lb = graph_step_row(rot)
    say(f"deep32: {us:.1f} us per layer-step ({nbytes / 1e6:.1f} MB, {nbytes / us / 1e3:.0f} GB/s)")
    out = row(us, nbytes, workload="deep32: batch 1, 40 heads x 128, context 8193, 32 loops, 10% rows and "
                                   "10% columns from loop 3, 2 rotated layers, graph replay")
    del rot
    return out


def extra_c4(args):
    """8 sequences x 16 heads x 128, 16K context each: the bulk encode of all 4 loops from the
    prompt, then 128 decode steps with appends and fused flushes."""
    import numpy as np
    import torch

    import quantized_kv_attention_amd as qkv
    from quantized_kv_attention_amd import bytes_model as bm
    from quantized_kv_attention_amd import cache as qcache
    from quantized_kv_attention_amd import synth
    w = synth.WORKLOADS["batch8"]
    n = w.n
    cap = int(math.ceil((n + 128 + 128) / 64) * 64)
    K, V, act = synth.gen_layer_torch(w, 400)
    nb = qkv.body_len(n)
    c = qcache.LayerCache(w.B, w.H, w.d, w.R, cap)
    for r in range(w.R):
        c.act[r, :, :n] = np.asarray(act[r])
    calls = []
    for r in range(w.R):
        if r < w.n_dense:
            calls.append((r, None, None, K[r][:, :, :nb].contiguous(), V[r][:, :, :nb].contiguous()))
        else:
            ap, na = c._active_lists(r, 0, nb)
            ks = torch.zeros((w.B, w.H, nb, w.d), dtype=torch.bfloat16, device="cuda")
            vs = torch.zeros_like(ks)
            for b in range(w.B):
                cnt = int(na[b])
                rr = torch.from_numpy(ap[b, :cnt].astype(np.int64)).cuda()
                ks[b, :, :cnt] = K[r][b].index_select(1, rr)
                vs[b, :, :cnt] = V[r][b].index_select(1, rr)
            calls.append((r, torch.from_numpy(ap).cuda(), torch.from_numpy(na).cuda(), ks, vs))
    torch.cuda.synchronize()
    enc = {}
    total_us, total_b = 0.0, 0
    for r, ap, na, ks, vs in calls:
        us = timed(lambda: qkv.kv_encode_loop(c, r + 1, 0, nb, ap, na, ks, vs), 3)
        stored = [nb if r < w.n_dense else int(np.asarray(act[r][b, :nb]).sum()) for b in range(w.B)]
        nbytes = sum(w.H * bm.encode_bytes(st, w.d, r + 1) for st in stored)
        enc[f"loop {r + 1}"] = row(us, nbytes)
        total_us += us
        total_b += nbytes
    for r in range(w.R):
        qkv.kv_append_tail(c, r + 1, nb, K[r][:, :, nb:n].contiguous(), V[r][:, :, nb:n].contiguous())
    c.n_ctx = n
    del K, V, calls
    torch.cuda.empty_cache()
    bufs = qcache.DecodeBuffers(c, max_k=w.k_cols(n + 128))
    toks = []
    for step in range(128):
        kn, vn = synth.gen_new_token(w, step)
        toks.append(([dev_bf16(x) for x in kn], [dev_bf16(x) for x in vn],
                     [dev_bf16(x) for x in synth.gen_queries(w, step)]))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    flushes = 0
    e0.record()
    for step in range(128):
        kn, vn, q = toks[step]
        c.advance_token()
        flushes += c.tail_full()
        qcache.decode_step(c, bufs, q, w.n_dense, w.k_cols(c.n_ctx), k_new=kn, v_new=vn, fused_flush=True)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / 128
    say(f"batch8: bulk encode {total_b / 1e6:.0f} MB in {total_us:.0f} us ({total_b / total_us / 1e3:.0f} GB/s); "
        f"128 decode steps {us:.1f} us per step ({flushes} fused flushes)")
    del c, bufs
    torch.cuda.empty_cache()
    return {"workload": "batch8: 8 sequences x 16 heads x 128, context 16384 (+128 generated), 4 loops, one layer",
            "bulk_encode": row(total_us, total_b, loops=enc),
            "decode_us_per_step": round(us, 2), "decode_steps": 128, "flushes": int(flushes),
            "decode_note": "eager launches (the context grows each step), appends in the attention calls"}


def extra_codecs(args):
    """The 32K step with the codec variants: 2-bit residual planes, per-loop full-state INT4."""
    from quantized_kv_attention_amd import synth
    w = synth.WORKLOADS["ctx32k"]
    out = {}
    for name, codec in (("int2_residual", dict(residual_bits=2)), ("full_state_int4", dict(full_state=True))):
        rot = Rotation(w, 4, codec=codec, seed=500)
        us, nbytes, lb = graph_step_row(rot)
        say(f"ctx32k {name}: {us:.1f} us per layer-step ({nbytes / 1e6:.1f} MB, {nbytes / us / 1e3:.0f} GB/s)")
        out[name] = row(us, nbytes, bytes_per_loop=[int(x) for x in lb],
                        workload=f"ctx32k with {codec}, 4 rotated layers, graph replay, flush not included")
        del rot
    return out


def extra_tokens(args):
    """select_tokens at 32K tokens, hidden width 2048: loop 3 (every token ranked) and loop 4
    (loop 3's active set ranked)."""
    import numpy as np
    import torch

    import quantized_kv_attention_amd as qkv
    from quantized_kv_attention_amd import bytes_model as bm
    n, dm = 32768, 2048
    g = torch.Generator(device="cuda").manual_seed(7)
    h0 = torch.randn((1, n, dm), generator=g, device="cuda").to(torch.bfloat16)
    gt = torch.exp(1.5 * torch.randn((1, n, 1), generator=g, device="cuda"))
    h1 = (h0.float() + 0.3 * gt * torch.randn((1, n, dm), generator=g, device="cuda")).to(torch.bfloat16)
    h2 = (h1.float() + 0.1 * gt * torch.randn((1, n, dm), generator=g, device="cuda")).to(torch.bfloat16)
    k3, k4 = math.ceil(0.25 * n), math.ceil(0.10 * n)
    score = torch.zeros((1, n), dtype=torch.float32, device="cuda")
    a3 = torch.zeros((1, k3), dtype=torch.int32, device="cuda")
    a4 = torch.zeros((1, k4), dtype=torch.int32, device="cuda")
    n3 = torch.zeros(1, dtype=torch.int32, device="cuda")
    n4 = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(qkv.token_workspace_bytes(1, k3), dtype=torch.uint8, device="cuda")
    t3 = timed(lambda: qkv.select_tokens(h1, h0, n, k3, score, a3, n3, ws), 10)
    t4 = timed(lambda: qkv.select_tokens(h2, h1, n, k4, score, a4, n4, ws, act_prev=a3, n_act_prev=n3), 10)
    b3, b4 = bm.token_select_bytes(n, n, dm, k3), bm.token_select_bytes(k3, n, dm, k4)
    say(f"select_tokens 32K x {dm}: loop 3 {t3:.1f} us, loop 4 {t4:.1f} us")
    del h0, h1, h2
    torch.cuda.empty_cache()
    return {"workload": f"one sequence, {n} tokens, hidden width {dm}, keep 25% then 10% (nested)",
            "loop3": row(t3, b3, kept=k3), "loop4": row(t4, b4, kept=k4)}


def extra_prefill(args):
    """attn_prefill_sparse at the 32K prompt: loop 3's 8192 active rows against 3277 selected
    columns per head, 16 heads x 128 (with the gathers that build its compact buffers)."""
    import numpy as np
    import torch

    import quantized_kv_attention_amd as qkv
    from quantized_kv_attention_amd import bytes_model as bm
    from quantized_kv_attention_amd import synth
    w = synth.WORKLOADS["ctx32k"]
    n, H, d = w.n, w.H, w.d
    act = synth.gen_masks(w, n)
    qpos = np.nonzero(act[2][0])[0].astype(np.int32)[None]
    nq = qpos.shape[1]
    k = w.k_cols(n)
    cpos = np.stack([synth.gen_columns(w, n, k, 0, h) for h in range(H)])[None]
    g = torch.Generator(device="cuda").manual_seed(11)
    full = [(torch.randn((1, H, n, d), generator=g, device="cuda") * s).to(torch.bfloat16)
            for s in (0.09, 0.09, 1.0, 1.0, 1.0, 1.0)]   # q, q0, k, k0, v, v0
    qp, cp = torch.from_numpy(qpos).cuda(), torch.from_numpy(cpos).cuda()
    lse0 = torch.log(qp.float() + 1.0).view(1, 1, nq).expand(1, H, nq).contiguous()
    o0 = torch.randn((1, H, nq, d), generator=g, device="cuda") * 0.3
    o32 = torch.zeros_like(o0)
    o16 = torch.zeros((1, H, nq, d), dtype=torch.bfloat16, device="cuda")
    mass = torch.zeros((1, H, nq), device="cuda")
    bufs = {}

    def gather():
        bufs["q"] = qkv.gather_rows(full[0], qp)
        bufs["q0"] = qkv.gather_rows(full[1], qp)
        bufs["k"] = qkv.gather_rows(full[2], cp)
        bufs["k0"] = qkv.gather_rows(full[3], cp)
        bufs["vt"] = qkv.gather_rows(full[4], cp, transpose=True)
        bufs["v0t"] = qkv.gather_rows(full[5], cp, transpose=True)

    tg = timed(gather, 5)

    def attend():
        qkv.attn_prefill_sparse(bufs["q"], bufs["q0"], qp, lse0, o0, bufs["k"], bufs["k0"], bufs["vt"], bufs["v0t"],
                                cp, 1.0, o32, o16, mass)

    ta = timed(attend, 5)
    flops = sum(bm.prefill_sparse_flops(qpos[0], cpos[0, h], d) for h in range(H))
    nbytes = H * bm.prefill_sparse_bytes(nq, k, d)
    gather_bytes = H * (2 * nq * d * 2 * 2 + 4 * k * d * 2 * 2)
    tf = flops / (ta * 1e-6) / 1e12
    say(f"prefill 32K loop 3: gathers {tg:.1f} us, attention {ta:.1f} us = {tf:.1f} TFLOP/s "
        f"({tf / MFMA_BF16_PEAK_TFLOPS:.3f} of the bf16 MFMA peak)")
    del full, bufs
    torch.cuda.empty_cache()
    return {"workload": f"32K prompt, loop 3: {nq} active rows x {k} selected columns per head, {H} heads x {d}",
            "attention": {"us": round(ta, 2), "flops": int(flops), "TFLOPs": round(tf, 2),
                          "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)},
                          "bytes": int(nbytes), "GBps": round(nbytes / (ta * 1e-6) / 1e9, 1)},
            "gathers": row(tg, gather_bytes, note="six kv_gather_rows calls (queries and keys of two loops, "
                                                  "transposed values of two loops)")}


# ------------------------------------------------------------------------ CPU side ----
def cpu_info():
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        nproc = int(subprocess.run(["nproc"], capture_output=True, text=True).stdout.strip())
    except (OSError, ValueError):
        nproc = os.cpu_count() or 1
    return model, nproc


def cpu_baseline(w, seconds):
    """The fp64 oracle on every head of the headline workload: decode steps (every loop), each
    head first rebuilding its keys and values from the stored planes (the chain
    dequantisation), until `seconds` of wall time have passed; once on every host core (one
    thread per head, up to the core count) and once on one core.  The cache build is not
    timed."""
    import oracle as orc
    from quantized_kv_attention_amd import synth

    model, nproc = cpu_info()
    hs = list(range(w.H))
    K, V, act = synth.gen_layer(w, heads=hs)
    oc = orc.OracleCache(w.B, len(hs), w.d, w.R, w.n + 128)
    oc.prefill(K, V, act)
    del K, V
    kn, vn = synth.gen_new_token(w, 1000, heads=hs)
    oc.append(kn, vn)
    k = w.k_cols(oc.n)
    runs = {}
    for label, threads in (("all_cores", max(1, min(nproc, len(hs) * w.B))), ("one_core", 1)):
        steps = 0
        t0 = time.perf_counter()
        while True:
            oc.step(synth.gen_queries(w, 2000 + steps, heads=hs), w.n_dense, k, threads=threads, from_planes=True)
            steps += 1
            dt = time.perf_counter() - t0
            if dt >= seconds:
                break
        runs[label] = (dt / steps * 1e6, threads, steps, dt)
        say(f"oracle baseline ({label}, {threads} threads): {dt / steps * 1e3:.1f} ms per step over {steps} steps")
    us_all, thr, steps, dt = runs["all_cores"]
    us_one = runs["one_core"][0]
    return {"value": round(us_all, 1), "unit": "us/step", "cores": thr, "kind": "oracle",
            "sample": f"all {w.H} heads x {steps} decode steps (all {w.R} loops, context {oc.n}, keys and values "
                      f"rebuilt from the stored planes each step), {dt:.1f} s wall on {thr} threads",
            "single_core_us_per_step": round(us_one, 1), "host_nproc": nproc, "host_cpu": model,
            "note": "a correctness reference, not a tuned CPU implementation"}


# ---------------------------------------------------------------------- summaries ----
def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(key):
    """HBM bytes per launch of a kernel family from its committed counter summary, or None
    when the summary is missing or was taken on another version of the kernel source."""
    fname, _, srcs = TRAFFIC[key]
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "|")):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_hash") != source_hash(srcs):
        return None
    try:
        return int(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _rocprof_db(d):
    import glob
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {d}")
    return sqlite3.connect(dbs[0])


def _short(name):
    """Kernel name without its trailing parameter list."""
    name = name.strip()
    if name.endswith(")"):
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                return name[:i].strip()
    return name


def summarize_trace(args):
    """Per-kernel launch count and durations of a `rocprofv3 --kernel-trace --stats` run."""
    con = _rocprof_db(args.summarize_trace)
    rows = list(con.execute("select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
                            "from kernels group by name order by sum(duration) desc"))
    tot = sum(r[5] for r in rows) or 1
    lines = ["# rocprofv3 kernel trace summary", f"command: {args.cmd}", "",
             "| kernel | launches | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for name, cnt, avg, mn, mx, sm in rows:
        lines.append(f"| {_short(name)[:100]} | {cnt} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | "
                     f"{100 * sm / tot:.1f}% |")
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_per_dispatch(d, counter, names, last=None):
    """Mean counter value per dispatch of each kernel name (substring), over its `last`
    dispatches in dispatch order when given (the profiled calls come after a warm-up step
    whose dispatches of the same kernel, e.g. another loop's, must not enter the mean)."""
    con = _rocprof_db(d)
    vals = {}
    for name, did, cn, cv in con.execute("select name, dispatch_id, counter_name, counter_value from pmc_events"):
        if cn != counter:
            continue
        for k in names:
            if k in name:
                vals.setdefault(k, []).append((int(did), float(cv)))
    out = {}
    for k, v in vals.items():
        v.sort()
        if last:
            v = v[-last:]
        out[k] = (sum(x for _, x in v) / len(v), len(v))
    return out


# Dispatches of each kernel of a family that `--profile <key> --steps 2 --warmup 1` makes
# after its warm-up step: (1 + 2) calls over the 8 rotated layers, or 1 + 2 selections.
PROFILE_STEPS, PROFILE_WARMUP = 2, 1


def profiled_dispatches(key, layers=8):
    return (PROFILE_STEPS + PROFILE_WARMUP) * (1 if key == "select" else layers)


def summarize_traffic(args):
    """Calibrated HBM bytes per launch of one kernel family (its kernels summed): FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch) scaled by what the same counters read for a plain
    elementwise copy that reads and writes COPY_BYTES each."""
    key, fdir, wdir, cfdir, cwdir = args.summarize_traffic
    fname, kernels, srcs = TRAFFIC[key]
    cf = _counter_per_dispatch(cfdir, "FETCH_SIZE", ("neg",)).get("neg")
    cw = _counter_per_dispatch(cwdir, "WRITE_SIZE", ("neg",)).get("neg")
    if not cf or not cw:
        raise SystemExit("copy calibration dispatches not found")
    f_fac = COPY_BYTES / (cf[0] * 1024.0)
    w_fac = COPY_BYTES / (cw[0] * 1024.0)
    n_last = profiled_dispatches(key)
    fe = _counter_per_dispatch(fdir, "FETCH_SIZE", kernels, n_last)
    wr = _counter_per_dispatch(wdir, "WRITE_SIZE", kernels, n_last)
    rd = sum(fe[k][0] for k in fe) * 1024.0 * f_fac
    wt = sum(wr[k][0] for k in wr) * 1024.0 * w_fac
    lines = [f"# HBM traffic of {key} at 32K context (16 heads x 128; one launch = {' + '.join(kernels)})",
             f"command: {args.cmd}", "",
             "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | dispatches |", "|---|---|---|---|"]
    for k in kernels:
        lines.append(f"| {k} | {fe.get(k, (0, 0))[0]:.1f} | {wr.get(k, (0, 0))[0]:.1f} | {fe.get(k, (0, 0))[1]} |")
    lines += ["", f"| copy of {COPY_BYTES} B | {cf[0]:.1f} | {cw[0]:.1f} | {cf[1]} |", "",
              f"fetch_factor: {f_fac:.4f}", f"write_factor: {w_fac:.4f}",
              f"read_bytes_per_launch: {int(rd)}", f"write_bytes_per_launch: {int(wt)}",
              f"hbm_bytes_per_launch: {int(rd + wt)}", f"kernel_source_hash: {source_hash(srcs)}"]
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_inflight(args):
    """Reads in flight and their latency for the main kernel of a family, from one
    `rocprofv3 --pmc TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_RDREQ_sum GRBM_GUI_ACTIVE` run of
    `--profile <key>`: LEVEL accumulates the outstanding 128-byte reads every cycle, so
    LEVEL / active cycles is the mean number in flight and LEVEL / requests their mean
    latency in cycles."""
    key, d = args.summarize_inflight
    fname, kernels, srcs = TRAFFIC[key]
    main_k = kernels[0]
    con = _rocprof_db(d)
    per = {}
    for name, did, cn, cv in con.execute("select name, dispatch_id, counter_name, counter_value from pmc_events"):
        if main_k in name:
            per.setdefault(int(did), {}).setdefault(cn, []).append(float(cv))
    dids = sorted(per)[-profiled_dispatches(key):]
    lvl = [sum(per[i]["TCC_EA0_RDREQ_LEVEL_sum"]) for i in dids]
    req = [sum(per[i]["TCC_EA0_RDREQ_sum"]) for i in dids]
    act = [max(per[i]["GRBM_GUI_ACTIVE"]) for i in dids]   # the slowest XCD: the dispatch's span
    mean = lambda v: sum(v) / len(v)
    inflight = mean([a / b for a, b in zip(lvl, act)])
    latency = mean([a / b for a, b in zip(lvl, req)])
    lines = [f"# Reads in flight of {main_k} ({key}) at 32K context (16 heads x 128)",
             f"command: {args.cmd}", "",
             "| dispatches | 128-B read requests / dispatch | active cycles / dispatch | reads in flight (mean) | "
             "read latency (cycles, mean) |", "|---|---|---|---|---|",
             f"| {len(dids)} | {mean(req):.0f} | {mean(act):.0f} | {inflight:.0f} | {latency:.0f} |", "",
             f"kernel_source_hash: {source_hash(srcs)}"]
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# --------------------------------------------------------------------------- main ----
def main():
    args = parse()
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_traffic:
        return summarize_traffic(args)
    if args.summarize_inflight:
        return summarize_inflight(args)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by head with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_kv_attention_amd import synth

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(COPY_REPS):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        say(f"copy calibration: {COPY_REPS} x neg over {COPY_BYTES} B")
        return
    w = synth.WORKLOADS["ctx32k"]
    sections = {"c1": extra_c1, "c3": extra_c3, "c4": extra_c4, "codecs": extra_codecs, "tokens": extra_tokens,
                "prefill": extra_prefill, "shard": extra_shard}
    if args.only and args.only != "headline":
        res = sections[args.only](args)
        print(json.dumps({"section": args.only, "result": res}), flush=True)
        return
    head = headline(args, w)
    if head is None:   # profiling run
        return
    extra = None
    if not args.no_extra and args.only is None:
        extra = {}
        for name, fn in sections.items():
            extra[name] = fn(args)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds)
    out = {
        "metric": "decode-attn us/step & achieved HBM GB/s (% peak), 32K ctx, 4 loops, 1 GPU",
        "value": head["value"],
        "unit": "us/step",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
    }
    for key in ("config", "flush_surcharge_us_per_layer_step", "eager_us_per_layer_step", "read_ceiling",
                "hbm_GBps_step", "pct_peak_step", "bytes_per_layer_step", "bytes_per_loop", "roofline", "rooflines"):
        out[key] = head[key]
    out["cpu_baseline"] = cpu
    out["rows"] = head["rows"]
    out["extra"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
