#!/usr/bin/env python3
"""Decode-attention bench: quantized cross-loop KV cache, 32K context, 4 loops, one MI355X.

One step = one decode step of every rotated layer, run loop-major as a looped model does
(loop r over all layers before loop r+1): dense attention in loops 1-2, top-k selection
and the sparse splice in loops 3-4, each loop's call storing the new token's K/V row of
that loop in its BF16 tail (plus, once every 64 steps, the 64-row tail flush into every
loop's plane).  A
selection reads only the previous loop's scores, which loop-major order has ready for every
layer before the sparse loop's first layer, so each sparse loop begins with one
select_columns call over all layers (layers are that call's batch).
Eight distinct layer caches (about 200 MB each) rotate so that no loop finds its planes
in the 256 MB last-level cache.  Steps are replayed from two captured HIP graphs (with and
without the flush); the context stays at n+1 columns.

Prints one JSON line.  `value` is microseconds per decode step of one layer (lower is
better); `roofline` reports the dominant kernel (the loop-2 dense reader, which streams
the base and the loop-2 residual plane) against the 8 TB/s HBM peak; `cpu_baseline` times
the fp64 oracle on a sample of the same workload.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
COPY_BYTES = 1 << 30            # the calibration copy reads and writes this many bytes per launch
COPY_REPS = 8
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dense_split_kernel_ctx32k_traffic.txt")
DENSE_KERNELS = ("dense_split_kernel", "dense_combine_kernel")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--workload", default="ctx32k")
    ap.add_argument("--cpu-heads", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="the oracle baseline runs decode steps until this much wall time has passed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--select-per-layer", action="store_true",
                    help="one select_columns call per layer instead of one per sparse loop for all layers")
    ap.add_argument("--kernel-reps", type=int, default=4, help="timed launches per layer of the dominant kernel")
    ap.add_argument("--no-rows", action="store_true", help="skip the per-entry-point measurements")
    ap.add_argument("--profile-dense", action="store_true",
                    help="only launch the loop-2 dense reader (for counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain elementwise copy of 1 GiB (reference for the byte counters)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write a per-kernel table of the rocprofv3 kernel trace under DIR to --out")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of --profile-dense and of "
                         "--copy-calibration): write the calibrated HBM bytes of the dense reader to --out")
    ap.add_argument("--out", help="output file of the summaries")
    ap.add_argument("--cmd", default="", help="command line recorded in a summary")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_traffic:
        return summarize_traffic(args)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by head with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_kv_attention_amd as qkv
    from quantized_kv_attention_amd import bytes_model as bm
    from quantized_kv_attention_amd import cache as qcache
    from quantized_kv_attention_amd import synth

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(COPY_REPS):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {COPY_REPS} x neg over {COPY_BYTES} B", file=sys.stderr, flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    L = args.layers
    n = w.n
    n_step = n + 1                       # context of the step: prompt + the new token
    k = w.k_cols(n_step)
    cap = int(math.ceil((n + 128) / 64) * 64)
    nb = qkv.body_len(n_step)
    dense = [w.rho[r] >= 1.0 for r in range(w.R)]

    def dev(u16):
        return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()

    t_setup = time.time()
    layers = []
    for l in range(L):
        K, V, act = synth.gen_layer_torch(w, l)
        c = qcache.LayerCache(w.B, w.H, w.d, w.R, cap, dense=dense)
        c.prefill(K, V, act)
        del K, V
        qs = [dev(x) for x in synth.gen_queries(w, 1000 + l)]
        kn, vn = synth.gen_new_token(w, 1000 + l)
        kn = torch.stack([dev(x).view(w.B, w.H, 1, w.d) for x in kn])  # [R, B, H, 1, d]
        vn = torch.stack([dev(x).view(w.B, w.H, 1, w.d) for x in vn])
        c.act[:, :, n] = True
        flush = []
        for r in range(w.R):
            if dense[r]:
                flush.append(None)
            else:
                ap, na = c._active_lists(r, nb, nb + 64)
                flush.append((torch.from_numpy(ap).cuda(), torch.from_numpy(na).cuda()))
        c.n_ctx = n_step
        layers.append(dict(c=c, q=qs, kn=kn, vn=vn, flush=flush, act=act))
        torch.cuda.synchronize()
    stack = qcache.LayerStack([ly["c"] for ly in layers], max_k=k)
    for ly, b in zip(layers, stack.layers):
        ly["b"] = b
    torch.cuda.empty_cache()
    setup_s = time.time() - t_setup
    print(f"[bench] {L} layer caches of {layers[0]['c'].nbytes() / 1e6:.1f} MB ready in {setup_s:.1f}s "
          f"(n={n_step}, k={k})", file=sys.stderr, flush=True)

    def step(with_flush):
        for ly in layers:
            c = ly["c"]
            if with_flush:
                for r in range(w.R):
                    f = ly["flush"][r]
                    if f is None:
                        qkv.kv_encode_loop(c, r + 1, nb, 64)
                    else:
                        qkv.kv_encode_loop(c, r + 1, nb, 64, f[0], f[1])
        for loop in range(1, w.R + 1):
            batched = loop > w.n_dense and not args.select_per_layer
            if batched:
                stack.select(loop, k)    # loop `loop`'s selections of every layer in one call
            for ly in layers:
                # the call stores this loop's row of the new token (position n) in the tail
                # (a loop stores scores only when the next loop selects from them)
                qcache.decode_loop(ly["c"], ly["b"], loop, ly["q"][loop - 1], w.n_dense, k, selected=batched,
                                   k_new=ly["kn"][loop - 1], v_new=ly["vn"][loop - 1],
                                   need_scores=qcache.scores_read_after(loop, w.n_dense, w.R))

    def dense2():
        for ly in layers:
            qcache.decode_loop(ly["c"], ly["b"], 2, ly["q"][1], w.n_dense, k)

    if args.profile_dense:
        for _ in range(args.warmup + args.steps):
            dense2()
        torch.cuda.synchronize()
        print("[bench] dense-reader profiling run done", file=sys.stderr, flush=True)
        return

    # eager warm-up, then capture the two step variants
    step(True)
    step(False)
    torch.cuda.synchronize()
    g_plain, g_flush = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_plain):
        step(False)
    with torch.cuda.graph(g_flush):
        step(True)
    for _ in range(args.warmup):
        g_plain.replay()
    torch.cuda.synchronize()
    # graph replays give the eager result
    ref_o = layers[0]["b"].o_f32.clone()
    step(False)
    torch.cuda.synchronize()
    eager_o = layers[0]["b"].o_f32.clone()
    g_plain.replay()
    torch.cuda.synchronize()
    assert torch.equal(eager_o, layers[0]["b"].o_f32) and torch.equal(ref_o, eager_o), "graph replay differs"

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
    us_step_layer = total_ms * 1000.0 / (K * L)
    print(f"[bench] {K} steps x {L} layers: {total_ms:.2f} ms (wall {wall * 1e3:.2f} ms), "
          f"{us_step_layer:.2f} us per layer-step", file=sys.stderr, flush=True)

    # the same step launched eagerly (no graph), flush excluded
    Ke = min(K, 16)
    e0.record()
    for _ in range(Ke):
        step(False)
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1000.0 / (Ke * L)
    print(f"[bench] eager (no graph), {Ke} steps without flush: {eager_us:.2f} us per layer-step",
          file=sys.stderr, flush=True)
    ceiling = read_ceiling()

    # ---- algorithmic bytes of one layer-step (from the actual masks and selections) ----
    c0, b0, act0 = layers[0]["c"], layers[0]["b"], layers[0]["act"]
    T = n_step - nb
    B, H, d = w.B, w.H, w.d
    rows = []
    slots = []
    for r in range(w.R):
        per_b = []
        sl = []
        for b in range(B):
            if dense[r]:
                per_b.append(nb)
                sl.append(np.arange(nb))
            else:
                a = act0[r][b, :nb]
                s = np.full(nb, -1, np.int64)
                s[a] = np.arange(int(a.sum()))
                per_b.append(int(a.sum()))
                sl.append(s)
        rows.append(per_b)
        slots.append(sl)
    step_bytes = 0
    loop_bytes = []
    for r in range(w.R):
        lb = 0
        if r < w.n_dense:
            for b in range(B):
                lb += H * bm.dense_loop_bytes([rows[p][b] for p in range(r + 1)], T, n_step, d,
                                              scores=qcache.scores_read_after(r + 1, w.n_dense, w.R))
        else:
            # the selection loop r made in the last replay
            idx_all = b0.selection(r + 1, k)[0].cpu().numpy()
            lb += B * H * bm.select_bytes(n_step, k)
            for b in range(B):
                for h in range(H):
                    lb += bm.sparse_loop_bytes(idx_all[b, h], [slots[p][b] for p in range(r + 1)], nb, d,
                                               scores=qcache.scores_read_after(r + 1, w.n_dense, w.R))
        loop_bytes.append(lb)
        step_bytes += lb
    append_bytes = w.R * B * H * d * 2 * 2 * 2               # read new K/V, write the tail rows
    # flush of the 64 oldest tail rows: BF16 rows in, the loop's plane rows out, and the
    # rows' chain through planes 1..r-1 re-read to form the residual
    flush_bytes = 0
    flush_loop_bytes = []
    for r in range(w.R):
        fb = 0
        for b in range(B):
            stored = 64 if dense[r] else int(act0[r][b, nb:nb + 64].sum())
            fb += H * bm.encode_bytes(stored, d, r + 1)
        flush_loop_bytes.append(fb)
        flush_bytes += fb
    step_bytes += append_bytes + flush_bytes * n_flush / K
    gbps_step = step_bytes / (us_step_layer * 1e-6) / 1e9

    # ---- dominant kernel: the loop-2 dense reader, timed on its stream ----
    # HIP events bracket kernel_reps x L back-to-back calls (one call = split + combine
    # launch); a pair of events around every single call would add its own packets' time.
    dense2_bytes = loop_bytes[1]
    s = torch.cuda.current_stream()
    trials = []
    for trial in range(5):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(s)
        for rep in range(args.kernel_reps):
            for ly in layers:
                qkv.attn_decode_dense(ly["c"], 2, ly["q"][1], 1.0, ly["b"].o[1], ly["b"].o_f32[1], ly["b"].scores,
                                      ly["b"].lse, ly["b"].ws, s)
        a1.record(s)
        trials.append((a0, a1))
    torch.cuda.synchronize()
    per_call = sorted(a0.elapsed_time(a1) * 1000.0 / (args.kernel_reps * L) for a0, a1 in trials)
    dense2_us = float(np.mean(per_call))
    achieved = dense2_bytes / (dense2_us * 1e-6) / 1e9
    print(f"[bench] loop-2 dense reader: {dense2_bytes / 1e6:.1f} MB/call, mean {dense2_us:.2f} us over "
          f"{len(per_call)} x {args.kernel_reps * L} calls (min {per_call[0]:.2f}, max {per_call[-1]:.2f}) "
          f"-> {achieved:.0f} GB/s", file=sys.stderr, flush=True)

    traffic = read_traffic()
    full_chain_bytes = sum(w.H * bm.dense_loop_bytes([rows[p][b] for p in range(w.R)], T, n_step, d)
                           for b in range(B))

    rows_out = None
    if not args.no_rows:
        rows_out = measure_rows(w, layers, stack, dense, n, nb, k, loop_bytes, flush_loop_bytes, append_bytes,
                                full_chain_bytes, args)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_heads, args.cpu_seconds)

    out = {
        "metric": "decode-attn us/step & achieved HBM GB/s (% peak), 32K ctx, 4 loops, 1 GPU",
        "value": round(us_step_layer, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: batch {B}, {H} heads x {d}, context {n_step}, {w.R} loops, "
                               f"token retention {w.rho}, {int(w.k_frac * 100)}% key columns in loops "
                               f"{w.n_dense + 1}-{w.R}, INT4 g64 + fp32 scale/zero, 64-token BF16 tail",
                   "layers_rotated": L, "k_columns": k, "step": "R-loop attention, each loop's call storing the new token's tail row, + amortised 64-row flush",
                   "selection": ("one call per layer" if args.select_per_layer
                                 else f"one call per sparse loop for all {L} layers"),
                   "value_is": "microseconds per decode step of one layer"},
        "eager_us_per_layer_step": round(eager_us, 3),
        "read_ceiling": ceiling,
        "hbm_GBps_step": round(gbps_step, 1),
        "pct_peak_step": round(100 * gbps_step / HBM_PEAK_GBPS, 2),
        "bytes_per_layer_step": int(step_bytes),
        "bytes_per_loop": [int(x) for x in loop_bytes],
        "roofline": {"bound": "hbm", "kernel": "dense_split_kernel<128, 2> + dense_combine_kernel<128> (one loop-2 reader call: base + loop-2 residual plane)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "bytes_per_launch": int(dense2_bytes), "mean_launch_us": round(dense2_us, 3),
                     "timing": f"HIP events around {args.kernel_reps * L} back-to-back calls, mean of 5"},
        "cpu_baseline": cpu,
        "rows": rows_out,
    }
    print(json.dumps(out), flush=True)


def read_ceiling():
    """A read-only reference on the same device: the library's plain streaming read of 2 GiB
    (nothing but loads), next to the 8 TB/s peak."""
    import torch
    import quantized_kv_attention_amd as qkv
    x = torch.zeros(1 << 31, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(qkv.STREAM_READ_GROUPS, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    qkv.stream_read(x, sink, s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record(s)
    for _ in range(reps):
        qkv.stream_read(x, sink, s)
    e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    gbps = x.numel() / (us * 1e-6) / 1e9
    del x, sink
    torch.cuda.empty_cache()
    print(f"[bench] read ceiling (plain streaming read of 2 GiB): {gbps:.0f} GB/s", file=sys.stderr, flush=True)
    return {"GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "how": "qkv_stream_read over 2 GiB, HIP events around 10 calls"}


def _dense_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("dense.hip", "common.h"):
        h.update(open(os.path.join(ROOT, "quantized_kv_attention_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measure_rows(w, layers, stack, dense, n, nb, k, loop_bytes, flush_loop_bytes, append_bytes, full_chain_bytes,
                 args):
    """Each entry point of the path timed on its own (events around back-to-back calls over
    the rotated layers), with its algorithmic bytes and the fraction of the HBM peak."""
    import numpy as np
    import torch

    import quantized_kv_attention_amd as qkv
    from quantized_kv_attention_amd import bytes_model as bm
    from quantized_kv_attention_amd import cache as qcache
    from quantized_kv_attention_amd import synth

    s = torch.cuda.current_stream()

    def timed(fn, reps=4):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / reps

    def row(us_total, calls, nbytes, bound="hbm"):
        us = us_total / calls
        gbps = nbytes / (us * 1e-6) / 1e9
        return {"us": round(us, 2), "bytes": int(nbytes), "GBps": round(gbps, 1),
                "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "bound": bound}

    L = len(layers)
    out = {}
    kR = lambda r: k  # same key budget in every sparse loop

    # dense loops (every loop the configuration runs densely), selection, sparse loops
    for loop in range(1, w.R + 1):
        if loop <= w.n_dense:
            t = timed(lambda: [qcache.decode_loop(ly["c"], ly["b"], loop, ly["q"][loop - 1], w.n_dense, k,
                                                  need_scores=qcache.scores_read_after(loop, w.n_dense, w.R))
                               for ly in layers])
            out[f"attn_decode_dense loop {loop}"] = row(t, L, loop_bytes[loop - 1])
        else:
            sel = lambda ly: qkv.select_columns(ly["b"].scores, ly["b"].lse, n + 1, kR(loop),
                                                *ly["b"].selection(loop, kR(loop)), None, s)
            t = timed(lambda: [sel(ly) for ly in layers])
            out[f"select_columns loop {loop} (one call per layer)"] = row(t, L, w.B * w.H * bm.select_bytes(n + 1, k),
                                                                         "latency")
            t = timed(lambda: stack.select(loop, k, s))
            out[f"select_columns loop {loop} ({L} layers per call)"] = row(t, L, w.B * w.H * bm.select_bytes(n + 1, k),
                                                                          "latency")
            def sp(ly):
                idx, ps, mass = ly["b"].selection(loop, k)
                qkv.attn_decode_sparse(ly["c"], loop, ly["q"][loop - 1], 1.0, idx, ps, mass, k,
                                       ly["b"].o_f32[loop - 2], ly["b"].lse,
                                       ly["b"].scores if qcache.scores_read_after(loop, w.n_dense, w.R) else None,
                                       ly["b"].o[loop - 1],
                                       ly["b"].o_f32[loop - 1], ly["b"].ws, s)
            t = timed(lambda: [sp(ly) for ly in layers])
            sel_b = w.B * w.H * bm.select_bytes(n + 1, k)
            out[f"attn_decode_sparse loop {loop}"] = row(t, L, loop_bytes[loop - 1] - sel_b)

    # the last loop read densely through its whole chain (every plane, sparse ones by their
    # row maps), for comparison with the sparse splice; overwrites that loop's outputs only
    R = w.R
    t = timed(lambda: [qkv.attn_decode_dense(ly["c"], R, ly["q"][R - 1], 1.0, ly["b"].o[R - 1], ly["b"].o_f32[R - 1],
                                             ly["b"].scores, ly["b"].lse, ly["b"].ws, s) for ly in layers])
    out[f"attn_decode_dense loop {R} (full chain, {R} planes)"] = row(t, L, full_chain_bytes)

    # token append into every loop's tail, and the 64-row flush of every loop
    t = timed(lambda: [qkv.kv_append_tail(ly["c"], 0, n, ly["kn"], ly["vn"], s) for ly in layers])
    out["kv_append_tail (all loops)"] = row(t, L, append_bytes, "latency")
    for r in range(w.R):
        def fl(ly, r=r):
            f = ly["flush"][r]
            if f is None:
                qkv.kv_encode_loop(ly["c"], r + 1, nb, 64, stream=s)
            else:
                qkv.kv_encode_loop(ly["c"], r + 1, nb, 64, f[0], f[1], stream=s)
        t = timed(lambda: [fl(ly) for ly in layers])
        out[f"kv_encode_loop flush loop {r + 1}"] = row(t, L, flush_loop_bytes[r], "latency")

    # bulk encode of a whole prompt, loop by loop, into a fresh cache
    K, V, act = synth.gen_layer_torch(w, 4242)
    c = qcache.LayerCache(w.B, w.H, w.d, w.R, layers[0]["c"].cap, dense=dense)
    for r in range(w.R):
        c.act[r, :, :n] = np.asarray(act[r])
    calls = []
    for r in range(w.R):
        if dense[r]:
            ks, vs = K[r][:, :, :nb].contiguous(), V[r][:, :, :nb].contiguous()
            calls.append((r, None, None, ks, vs))
        else:
            ap, na = c._active_lists(r, 0, nb)
            ks = torch.zeros((w.B, w.H, nb, w.d), dtype=torch.bfloat16, device="cuda")
            vs = torch.zeros_like(ks)
            for b in range(w.B):
                cnt = int(na[b])
                rows_ = torch.from_numpy(ap[b, :cnt].astype(np.int64)).cuda()
                ks[b, :, :cnt] = K[r][b].index_select(1, rows_)
                vs[b, :, :cnt] = V[r][b].index_select(1, rows_)
            calls.append((r, torch.from_numpy(ap).cuda(), torch.from_numpy(na).cuda(), ks, vs))
    del K, V
    for r, ap, na, ks, vs in calls:
        t = timed(lambda: qkv.kv_encode_loop(c, r + 1, 0, nb, ap, na, ks, vs, s), reps=3)
        stored = [nb if dense[r] else int(act[r][b, :nb].sum()) for b in range(w.B)]
        nbytes = sum(w.H * bm.encode_bytes(st, w.d, r + 1) for st in stored)
        out[f"kv_encode_loop bulk loop {r + 1} ({nb} positions)"] = row(t, 1, nbytes)
    del calls, c
    torch.cuda.empty_cache()
    for name, v in out.items():
        print(f"[bench] {name:40s} {v['us']:9.2f} us  {v['bytes'] / 1e6:8.2f} MB  {v['GBps']:8.1f} GB/s",
              file=sys.stderr, flush=True)
    return out


def read_traffic():
    """HBM bytes per launch of the dense reader from the committed counter summary, or None
    when the summary is missing or was taken on another version of the kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith((" ", "#", "|")):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_hash") != _dense_source_hash():
        return None
    try:
        return int(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _rocprof_db(d):
    import glob
    dbs = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {d}")
    import sqlite3
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
    lines = [f"# rocprofv3 kernel trace summary", f"command: {args.cmd}", "",
             "| kernel | launches | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for name, cnt, avg, mn, mx, sm in rows:
        lines.append(f"| {_short(name)[:90]} | {cnt} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | "
                     f"{100 * sm / tot:.1f}% |")
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_per_dispatch(d, counter, names):
    """Mean value of `counter` per dispatch of each kernel whose name contains one of `names`."""
    con = _rocprof_db(d)
    vals = {}
    for name, cn, cv in con.execute("select name, counter_name, counter_value from pmc_events"):
        if cn != counter:
            continue
        for k in names:
            if k in name:
                vals.setdefault(k, []).append(float(cv))
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}


def summarize_traffic(args):
    """Calibrated HBM bytes per launch of the dense reader (split + combine kernels).

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the same counters read
    for a plain elementwise copy that reads and writes COPY_BYTES each."""
    fdir, wdir, cfdir, cwdir = args.summarize_traffic
    cf = _counter_per_dispatch(cfdir, "FETCH_SIZE", ("neg",)).get("neg")
    cw = _counter_per_dispatch(cwdir, "WRITE_SIZE", ("neg",)).get("neg")
    if not cf or not cw:
        raise SystemExit("copy calibration dispatches not found")
    f_fac = COPY_BYTES / (cf[0] * 1024.0)
    w_fac = COPY_BYTES / (cw[0] * 1024.0)
    fe = _counter_per_dispatch(fdir, "FETCH_SIZE", DENSE_KERNELS)
    wr = _counter_per_dispatch(wdir, "WRITE_SIZE", DENSE_KERNELS)
    rd = sum(fe[k][0] for k in fe) * 1024.0 * f_fac
    wt = sum(wr[k][0] for k in wr) * 1024.0 * w_fac
    lines = ["# HBM traffic of the loop-2 dense reader, 32K context (16 heads x 128, one launch = split + combine)",
             f"command: {args.cmd}", "",
             "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | dispatches |", "|---|---|---|---|"]
    for k in DENSE_KERNELS:
        lines.append(f"| {k} | {fe.get(k, (0, 0))[0]:.1f} | {wr.get(k, (0, 0))[0]:.1f} | {fe.get(k, (0, 0))[1]} |")
    lines += ["", f"| copy of {COPY_BYTES} B | {cf[0]:.1f} | {cw[0]:.1f} | {cf[1]} |", "",
              f"fetch_factor: {f_fac:.4f}", f"write_factor: {w_fac:.4f}",
              f"read_bytes_per_launch: {int(rd)}", f"write_bytes_per_launch: {int(wt)}",
              f"hbm_bytes_per_launch: {int(rd + wt)}", f"kernel_source_hash: {_dense_source_hash()}"]
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(w, heads, seconds):
    """The fp64 oracle on `heads` heads of the same workload: decode steps (every loop, from
    the encoded cache) until `seconds` of wall time have passed, scaled to all heads of one
    layer.  The cache build is not timed."""
    import numpy as np

    import oracle as orc
    from quantized_kv_attention_amd import synth

    hs = list(range(min(heads, w.H)))
    K, V, act = synth.gen_layer(w, heads=hs)
    oc = orc.OracleCache(w.B, len(hs), w.d, w.R, w.n + 128)
    oc.prefill(K, V, act)
    del K, V
    kn, vn = synth.gen_new_token(w, 1000, heads=hs)
    oc.append(kn, vn)
    k = w.k_cols(oc.n)
    threads = max(1, min(len(hs) * w.B, os.cpu_count() or 1, 16))
    steps = 0
    t0 = time.perf_counter()
    while True:
        oc.step(synth.gen_queries(w, 2000 + steps, heads=hs), w.n_dense, k, threads=threads)
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds or steps >= 100000:
            break
    per_step_us = dt / steps * 1e6 * (w.H / len(hs))
    return {"value": round(per_step_us, 1), "unit": "us/step", "cores": threads, "kind": "oracle",
            "sample": f"{len(hs)} of {w.H} heads x {steps} decode steps (all {w.R} loops, context {oc.n}), "
                      f"{dt:.1f} s wall on {threads} threads" + (f", scaled to {w.H} heads" if len(hs) < w.H else "")}


if __name__ == "__main__":
    main()
