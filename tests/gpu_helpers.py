"""Helpers of the GPU parity tests: run the HIP path and the oracle on the same seeded
inputs and compare them.  Planes are read back through the library's qkv_export_plane, so
codes and metadata compare as logical content, whatever the packed layout."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle as orc
import quantized_kv_attention_amd as qkv
from quantized_kv_attention_amd import cache as qcache
from quantized_kv_attention_amd import synth

REL_L2 = 2e-3
MAX_ABS = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_bf16(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_tensor_to_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def unpack_plane(cache: qcache.LayerCache, r: int, b: int, h: int, nslots: int):
    """Logical content of slots [0, nslots) of loop r+1's plane for (b, h), unpacked by the
    library's qkv_export_plane (one code per byte, fp32 metadata)."""
    out = qkv.export_plane(cache, r + 1, b, h, nslots)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def compare_planes(cache: qcache.LayerCache, oc: orc.OracleCache, heads_gpu, heads_orc, loops=None):
    """Bit-exact comparison of codes, scales and zeros of every stored slot."""
    loops = range(cache.R) if loops is None else loops
    for b in range(cache.B):
        for hg, ho in zip(heads_gpu, heads_orc):
            for r in loops:
                rec = oc.planes[b][ho][r]
                ns = rec.pos.size
                if ns == 0:
                    continue
                g = unpack_plane(cache, r, b, hg, ns)
                where = f"b={b} h={hg} loop={r + 1}"
                if not cache.dense[r]:
                    rp = cache.rowpos[r][b, :ns].cpu().numpy()
                    assert np.array_equal(rp, rec.pos), f"rowpos {where}"
                assert np.array_equal(g["kc"], rec.kc), f"K codes {where}: {np.argwhere(g['kc'] != rec.kc)[:5]}"
                assert np.array_equal(g["vc"], rec.vc), f"V codes {where}"
                assert np.array_equal(g["ks"].view(np.uint32), rec.ks.view(np.uint32)), f"K scales {where}"
                assert np.array_equal(g["kz"].view(np.uint32), rec.kz.view(np.uint32)), f"K zeros {where}"
                assert np.array_equal(g["vs"].view(np.uint32), rec.vs.view(np.uint32)), f"V scales {where}"
                assert np.array_equal(g["vz"].view(np.uint32), rec.vz.view(np.uint32)), f"V zeros {where}"


def out_error(o_gpu_bf16: np.ndarray, o_ref_f64: np.ndarray):
    ref = orc.bf16_bits_to_f32(orc.f64_to_bf16_bits(o_ref_f64)).astype(np.float64)
    g = o_gpu_bf16.astype(np.float64)
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    return rel, float(np.abs(g - ref).max())


def assert_out(o_gpu_bf16, o_ref_f64, what):
    rel, mx = out_error(o_gpu_bf16, o_ref_f64)
    say(f"  {what}: rel-L2 {rel:.2e}  max-abs {mx:.2e}")
    assert rel <= REL_L2 and mx <= MAX_ABS, f"{what}: rel-L2 {rel:.3e} max-abs {mx:.3e}"


class Pair:
    """GPU cache + oracle cache built from the same seeded inputs."""

    def __init__(self, w: synth.Workload, n=None, heads=None, extra=0, dense=None, oracle_heads=None,
                 residual_bits=4, full_state=False):
        self.w = w
        self.n = w.n if n is None else n
        self.heads = list(range(w.H)) if heads is None else list(heads)
        H = len(self.heads)
        # oracle_heads: positions in self.heads the oracle models (default: all)
        self.oh = list(range(H)) if oracle_heads is None else list(oracle_heads)
        K, V, act = synth.gen_layer(w, heads=self.heads, n=self.n)
        self.act = act
        cap = int(math.ceil((self.n + extra + 64) / 64) * 64)
        self.dense = [w.rho[r] >= 1.0 for r in range(w.R)] if dense is None else dense
        self.gpu = qcache.LayerCache(w.B, H, w.d, w.R, cap, dense=self.dense, residual_bits=residual_bits,
                                     full_state=full_state)
        self.gpu.prefill([to_dev_bf16(k) for k in K], [to_dev_bf16(v) for v in V], act)
        self.orc = orc.OracleCache(w.B, len(self.oh), w.d, w.R, cap, residual_bits=residual_bits,
                                   full_state=full_state)
        self.orc.prefill([k[:, self.oh] for k in K], [v[:, self.oh] for v in V], act)
        del K, V
        self.bufs = qcache.DecodeBuffers(self.gpu, max_k=self.n + extra)
        self.step_no = 0

    def append(self, step):
        k, v = synth.gen_new_token(self.w, step, heads=self.heads)
        self.gpu.append_token([to_dev_bf16(x) for x in k], [to_dev_bf16(x) for x in v])
        self.orc.append([x[:, self.oh] for x in k], [x[:, self.oh] for x in v])

    def queries(self, step):
        return synth.gen_queries(self.w, step, heads=self.heads)

    def run_gpu_loopwise(self, q, n_dense, k):
        """Runs the GPU step loop by loop, snapshotting what each loop consumed/produced."""
        snaps = []
        bufs, c = self.bufs, self.gpu
        n = c.n_ctx
        for loop in range(1, c.R + 1):
            snap = {}
            if loop > n_dense:
                snap["scores_in"] = bufs.scores[:, :, :n].cpu().numpy().copy()
                snap["lse_in"] = bufs.lse.cpu().numpy().copy()
                snap["o_prev"] = bufs.o_f32[loop - 2].cpu().numpy().copy()
            qcache.decode_loop(c, bufs, loop, to_dev_bf16(q[loop - 1]), n_dense, k)
            torch.cuda.synchronize()
            snap["o"] = bf16_tensor_to_f32(bufs.o[loop - 1])
            snap["o_f32"] = bufs.o_f32[loop - 1].cpu().numpy().copy()
            snap["scores"] = bufs.scores[:, :, :n].cpu().numpy().copy()
            snap["lse"] = bufs.lse.cpu().numpy().copy()
            if loop > n_dense and k > 0:
                idx, ps, mass = bufs.selection(loop, k)
                snap["idx"] = idx.cpu().numpy().copy()
                snap["p_sel"] = ps.cpu().numpy().copy()
                snap["mass"] = mass.cpu().numpy().copy()
            snaps.append(snap)
        return snaps


def check_step(pair: Pair, q, n_dense, k, label=""):
    """Staged parity of one decode step: dense loops, then teacher-forced selection and
    splice, then the untaught end-to-end outputs."""
    snaps = pair.run_gpu_loopwise(q, n_dense, k)
    oh = pair.oh
    for s in snaps:  # keep the oracle's heads only
        for key in list(s.keys()):
            s[key] = s[key][:, oh]
    q = [x[:, oh] for x in q]
    oc = pair.orc
    n = oc.n
    B, H = oc.B, oc.H
    # untaught oracle step
    ref = oc.step(q, n_dense=n_dense, k=k, threads=8)
    # (b, h) whose selections so far equal the untaught oracle's (their selection inputs agree)
    same = np.ones((B, H), bool)
    gapped = 0
    for r in range(oc.R):
        s = snaps[r]
        if r < n_dense:
            assert_out(s["o"], ref[r]["o"], f"{label} loop {r + 1} dense o")
            np.testing.assert_allclose(s["lse"], ref[r]["lse"], rtol=0, atol=2e-4)
            np.testing.assert_allclose(s["scores"], ref[r]["scores"], rtol=0, atol=2e-4)
            continue
        # teacher-forced selection on the GPU's own fp32 scores and lse
        for b in range(B):
            for h in range(H):
                sc = s["scores_in"][b, h]
                lse = float(s["lse_in"][b, h])
                idx, p, m = orc.select(sc, lse, k)
                if k > 0:
                    assert np.array_equal(s["idx"][b, h], idx), f"{label} loop {r + 1} idx b={b} h={h}"
                    np.testing.assert_allclose(s["p_sel"][b, h], p, rtol=1e-5, atol=1e-30)
                    assert abs(s["mass"][b, h] - m) <= 1e-5 * max(m, 1e-30)
        # teacher-forced splice: the oracle takes the GPU's selection, mass and o_prev; the
        # spliced scores it leaves for the next selection are compared too
        o_tf = np.zeros((B, H, oc.d))
        for b in range(B):
            for h in range(H):
                qf = orc.bf16_bits_to_f32(q[r][b, h])
                if k > 0:
                    idx = s["idx"][b, h]
                    p = s["p_sel"][b, h].astype(np.float64)
                    m = float(s["mass"][b, h])
                else:
                    idx, p, m = np.zeros(0, np.int32), np.zeros(0), 0.0
                o_tf[b, h], sc_tf = orc.attend_sparse(qf, oc.Khat[r][b, h, :n], oc.Vhat[r][b, h, :n],
                                                      oc.Vhat[r - 1][b, h, :n], idx, p, m,
                                                      s["o_prev"][b, h].astype(np.float64),
                                                      float(s["lse_in"][b, h]),
                                                      s["scores_in"][b, h].astype(np.float64))
                np.testing.assert_allclose(s["scores"][b, h], sc_tf, rtol=0, atol=2e-4,
                                           err_msg=f"{label} loop {r + 1} spliced scores b={b} h={h}")
        assert_out(s["o"], o_tf, f"{label} loop {r + 1} sparse o (teacher-forced)")
        # end to end against the untaught oracle
        assert_out(s["o"], ref[r]["o"], f"{label} loop {r + 1} sparse o (end-to-end)")
        if 0 < k < n:
            # Untaught selections: where the oracle's selection input has a gap of more than
            # 1e-3 between its k-th and (k+1)-th largest scores (five times the score
            # tolerance) and every earlier selection of the head matched, the sets must be
            # identical; elsewhere near-ties may resolve differently, so report the Jaccard.
            jac = []
            prev = ref[r - 1]["scores"]
            for b in range(B):
                for h in range(H):
                    a, c = set(s["idx"][b, h].tolist()), set(ref[r]["idx"][b][h].tolist())
                    jac.append(len(a & c) / max(1, len(a | c)))
                    top = np.sort(prev[b, h].astype(np.float32))[::-1]
                    if same[b, h] and float(top[k - 1]) - float(top[k]) > 1e-3:
                        gapped += 1
                        assert a == c, f"{label} loop {r + 1} gapped selection b={b} h={h} differs"
                    same[b, h] &= a == c
            say(f"  {label} loop {r + 1} selection Jaccard vs untaught oracle: min {min(jac):.4f}; "
                f"gapped (b, h) so far asserted identical: {gapped}")
    pair.gapped = gapped
    return snaps, ref
