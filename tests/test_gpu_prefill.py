"""attn_prefill_sparse (and kv_gather_rows building its compact buffers) against the oracle:
active query rows of a sparse prefill loop against one selected column set per head, causal
(project page, The Method, after STEP 03; STEP 02; explainer section 3).  bf16 outputs within
rel-L2 2e-3 and max-abs 1e-2 of bf16(oracle), the cached mass m_i within 1e-4 relative; the
gathered rows bit-exact."""
import math

import numpy as np
import pytest
import torch

import oracle as orc
import quantized_kv_attention_amd as qkv
from gpu_helpers import assert_out, say, to_dev_bf16
from quantized_kv_attention_amd import synth

pytestmark = pytest.mark.gpu


def _f(u16):
    return orc.bf16_bits_to_f32(u16)


def _lse_rows(q, k, qpos):
    """log-sum-exp of each query row over its causal columns (fp64 numpy, rows in chunks)."""
    out = np.zeros(q.shape[0], np.float64)
    kk = k.astype(np.float64)
    for i0 in range(0, q.shape[0], 512):
        s = q[i0:i0 + 512].astype(np.float64) @ kk.T
        s[np.arange(k.shape[0])[None, :] > qpos[i0:i0 + 512][:, None]] = -np.inf
        mx = s.max(1, keepdims=True)
        out[i0:i0 + 512] = mx[:, 0] + np.log(np.exp(s - mx).sum(1))
    return out


def _case(w, B, H, n, r, k, sample_rows=None, seed_shift=0, check_heads=None):
    """Builds full per-loop K/V/Q, gathers compact buffers on the GPU, runs the kernel and the
    oracle; r is the sparse loop (0-based, >= 1).  The GPU runs every head; the oracle checks
    check_heads (default all), whose lse inputs are exact (the others get log(position + 1))."""
    check_heads = list(range(H)) if check_heads is None else list(check_heads)
    act = synth.gen_masks(w, n)
    Kf = np.zeros((2, B, H, n, w.d), np.uint16)
    Vf = np.zeros_like(Kf)
    Qf = np.zeros_like(Kf)
    cpos = np.zeros((B, H, k), np.int32)
    for b in range(B):
        for h in range(H):
            Kb, Vb = synth.gen_head_kv(w, b, h + seed_shift, act, n)
            Qb = synth.gen_prefill_queries(w, b, h + seed_shift, n)
            for t, rr in enumerate((r - 1, r)):
                Kf[t, b, h], Vf[t, b, h], Qf[t, b, h] = Kb[rr], Vb[rr], Qb[rr]
            cpos[b, h] = synth.gen_columns(w, n, k, b, h + seed_shift)
    qpos_l = [np.nonzero(act[r][b])[0].astype(np.int32) for b in range(B)]
    nq = min(x.size for x in qpos_l)
    qpos = np.stack([x[:nq] for x in qpos_l])
    # the preceding loop's log-sum-exp of each active row over its causal columns (input
    # preparation, fp64 numpy), and a synthetic preceding output
    lse0 = np.zeros((B, H, nq), np.float32)
    for b in range(B):
        for h in range(H):
            if h in check_heads:
                lse0[b, h] = _lse_rows(_f(Qf[0, b, h, qpos[b]]), _f(Kf[0, b, h]), qpos[b]).astype(np.float32)
            else:
                lse0[b, h] = np.log(qpos[b] + 1.0).astype(np.float32)
    o0 = np.random.default_rng(n + H).standard_normal((B, H, nq, w.d)).astype(np.float32) * 0.3
    # compact buffers on the GPU
    dq = [to_dev_bf16(Qf[t]) for t in range(2)]
    dk = [to_dev_bf16(Kf[t]) for t in range(2)]
    dv = [to_dev_bf16(Vf[t]) for t in range(2)]
    qp = torch.from_numpy(qpos).cuda()
    cp = torch.from_numpy(cpos).cuda()
    q1c, q0c = qkv.gather_rows(dq[1], qp), qkv.gather_rows(dq[0], qp)
    k1c, k0c = qkv.gather_rows(dk[1], cp), qkv.gather_rows(dk[0], cp)
    v1t, v0t = qkv.gather_rows(dv[1], cp, transpose=True), qkv.gather_rows(dv[0], cp, transpose=True)
    o32 = torch.zeros((B, H, nq, w.d), dtype=torch.float32, device="cuda")
    o16 = torch.zeros((B, H, nq, w.d), dtype=torch.bfloat16, device="cuda")
    mass = torch.zeros((B, H, nq), dtype=torch.float32, device="cuda")
    qkv.attn_prefill_sparse(q1c, q0c, qp, torch.from_numpy(lse0).cuda(), torch.from_numpy(o0).cuda(), k1c, k0c, v1t,
                            v0t, cp, 1.0, o32, o16, mass)
    torch.cuda.synchronize()
    # the gathers, bit for bit
    g_q1 = q1c.view(torch.int16).cpu().numpy().view(np.uint16)
    g_v0 = v0t.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(B):
        assert np.array_equal(g_q1[b], Qf[1, b][:, qpos[b]]), "gathered query rows"
        for h in range(H):
            assert np.array_equal(g_v0[b, h, :, :k], Vf[0, b, h, cpos[b, h]].T), "gathered transposed values"
            assert not g_v0[b, h, :, k:].any(), "transposed padding"
    og = o16.float().cpu().numpy()
    ms = mass.cpu().numpy()
    rows = np.arange(nq) if sample_rows is None else sample_rows
    for b in range(B):
        for h in check_heads:
            O, m = orc.prefill_sparse(_f(Qf[1, b, h, qpos[b, rows]]), _f(Qf[0, b, h, qpos[b, rows]]), qpos[b, rows],
                                      lse0[b, h, rows].astype(np.float64), o0[b, h, rows].astype(np.float64),
                                      _f(Kf[1, b, h, cpos[b, h]]), _f(Vf[1, b, h, cpos[b, h]]),
                                      _f(Kf[0, b, h, cpos[b, h]]), _f(Vf[0, b, h, cpos[b, h]]), cpos[b, h])
            assert_out(og[b, h, rows], O, f"prefill n={n} d={w.d} b={b} h={h} rows={len(rows)}")
            np.testing.assert_allclose(ms[b, h, rows], m, rtol=1e-4, atol=1e-30)
    return nq


@pytest.mark.parametrize("wname,B,H,n,loop", [("tiny", 1, 1, 256, 3), ("tiny", 2, 3, 3000, 4),
                                              ("ctx4k", 2, 3, 2048, 3), ("ctx4k", 1, 2, 3001, 4)])
def test_prefill_sparse_small(wname, B, H, n, loop):
    w = synth.WORKLOADS[wname]
    w = synth.Workload(w.name, B, H, w.d, n, w.R, w.sigma, w.rho, w.n_dense, w.k_frac, 1, w.seed)
    k = w.k_cols(n)
    nq = _case(w, B, H, n, loop - 1, k)
    say(f"  prefill loop {loop}: {nq} active rows x {k} columns, n={n}, d={w.d}, B={B}, H={H}")


def test_prefill_sparse_no_columns_keeps_previous_output():
    w = synth.WORKLOADS["tiny"]
    B, H, n, d = 1, 2, 128, 64
    q = torch.zeros((B, H, 8, d), dtype=torch.bfloat16, device="cuda")
    qp = torch.arange(8, dtype=torch.int32, device="cuda").view(1, 8) * 16
    o0 = torch.randn((B, H, 8, d), device="cuda")
    o32 = torch.zeros_like(o0)
    empty = torch.zeros((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    qkv.attn_prefill_sparse(q, q, qp, torch.zeros((B, H, 8), device="cuda"), o0, empty, empty, empty, empty,
                            torch.zeros((B, H, 0), dtype=torch.int32, device="cuda"), 1.0, o32)
    torch.cuda.synchronize()
    assert torch.equal(o32, o0)


@pytest.mark.timeout(300)
def test_prefill_sparse_ctx32k_sampled_rows():
    """16 heads x 128, 32K prompt: loop 3's 8192 active rows against 3277 selected columns per
    head on the GPU (every head), the oracle on 2 heads and a sample of rows across the range."""
    w = synth.WORKLOADS["ctx32k"]
    n, k = w.n, w.k_cols(w.n)
    rows = np.unique(np.concatenate([np.arange(0, 8192, 97), np.arange(8100, 8192)]))
    nq = _case(w, 1, w.H, n, 2, k, sample_rows=rows, check_heads=[0, 11])
    say(f"  prefill 32K loop 3: {nq} rows x {k} columns x {w.H} heads, heads 0 and 11 x {rows.size} rows checked")
