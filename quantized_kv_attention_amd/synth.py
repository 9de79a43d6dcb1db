"""Seeded synthetic inputs for looped-transformer decode attention.

This module only draws inputs; it holds none of the method's arithmetic and is the one
piece shared by the tests (which feed both the oracle and the HIP path) and the bench.

Recipe (Ouro-shaped layer caches; the pages evaluate real Ouro/Huginn checkpoints on
public benchmarks, which these synthetic caches stand in for):

* loop-1 keys and values ~ N(0, 1), rounded to bf16 (nearest-even);
* loop r >= 2: active rows X^(r) = bf16(X^(r-1) + sigma_r * N(0, 1)); inactive rows
  reuse X^(r-1) (project page, The Method, STEP 01);
* active sets: loops 1..n_dense keep every token; loop r keeps ceil(rho_r * n) tokens
  drawn uniformly from the loop r-1 set, so the sets nest (explainer section 2);
* queries: q^(1) ~ N(0,1)/sqrt(d); q^(r) = bf16(q^(r-1) + sigma_r * N(0,1)/sqrt(d)),
  so consecutive loops attend to related columns; the softmax scale is 1;
* generated decode tokens are active in every loop and follow the same K/V recipe.

Every (kind, sequence, head) draws from its own numpy PCG64 stream seeded by
SeedSequence([seed, kind, b, h]), so any head can be regenerated on its own.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

KIND_KV, KIND_MASK, KIND_Q, KIND_NEW, KIND_HIDDEN, KIND_PREFILL_Q, KIND_COLS = 1, 2, 3, 4, 5, 6, 7


@dataclass
class Workload:
    name: str
    B: int
    H: int
    d: int
    n: int
    R: int
    sigma: list          # sigma_r for r = 2..R (len R-1)
    rho: list            # token retention per loop (len R); 1.0 = dense
    n_dense: int = 2     # loops 1..n_dense use dense attention
    k_frac: float = 0.10 # key-column budget of sparse loops
    steps: int = 1       # decode steps of the workload
    seed: int = 20260924

    def k_cols(self, n: int | None = None) -> int:
        n = self.n if n is None else n
        return int(math.ceil(self.k_frac * n))


def _ouro_sigma(R):
    base = [0.3, 0.1, 0.05]
    return [base[i] if i < 3 else 0.05 for i in range(R - 1)]


WORKLOADS = {
    # 1 layer, 1 head, d 64, context 256, R=4, loops 3-4 keep 25%/10% rows, 10% top-K
    "tiny": Workload("tiny", 1, 1, 64, 256, 4, [0.3, 0.1, 0.05], [1, 1, 0.25, 0.10], 2, 0.10, 4, 20260924),
    # 16x128 heads, 4K context, 64 decode steps
    "ctx4k": Workload("ctx4k", 1, 16, 128, 4096, 4, [0.3, 0.1, 0.05], [1, 1, 0.25, 0.10], 2, 0.10, 64, 20260925),
    # 16x128 heads, 32K context: the long-context decode case
    "ctx32k": Workload("ctx32k", 1, 16, 128, 32768, 4, [0.3, 0.1, 0.05], [1, 1, 0.25, 0.10], 2, 0.10, 64, 20260926),
    # 40x128 heads, 8K context, 32 loops, 10% rows and 10% columns from loop 3 on
    "deep32": Workload("deep32", 1, 40, 128, 8192, 32, [0.5 * 0.85 ** r for r in range(2, 33)],
                       [1, 1] + [0.10] * 30, 2, 0.10, 8, 20260927),
    # batch 8 x 16x128 heads, 16K context per sequence
    "batch8": Workload("batch8", 8, 16, 128, 16384, 4, [0.3, 0.1, 0.05], [1, 1, 0.25, 0.10], 2, 0.10, 128, 20260928),
}


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (input formatting only; finite
    inputs: the 32-bit sum cannot carry out of the top bit)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_float(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed, kind, b, h=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, kind, b, h])))


def gen_masks(w: Workload, n: int | None = None) -> list:
    """Active-token masks act[r] (bool [B, n]) for r = 0..R-1, nested after the dense loops."""
    n = w.n if n is None else n
    act = [np.ones((w.B, n), bool) for _ in range(w.R)]
    for b in range(w.B):
        g = _rng(w.seed, KIND_MASK, b)
        cur = np.arange(n)
        for r in range(w.R):
            if w.rho[r] >= 1.0:
                continue
            size = min(int(math.ceil(w.rho[r] * n)), cur.size)
            cur = np.sort(g.choice(cur, size=size, replace=False))
            m = np.zeros(n, bool)
            m[cur] = True
            act[r][b] = m
    return act


def gen_head_kv(w: Workload, b: int, h: int, act: list, n: int | None = None):
    """Per-loop K/V of one (sequence, head): two lists of R uint16 arrays [n, d]."""
    n = w.n if n is None else n
    g = _rng(w.seed, KIND_KV, b, h)
    K = [None] * w.R
    V = [None] * w.R
    kf = g.standard_normal((n, w.d), dtype=np.float32)
    vf = g.standard_normal((n, w.d), dtype=np.float32)
    K[0] = bf16_round_bits(kf)
    V[0] = bf16_round_bits(vf)
    for r in range(1, w.R):
        sig = np.float32(w.sigma[r - 1])
        rows = np.nonzero(act[r][b])[0]          # noise is drawn for the active rows only
        nk = g.standard_normal((rows.size, w.d), dtype=np.float32)
        nv = g.standard_normal((rows.size, w.d), dtype=np.float32)
        K[r] = K[r - 1].copy()
        V[r] = V[r - 1].copy()
        K[r][rows] = bf16_round_bits(bf16_bits_to_float(K[r - 1][rows]) + sig * nk)
        V[r][rows] = bf16_round_bits(bf16_bits_to_float(V[r - 1][rows]) + sig * nv)
    return K, V


def gen_layer(w: Workload, heads=None, n: int | None = None):
    """K[r], V[r]: uint16 [B, H', n, d] for the chosen heads (default all); act[r]: bool [B, n]."""
    n = w.n if n is None else n
    heads = list(range(w.H)) if heads is None else list(heads)
    act = gen_masks(w, n)
    K = [np.zeros((w.B, len(heads), n, w.d), np.uint16) for _ in range(w.R)]
    V = [np.zeros((w.B, len(heads), n, w.d), np.uint16) for _ in range(w.R)]

    def one(bi):
        b, i = bi
        kh, vh = gen_head_kv(w, b, heads[i], act, n)
        for r in range(w.R):
            K[r][b, i] = kh[r]
            V[r][b, i] = vh[r]

    jobs = [(b, i) for b in range(w.B) for i in range(len(heads))]
    if len(jobs) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(min(8, len(jobs))) as ex:   # each (b, h) has its own stream
            list(ex.map(one, jobs))
    else:
        one(jobs[0])
    return K, V, act


def gen_queries(w: Workload, step: int, heads=None):
    """q[r]: uint16 bf16 bits [B, H', d] for decode step `step`."""
    heads = list(range(w.H)) if heads is None else list(heads)
    q = [np.zeros((w.B, len(heads), w.d), np.uint16) for _ in range(w.R)]
    inv = np.float32(1.0 / math.sqrt(w.d))
    for b in range(w.B):
        for i, h in enumerate(heads):
            g = _rng(w.seed, KIND_Q + 16 * step, b, h)
            cur = bf16_round_bits(g.standard_normal(w.d, dtype=np.float32) * inv)
            q[0][b, i] = cur
            for r in range(1, w.R):
                sig = np.float32(w.sigma[r - 1])
                nz = g.standard_normal(w.d, dtype=np.float32) * inv
                cur = bf16_round_bits(bf16_bits_to_float(cur) + sig * nz)
                q[r][b, i] = cur
    return q


def gen_new_token(w: Workload, step: int, heads=None):
    """k[r], v[r]: uint16 [B, H', d] of the token generated at decode step `step`."""
    heads = list(range(w.H)) if heads is None else list(heads)
    k = [np.zeros((w.B, len(heads), w.d), np.uint16) for _ in range(w.R)]
    v = [np.zeros((w.B, len(heads), w.d), np.uint16) for _ in range(w.R)]
    for b in range(w.B):
        for i, h in enumerate(heads):
            g = _rng(w.seed, KIND_NEW + 16 * step, b, h)
            kc = g.standard_normal(w.d, dtype=np.float32)
            vc = g.standard_normal(w.d, dtype=np.float32)
            k[0][b, i] = bf16_round_bits(kc)
            v[0][b, i] = bf16_round_bits(vc)
            for r in range(1, w.R):
                sig = np.float32(w.sigma[r - 1])
                k[r][b, i] = bf16_round_bits(bf16_bits_to_float(k[r - 1][b, i]) + sig * g.standard_normal(w.d, dtype=np.float32))
                v[r][b, i] = bf16_round_bits(bf16_bits_to_float(v[r - 1][b, i]) + sig * g.standard_normal(w.d, dtype=np.float32))
    return k, v


def active_positions(act_r: np.ndarray, p0: int, p1: int):
    """Sorted active positions of each sequence in [p0, p1) as a padded int32 [B, p1-p0]
    array plus counts [B] (the list form the encoder takes)."""
    B = act_r.shape[0]
    out = np.zeros((B, max(p1 - p0, 1)), np.int32)
    cnt = np.zeros(B, np.int32)
    for b in range(B):
        pos = p0 + np.nonzero(act_r[b, p0:p1])[0]
        out[b, :pos.size] = pos
        cnt[b] = pos.size
    return out, cnt


def gen_layer_torch(w: Workload, layer: int, device="cuda", n: int | None = None):
    """Same recipe as gen_layer, drawn with torch's generator on the GPU (for the large
    caches of the bench; the masks come from gen_masks).  Returns K[r], V[r] as bf16
    tensors [B, H, n, d] and act[r] as bool arrays [B, n]."""
    import torch
    n = w.n if n is None else n
    act = gen_masks(w, n)
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1000 + layer)
    shape = (w.B, w.H, n, w.d)
    K = [torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)]
    V = [torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)]
    for r in range(1, w.R):
        a = torch.from_numpy(act[r]).to(device)[:, None, :, None]
        sig = float(w.sigma[r - 1])
        nk = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        K.append(torch.where(a, (K[r - 1].float() + sig * nk).to(torch.bfloat16), K[r - 1]))
        del nk
        nv = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        V.append(torch.where(a, (V[r - 1].float() + sig * nv).to(torch.bfloat16), V[r - 1]))
        del nv
    return K, V, act


def gen_hidden(w: Workload, dm: int, n: int | None = None, b: int = 0):
    """Per-loop hidden states of one sequence for the token selection: H[r] uint16 (bf16
    bits) [n, dm], r = 0..R-1.  H^(1) ~ N(0, 1); loop r's update of token t has magnitude
    sigma_r * g_t with g_t log-normal (sigma 1.5), so that a minority of tokens carries most
    of the change, as the explainer's section 2 describes the token-update redundancy."""
    n = w.n if n is None else n
    g = _rng(w.seed, KIND_HIDDEN, b)
    H = [bf16_round_bits(g.standard_normal((n, dm), dtype=np.float32))]
    gt = np.exp(1.5 * g.standard_normal(n)).astype(np.float32)
    for r in range(1, w.R):
        sig = np.float32(w.sigma[r - 1])
        upd = (sig * gt)[:, None] * g.standard_normal((n, dm), dtype=np.float32)
        H.append(bf16_round_bits(bf16_bits_to_float(H[-1]) + upd))
    return H


def gen_prefill_queries(w: Workload, b: int, h: int, n: int | None = None):
    """Per-loop queries of every prompt token of one (sequence, head) for prefill: Q[r]
    uint16 (bf16 bits) [n, d]; q^(1) ~ N(0,1)/sqrt(d), q^(r) = bf16(q^(r-1) + sigma_r N(0,1)/sqrt(d))."""
    n = w.n if n is None else n
    g = _rng(w.seed, KIND_PREFILL_Q, b, h)
    sd = np.float32(1.0 / math.sqrt(w.d))
    Q = [bf16_round_bits(g.standard_normal((n, w.d), dtype=np.float32) * sd)]
    for r in range(1, w.R):
        sig = np.float32(w.sigma[r - 1])
        Q.append(bf16_round_bits(bf16_bits_to_float(Q[-1]) + sig * sd * g.standard_normal((n, w.d), dtype=np.float32)))
    return Q


def gen_columns(w: Workload, n: int, k: int, b: int, h: int):
    """A selected column set of one (sequence, head): k positions of [0, n), ascending."""
    g = _rng(w.seed, KIND_COLS, b, h)
    return np.sort(g.choice(n, size=min(k, n), replace=False)).astype(np.int32)
