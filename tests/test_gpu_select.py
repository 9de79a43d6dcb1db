"""select_columns against the oracle on identical fp32 scores: exact index sets (ties to
the lower index), p_sel and mass within 1e-5, across the selector's paths: spread scores,
heavy ties, a single repeated value, -inf entries, and contexts above 40960 columns."""
import numpy as np
import pytest
import torch

import oracle as orc
import quantized_kv_attention_amd as qkv
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def run_case(S, lse, k):
    B, H, n = S.shape
    sc = torch.from_numpy(S).cuda()
    ls = torch.from_numpy(lse).cuda()
    kk = max(k, 1)
    idx = torch.full((B, H, kk), -7, dtype=torch.int32, device="cuda")
    ps = torch.zeros((B, H, kk), dtype=torch.float32, device="cuda")
    ms = torch.zeros((B, H), dtype=torch.float32, device="cuda")
    qkv.select_columns(sc, ls, n, k, idx, ps, ms)
    torch.cuda.synchronize()
    idx, ps, ms = idx.cpu().numpy(), ps.cpu().numpy(), ms.cpu().numpy()
    for b in range(B):
        for h in range(H):
            ri, rp, rm = orc.select(S[b, h], float(lse[b, h]), k)
            if k > 0:
                assert np.array_equal(idx[b, h, :k], ri), f"b={b} h={h} n={n} k={k}"
                np.testing.assert_allclose(ps[b, h, :k], rp, rtol=1e-5, atol=1e-37)
            assert abs(ms[b, h] - rm) <= 1e-5 * max(rm, 1e-30) + 1e-37


@pytest.mark.parametrize("n,k", [(1, 1), (5, 0), (100, 10), (4097, 410), (32769, 3277), (40960, 4096),
                                 (40961, 4097), (70000, 7000)])
def test_spread_scores(n, k):
    g = np.random.default_rng(n)
    S = (g.standard_normal((1, 3, n)) * 1.7).astype(np.float32)
    lse = np.log(np.exp(S.astype(np.float64)).sum(-1)).astype(np.float32)
    say(f"  select n={n} k={k}")
    run_case(S, lse, k)


@pytest.mark.parametrize("n", [300, 33000])
def test_ties_and_degenerate(n):
    g = np.random.default_rng(7)
    S = np.zeros((1, 4, n), np.float32)
    S[0, 0] = g.integers(-4, 5, n).astype(np.float32) * 0.25       # heavy ties: crowded threshold bin
    S[0, 1] = 1.5                                                    # one value everywhere
    S[0, 2] = g.standard_normal(n).astype(np.float32)
    S[0, 2, ::7] = -np.inf                                           # masked-out columns
    S[0, 3] = g.standard_normal(n).astype(np.float32)
    S[0, 3, ::5] = 0.0
    S[0, 3, 1::5] = -0.0                                             # signed zeros tie
    lse = np.zeros((1, 4), np.float32)
    for k in (1, n // 10, n // 2, n - 1, n):
        run_case(S, lse, k)


@pytest.mark.parametrize("n,k", [(4097, 410), (32769, 3277)])
def test_few_ties_at_and_near_the_threshold(n, k):
    # spread scores with a handful of copies placed on the k-th largest score (a 2- and a
    # 3-way tie across the boundary of the selection, decided by index) and just above and
    # below it while the k-th score itself is unique
    g = np.random.default_rng(n + k)
    S = (g.standard_normal((1, 4, n)) * 1.3).astype(np.float32)
    for h, copies in ((0, 1), (1, 2)):
        row = S[0, h]
        order = np.argsort(-row, kind="stable")
        t = row[order[k - 1]]
        others = g.choice(np.setdiff1d(np.arange(n), [order[k - 1]]), copies, replace=False)
        row[others] = t
    row = S[0, 2]
    order = np.argsort(-row, kind="stable")
    row[g.choice(order[k + 5:], 3, replace=False)] = row[order[k - 3]]   # ties above the threshold
    row[g.choice(order[:k - 5], 3, replace=False)] = row[order[k + 2]]   # ties below it
    S[0, 3] = np.round(S[0, 3] * 64) / 64                                # many small ties everywhere
    lse = np.log(np.exp(S.astype(np.float64)).sum(-1)).astype(np.float32)
    say(f"  select few ties n={n} k={k}")
    for kk in (k - 1, k, k + 1):
        run_case(S, lse, kk)


@pytest.mark.parametrize("n", [4097, 32769])
def test_offset_rows(n):
    # scores far from zero relative to their spread (|min| / (max - min) from 1e3 to 1e6): a
    # bin formula with a rounded bias would put the smallest scores below the first bin
    g = np.random.default_rng(n + 99)
    S = np.zeros((1, 4, n), np.float32)
    for h, (off, spread) in enumerate(((1000.0, 0.05), (-2000.0, 0.01), (50.0, 1e-4), (3e4, 0.02))):
        S[0, h] = (off + spread * g.standard_normal(n)).astype(np.float32)
    lse = np.log(np.exp((S - S.max(-1, keepdims=True)).astype(np.float64)).sum(-1)).astype(np.float32)
    lse = (lse + S.max(-1)).astype(np.float32)
    for k in (1, -(-n // 10), n - 1):
        say(f"  select offset rows n={n} k={k}")
        run_case(S, lse, k)


@pytest.mark.parametrize("n", [4097, 32769])
def test_masked_scores(n):
    # most columns masked (-inf), as in a token selection restricted to the preceding set:
    # k at, below and above the number of finite scores
    g = np.random.default_rng(n + 5)
    S = np.full((1, 3, n), -np.inf, np.float32)
    fin = [n // 4, n // 10, 37]
    for h, m in enumerate(fin):
        cols = g.choice(n, m, replace=False)
        S[0, h, cols] = (g.standard_normal(m) * 0.8).astype(np.float32)
    lse = np.zeros((1, 3), np.float32)
    for k in (1, 30, 37, 38, n // 10, n // 10 + 1):
        say(f"  select masked rows n={n} k={k}")
        run_case(S, lse, k)


@pytest.mark.parametrize("n", [4097, 32769, 40960])
def test_skewed_rows(n):
    # heavy-tailed scores (log-normal, as the token-change ratios are): most columns share the
    # lowest bins of [min, max], so the threshold bin can be crowded past the exact-ranking
    # capacity (then the radix path decides); with exact duplicates planted around the k-th
    # score, and -inf columns
    g = np.random.default_rng(n + 17)
    S = np.zeros((1, 4, n), np.float32)
    for h, sig in enumerate((1.5, 3.0, 6.0, 1.5)):
        S[0, h] = np.exp(sig * g.standard_normal(n)).astype(np.float32)
    S[0, 3, ::5] = -np.inf
    srt = np.sort(S[0, 1])[::-1]
    S[0, 1, g.choice(n, 5, replace=False)] = srt[n // 4 - 1]   # a shared score near k = n/4
    mx = S.max(-1, keepdims=True)
    lse = (np.log(np.exp((S - mx).astype(np.float64)).sum(-1)) + mx[..., 0]).astype(np.float32)
    for k in (1, -(-n // 10), n // 4, n // 4 + 2, n // 2, n - 1):
        say(f"  select skewed rows n={n} k={k}")
        run_case(S, lse, k)


@pytest.mark.parametrize("n", [4097, 32768])
def test_nonnegative_wide_rows(n):
    # rows whose finite scores are all >= 0 and span many binades (binned by order key): with
    # exact zeros and -0.0 among them (equal to +0), values from 1e-30 to 1e30, a row of
    # half-normal scores, and ties planted at the k-th score
    g = np.random.default_rng(n + 31)
    S = np.zeros((1, 4, n), np.float32)
    S[0, 0] = np.abs(g.standard_normal(n)).astype(np.float32)
    S[0, 0, ::9] = 0.0
    S[0, 0, 4::9] = -0.0
    S[0, 1] = (10.0 ** g.uniform(-30, 30, n)).astype(np.float32)
    S[0, 2] = np.exp(2.0 * g.standard_normal(n)).astype(np.float32)
    S[0, 2, ::11] = -np.inf
    S[0, 3] = np.round(np.exp(g.standard_normal(n)) * 8) / 8          # coarse: many ties
    srt = np.sort(S[0, 2][np.isfinite(S[0, 2])])[::-1]
    S[0, 2, g.choice(n, 4, replace=False)] = srt[n // 4 - 1]
    mx = S.max(-1, keepdims=True).astype(np.float64)
    lse = (np.log(np.exp(S.astype(np.float64) - mx).sum(-1)) + mx[..., 0]).astype(np.float32)
    for k in (1, -(-n // 10), n // 4, n // 4 + 1, n // 2, n - 1):
        say(f"  select non-negative wide rows n={n} k={k}")
        run_case(S, lse, k)


@pytest.mark.parametrize("n", [10240, 10241, 20480, 20481])
def test_register_row_boundaries(n):
    # row lengths at the edges of the 10, 20 and 40 scores-per-thread forms, with spread,
    # tied, non-negative heavy-tailed and partly masked rows
    g = np.random.default_rng(n + 71)
    S = np.zeros((1, 4, n), np.float32)
    S[0, 0] = (g.standard_normal(n) * 1.7).astype(np.float32)
    S[0, 1] = (g.integers(-6, 7, n) * 0.5).astype(np.float32)
    S[0, 2] = np.exp(2.0 * g.standard_normal(n)).astype(np.float32)
    S[0, 3] = g.standard_normal(n).astype(np.float32)
    S[0, 3, ::3] = -np.inf
    mx = S.max(-1, keepdims=True).astype(np.float64)
    lse = (np.log(np.exp(S.astype(np.float64) - mx).sum(-1)) + mx[..., 0]).astype(np.float32)
    for k in (1, -(-n // 10), n // 3, n - 1):
        say(f"  select row boundaries n={n} k={k}")
        run_case(S, lse, k)
