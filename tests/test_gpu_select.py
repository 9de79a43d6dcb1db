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
