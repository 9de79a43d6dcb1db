"""Pins of the oracle's dense attention, column selection and sparse splice.

Dense attention is pinned to torch's fp64 scaled_dot_product_attention and to closed
forms; selection to a brute-force lexicographic sort and to the toy column mass
printed on the flozi.net explainer (section 2, Cell 2); the splice (project page
STEP 02, explainer section 3) to the identities that hold whatever the data:
all columns selected gives back dense attention, none selected leaves the previous
output, and the spliced scores still sum to one probability.
"""
import json
import math
import os
import random

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(n, d, seed):
    g = np.random.default_rng(seed)
    q = (g.standard_normal(d) / math.sqrt(d)).astype(np.float32)
    K = g.standard_normal((n, d)).astype(np.float32)
    V = g.standard_normal((n, d)).astype(np.float32)
    return q, K, V


# ---------------------------------------------------------------- dense ----------
@pytest.mark.parametrize("n,d,sm", [(1, 64, 1.0), (7, 64, 0.3), (300, 128, 1.0), (1000, 128, 0.125)])
def test_dense_matches_sdpa_fp64(orc, n, d, sm):
    q, K, V = _rand(n, d, n + d)
    o, sc, lse = orc.attend_dense(q, K, V, sm)
    qt = torch.from_numpy(q).double().view(1, 1, 1, d)
    Kt = torch.from_numpy(K).double().view(1, 1, n, d)
    Vt = torch.from_numpy(V).double().view(1, 1, n, d)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=sm).view(d).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-12)
    ref_sc = (Kt.view(n, d) @ qt.view(d)).numpy() * sm
    np.testing.assert_allclose(sc, ref_sc, rtol=1e-12, atol=1e-12)
    assert abs(lse - torch.logsumexp(torch.from_numpy(ref_sc), 0).item()) < 1e-11


def test_dense_closed_forms(orc):
    q, K, V = _rand(5, 64, 1)
    # one column: output is that value, lse is its score
    o, sc, lse = orc.attend_dense(q, K[:1], V[:1])
    np.testing.assert_array_equal(o, V[0].astype(np.float64))
    assert lse == sc[0]
    # equal keys: uniform weights, output is the mean value
    Ke = np.tile(K[:1], (5, 1))
    o, sc, lse = orc.attend_dense(q, Ke, V)
    np.testing.assert_allclose(o, V.astype(np.float64).mean(0), rtol=1e-13, atol=1e-14)
    assert abs(lse - (sc[0] + math.log(5))) < 1e-13
    # one dominant column (+50 above every other logit): output is its value
    Kd = np.zeros((5, 64), np.float32)
    qd = np.zeros(64, np.float32)
    qd[0] = 1.0
    Kd[3, 0] = 50.0
    o, sc, lse = orc.attend_dense(qd, Kd, V)
    np.testing.assert_allclose(o, V[3].astype(np.float64), rtol=0, atol=1e-18)


# ---------------------------------------------------------------- select ---------
def _brute_select(s, k):
    order = np.lexsort((np.arange(len(s)), -s.astype(np.float64)))
    return np.sort(order[:min(k, len(s))])


@pytest.mark.parametrize("seed", range(8))
def test_select_brute_force_with_ties(orc, seed):
    g = np.random.default_rng(seed)
    n = int(g.integers(1, 200))
    # few distinct values -> many ties at the threshold
    s = g.integers(-3, 4, n).astype(np.float32) * np.float32(0.5)
    if seed % 2:
        s = g.standard_normal(n).astype(np.float32)
    lse = float(np.log(np.exp(s.astype(np.float64)).sum()))
    for k in (0, 1, n // 3, n - 1, n, n + 5):
        idx, p, m = orc.select(s, lse, k)
        ref = _brute_select(s, k)
        np.testing.assert_array_equal(idx, ref)
        np.testing.assert_allclose(p, np.exp(s[ref].astype(np.float64) - lse), rtol=1e-15)
        assert abs(m - p.sum()) < 1e-15 * max(1, len(p))
    idx, p, m = orc.select(s, lse, n)
    assert abs(m - 1.0) < 1e-12


def test_select_signed_zero_is_a_tie(orc):
    s = np.array([0.0, -0.0, 0.0, -1.0, -0.0], np.float32)
    idx, p, m = orc.select(s, 0.0, 2)
    assert list(idx) == [0, 1]


def test_select_toy_mass_from_page(orc):
    # weights and k from the explainer's Cell 2; scores = log weights, lse = log total
    with open(os.path.join(GOLDEN, "cell2_toy_column_mass.json")) as f:
        gold = json.load(f)
    rng = random.Random(gold["seed"])
    w = np.array([rng.paretovariate(gold["pareto_alpha"]) for _ in range(gold["n"])])
    s = np.log(w).astype(np.float32)
    lse = float(np.log(w.sum()))
    idx, p, m = orc.select(s, lse, gold["k"])
    assert len(idx) == gold["k"]
    assert round(100 * m, gold["printed_digits_after_point"]) == gold["printed_top_mass_percent"]


# ---------------------------------------------------------------- splice ---------
def _two_loops(n, d, seed, sig=0.1):
    g = np.random.default_rng(seed)
    q1 = (g.standard_normal(d) / math.sqrt(d)).astype(np.float32)
    q2 = (q1 + sig * g.standard_normal(d) / math.sqrt(d)).astype(np.float32)
    K1 = g.standard_normal((n, d)).astype(np.float32)
    V1 = g.standard_normal((n, d)).astype(np.float32)
    K2 = (K1 + sig * g.standard_normal((n, d))).astype(np.float32)
    V2 = (V1 + sig * g.standard_normal((n, d))).astype(np.float32)
    return q1, q2, K1, V1, K2, V2


@pytest.mark.parametrize("n,d", [(50, 64), (333, 128)])
def test_splice_all_columns_is_dense(orc, n, d):
    q1, q2, K1, V1, K2, V2 = _two_loops(n, d, n)
    o1, s1, lse1 = orc.attend_dense(q1, K1, V1)
    o2_dense, _, _ = orc.attend_dense(q2, K2, V2)
    idx, p, m = orc.select(s1.astype(np.float32), lse1, n)
    assert abs(m - 1.0) < 1e-6
    o2, sc = orc.attend_sparse(q2, K2, V2, V1, idx, p, m, o1, lse1, s1)
    # o1 was built from the fp64 scores; p from their fp32 rounding: agreement to ~1e-6
    np.testing.assert_allclose(o2, o2_dense, rtol=0, atol=5e-6)
    # with the p's taken from the same fp64 scores the identity is exact to rounding
    p64 = np.exp(s1 - lse1)
    o2b, _ = orc.attend_sparse(q2, K2, V2, V1, np.arange(n, dtype=np.int32), p64, p64.sum(), o1, lse1, s1)
    np.testing.assert_allclose(o2b, o2_dense, rtol=0, atol=1e-12)


def test_splice_no_columns_keeps_previous(orc):
    q1, q2, K1, V1, K2, V2 = _two_loops(40, 64, 2)
    o1, s1, lse1 = orc.attend_dense(q1, K1, V1)
    o2, sc = orc.attend_sparse(q2, K2, V2, V1, np.zeros(0, np.int32), np.zeros(0), 0.0, o1, lse1, s1)
    np.testing.assert_array_equal(o2, o1)
    np.testing.assert_array_equal(sc, s1)


@pytest.mark.parametrize("k", [1, 5, 17, 39])
def test_splice_keeps_probability_normalised(orc, k):
    q1, q2, K1, V1, K2, V2 = _two_loops(40, 64, 3)
    o1, s1, lse1 = orc.attend_dense(q1, K1, V1)
    idx, _, _ = orc.select(s1.astype(np.float32), lse1, k)
    # probabilities of the selected columns from the same fp64 scores as o1
    p = np.exp(s1[idx] - lse1)
    m = p.sum()
    o2, sc = orc.attend_sparse(q2, K2, V2, V1, idx, p, m, o1, lse1, s1)
    # unselected probabilities are the previous ones; the selected ones sum to m
    pr = np.exp(sc - lse1)
    untouched = np.setdiff1d(np.arange(40), idx)
    np.testing.assert_array_equal(sc[untouched], s1[untouched])
    assert abs(pr[idx].sum() - m) < 1e-12
    assert abs(pr.sum() - np.exp(s1 - lse1).sum()) < 1e-6
    # the spliced output is the attention of the spliced distribution over the
    # columns' current values (loop-2 values on S, loop-1 values elsewhere)
    Vmix = V1.astype(np.float64).copy()
    Vmix[idx] = V2[idx]
    o_ref = (pr[:, None] * Vmix).sum(0)
    np.testing.assert_allclose(o2, o_ref + (o1 - (np.exp(s1 - lse1)[:, None] * V1).sum(0)), rtol=0, atol=1e-12)


def test_splice_single_column_closed_form(orc):
    # one column selected: it keeps its old probability m = p_j and takes its new value
    q1, q2, K1, V1, K2, V2 = _two_loops(6, 64, 4)
    o1, s1, lse1 = orc.attend_dense(q1, K1, V1)
    idx, p, m = orc.select(s1.astype(np.float32), lse1, 1)
    j = int(idx[0])
    assert j == int(np.argmax(s1))
    o2, sc = orc.attend_sparse(q2, K2, V2, V1, idx, p, m, o1, lse1, s1)
    np.testing.assert_allclose(o2, o1 + p[0] * (V2[j].astype(np.float64) - V1[j]), rtol=0, atol=1e-14)


def test_splice_unchanged_loop_is_identity(orc):
    # if loop r repeats loop r-1 (same keys, values and query), the in-set softmax
    # times m gives back each column's old probability and nothing changes; a splice
    # that renormalised the selected mass to one would not
    q1, _, K1, V1, _, _ = _two_loops(64, 64, 5)
    o1, s1, lse1 = orc.attend_dense(q1, K1, V1)
    p64 = np.exp(s1 - lse1)
    order = np.argsort(-s1)[:7]
    idx = np.sort(order).astype(np.int32)
    o2, sc = orc.attend_sparse(q1, K1, V1, V1, idx, p64[idx], p64[idx].sum(), o1, lse1, s1)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(sc, s1, rtol=0, atol=1e-12)


def test_select_is_thread_safe(orc):
    # the oracle is called from several threads at once (one per head)
    from concurrent.futures import ThreadPoolExecutor
    g = np.random.default_rng(11)
    inputs = [g.standard_normal(5000).astype(np.float32) for _ in range(16)]
    serial = [orc.select(s, 0.0, 500)[0] for s in inputs]
    with ThreadPoolExecutor(8) as ex:
        par = list(ex.map(lambda s: orc.select(s, 0.0, 500)[0], inputs * 4))
    for i, idx in enumerate(par):
        np.testing.assert_array_equal(idx, serial[i % 16])
