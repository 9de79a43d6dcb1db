"""Pins of the oracle's token selection (explainer section 3, cross-loop token-sparse
updates: the tokens updated in the preceding loop are ranked by their normalized
hidden-state change and a top-k subset stays active, so active sets nest; project page
STEP 01) against facts fixed outside the oracle."""
import numpy as np
import pytest

from quantized_kv_attention_amd import synth


def _bf16(x):
    return synth.bf16_bits_to_float(synth.bf16_round_bits(np.asarray(x, np.float32)))


def test_closed_form_one_hot_states(orc):
    # H_prev[t] = a_t e_0, H_cur[t] = H_prev[t] + b_t e_1: the change is |b_t| / |a_t| exactly
    rng = np.random.default_rng(11)
    n, dm = 50, 16
    a = _bf16(rng.uniform(0.5, 4, n) * rng.choice([-1, 1], n))
    bb = _bf16(rng.uniform(0, 2, n) * rng.choice([-1, 1], n))
    Hp = np.zeros((n, dm), np.float32)
    Hp[:, 0] = a
    Hc = Hp.copy()
    Hc[:, 1] = bb
    sc = orc.token_change(Hc, Hp)
    np.testing.assert_array_equal(sc, np.abs(bb.astype(np.float64)) / np.abs(a.astype(np.float64)))


def test_scale_invariance_and_zero_states(orc):
    rng = np.random.default_rng(12)
    Hp = _bf16(rng.standard_normal((40, 32)))
    Hc = _bf16(Hp + 0.1 * rng.standard_normal((40, 32)))
    s1 = orc.token_change(Hc, Hp)
    s2 = orc.token_change(Hc * np.float32(8.0), Hp * np.float32(8.0))  # a power of two: exact
    np.testing.assert_array_equal(s1, s2)
    Z = np.zeros((3, 32), np.float32)
    W = Z.copy()
    W[1, 5] = 1.0
    assert list(orc.token_change(W, Z)) == [0.0, np.inf, 0.0]


def test_selection_nests_and_takes_planted_tokens(orc):
    # a few tokens with a ten-times larger change are kept; nothing outside the preceding
    # active set is ever kept, and k beyond it keeps exactly that set
    rng = np.random.default_rng(13)
    n, dm = 300, 64
    Hp = _bf16(rng.standard_normal((n, dm)))
    mag = np.full(n, 0.01, np.float32)
    prev = np.zeros(n, bool)
    prev[rng.choice(n, 120, replace=False)] = True
    planted = rng.choice(np.nonzero(prev)[0], 9, replace=False)
    mag[planted] = 0.1
    decoy = np.nonzero(~prev)[0][:5]
    mag[decoy] = 1.0            # large changes outside the preceding set do not count
    Hc = _bf16(Hp + mag[:, None] * rng.standard_normal((n, dm)).astype(np.float32))
    sel = orc.select_tokens(Hc, Hp, prev, 9)
    assert list(sel) == sorted(planted.tolist())
    sel30 = orc.select_tokens(Hc, Hp, prev, 30)
    assert set(sel30) <= set(np.nonzero(prev)[0]) and set(planted) <= set(sel30) and len(sel30) == 30
    assert np.all(np.diff(sel30) > 0)
    allp = orc.select_tokens(Hc, Hp, prev, 500)
    assert np.array_equal(allp, np.nonzero(prev)[0])


def test_ties_go_to_the_lower_index(orc):
    n, dm = 10, 8
    Hp = np.ones((n, dm), np.float32)
    Hc = Hp.copy()
    Hc[[2, 4, 6, 8], 0] = 2.0      # four equal changes, three kept
    sel = orc.select_tokens(Hc, Hp, None, 3)
    assert list(sel) == [2, 4, 6]
