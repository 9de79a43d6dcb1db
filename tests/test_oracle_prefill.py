"""Pins of the oracle's prefill-side sparse loop (project page, The Method, after STEP 03:
selected tokens and keys in compact buffers; STEP 02 and explainer section 3: the rank-K
correction that keeps the cached mass) against facts fixed outside the oracle."""
import numpy as np
import torch

from quantized_kv_attention_amd import synth


def _bf(x):
    return synth.bf16_bits_to_float(synth.bf16_round_bits(np.asarray(x, np.float32)))


def _causal_ref(q, k, v):
    """fp64 causal attention by the library routine, and each row's log-sum-exp."""
    Q, K, V = (torch.from_numpy(np.asarray(a, np.float64)) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], is_causal=True, scale=1.0)[0]
    s = Q @ K.T
    n = s.shape[0]
    s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    return o.numpy(), torch.logsumexp(s, dim=1).numpy()


def test_all_columns_of_every_row_is_causal_attention(orc):
    # every token active and every column selected: m_i = 1 and the corrected output is the
    # loop's own causal attention (o0 = the preceding loop's causal attention)
    rng = np.random.default_rng(21)
    n, d = 40, 16
    q0, k0, v0 = (_bf(rng.standard_normal((n, d)) * s) for s in (0.4, 1.0, 1.0))
    q1, k1, v1 = (_bf(a + 0.2 * rng.standard_normal((n, d))) for a in (q0, k0, v0))
    o0, lse0 = _causal_ref(q0, k0, v0)
    o1, _ = _causal_ref(q1, k1, v1)
    pos = np.arange(n)
    O, mass = orc.prefill_sparse(q1, q0, pos, lse0, o0, k1, v1, k0, v0, pos)
    np.testing.assert_allclose(mass, 1.0, rtol=1e-12)
    np.testing.assert_allclose(O, o1, rtol=0, atol=1e-12)


def test_rows_without_visible_columns_keep_their_output(orc):
    rng = np.random.default_rng(22)
    d = 8
    q = _bf(rng.standard_normal((3, d)))
    k = _bf(rng.standard_normal((2, d)))
    o0 = rng.standard_normal((3, d))
    O, mass = orc.prefill_sparse(q, q, [1, 4, 9], np.zeros(3), o0, k, k, k, k, [5, 7])
    np.testing.assert_array_equal(O[:2], o0[:2])
    assert list(mass[:2]) == [0.0, 0.0] and mass[2] > 0
    O, mass = orc.prefill_sparse(q, q, [1, 4, 9], np.zeros(3), o0, k[:0], k[:0], k[:0], k[:0], [])
    np.testing.assert_array_equal(O, o0)


def test_one_visible_column_closed_form(orc):
    # one visible column: alpha = 1, o = o0 + (m - p) v with m = p, i.e. o0 + p (v - v0)
    rng = np.random.default_rng(23)
    d = 8
    q, q0 = _bf(rng.standard_normal((1, d))), _bf(rng.standard_normal((1, d)))
    k, k0, v, v0 = (_bf(rng.standard_normal((1, d))) for _ in range(4))
    o0 = rng.standard_normal((1, d))
    lse0 = 0.7
    O, mass = orc.prefill_sparse(q, q0, [3], [lse0], o0, k, v, k0, v0, [2])
    p = np.exp(float(q0[0].astype(np.float64) @ k0[0].astype(np.float64)) - lse0)
    assert abs(mass[0] - p) <= 1e-15 * p
    np.testing.assert_allclose(O[0], o0[0] + p * (v[0].astype(np.float64) - v0[0]), rtol=1e-12, atol=1e-12)


def test_last_row_equals_the_decode_splice(orc):
    # the last active row sees every selected column: the decode splice of the same set
    rng = np.random.default_rng(24)
    n, d = 60, 16
    K0 = _bf(rng.standard_normal((n, d)))
    V0 = _bf(rng.standard_normal((n, d)))
    K1, V1 = _bf(K0 + 0.1 * rng.standard_normal((n, d))), _bf(V0 + 0.1 * rng.standard_normal((n, d)))
    q0 = _bf(0.3 * rng.standard_normal(d))
    q1 = _bf(q0 + 0.05 * rng.standard_normal(d))
    o0, sc0, lse0 = orc.attend_dense(q0, K0, V0)
    sel = np.sort(rng.choice(n, 9, replace=False)).astype(np.int32)
    p = np.exp(sc0[sel] - lse0)
    o_dec, _ = orc.attend_sparse(q1, K1, V1, V0, sel, p, float(p.sum()), o0, lse0, sc0)
    O, mass = orc.prefill_sparse(q1[None], q0[None], [n - 1], [lse0], o0[None], K1[sel], V1[sel], K0[sel], V0[sel],
                                 sel)
    np.testing.assert_allclose(mass[0], p.sum(), rtol=1e-13)
    np.testing.assert_allclose(O[0], o_dec, rtol=0, atol=1e-13)
