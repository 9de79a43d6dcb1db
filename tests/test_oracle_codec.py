"""Pins of the oracle's INT4 residual codec against facts fixed outside the oracle.

Codec as described on the pages (flozi.net explainer section 3; project page STEP 03):
asymmetric group-wise 4-bit quantization with group 64, keys per channel over 64
tokens, values per token over 64 channels, loop 1 as base and later loops as the
residual against the previous loop's reconstruction.
"""
import numpy as np
import pytest


def f32(x):
    return np.float32(x)


def bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


# ---------------------------------------------------------------- quantizer ------
@pytest.mark.parametrize("value", [0.0, 1.0, -3.25, 1e-30, -7.0e5, 1e-41])
def test_constant_group_reconstructs_exactly(orc, value):
    x = np.full(64, value, np.float32)
    c, s, z = orc.quantize_group(x)
    assert s == 0.0 and np.all(c == 0)
    deq = orc.dequant(c, s, z)
    assert np.array_equal(bits(deq), bits(x))


def test_negative_zero_group_canonical(orc):
    x = np.full(64, -0.0, np.float32)
    c, s, z = orc.quantize_group(x)
    assert bits(s) == 0 and bits(z) == 0, "s and z are stored as +0"


def test_grid_roundtrip_exact(orc):
    # values on a 16-level grid whose step and offset are exact in fp32: the codes,
    # the scale and the zero point come back exactly
    rng = np.random.default_rng(1)
    for s0, z0 in [(0.25, -1.5), (2.0 ** -10, 3.0), (8.0, -64.0)]:
        c0 = rng.integers(0, 16, 64)
        c0[3], c0[40] = 0, 15
        x = (z0 + c0 * s0).astype(np.float32)
        c, s, z = orc.quantize_group(x)
        assert s == f32(s0) and z == f32(z0)
        assert np.array_equal(c, c0.astype(np.uint8))
        assert np.array_equal(orc.dequant(c, s, z), x)


def test_hand_example_and_half_even(orc):
    # min 0, max 15 -> s = 1, z = 0; 7.5 rounds to 8 and 2.5 to 2 (half to even)
    x = np.array([0.0, 7.5, 15.0, 11.25, 2.5, 3.5], np.float32)
    c, s, z = orc.quantize_group(x)
    assert s == 1.0 and z == 0.0
    assert list(c) == [0, 8, 15, 11, 2, 4]


def test_error_bound_random(orc):
    rng = np.random.default_rng(2)
    for _ in range(200):
        x = (rng.standard_normal(64) * rng.uniform(0.01, 100)).astype(np.float32)
        c, s, z = orc.quantize_group(x)
        assert c.max() <= 15
        deq = orc.dequant(c, s, z).astype(np.float64)
        xd = x.astype(np.float64)
        # half a step plus a few fp32 ulps of the operands
        tol = float(s) / 2 * (1 + 1e-6) + 4 * np.spacing(np.float32(np.abs(x).max()))
        assert np.max(np.abs(deq - xd)) <= tol
        assert deq.min() >= float(z) - 1e-30 or np.isclose(deq.min(), z)
        # both extremes are hit exactly by codes 0 and 15 up to rounding of s
        assert c[np.argmin(x)] == 0 and c[np.argmax(x)] == 15


def test_short_group(orc):
    x = np.array([1.0, 4.0], np.float32)
    c, s, z = orc.quantize_group(x)
    assert s == f32(3.0) / f32(15.0) and z == 1.0 and list(c) == [0, 15]


# ---------------------------------------------------------------- encode rows ----
def test_keys_are_grouped_per_channel(orc):
    # each channel constant over its 64 rows, channels all different: only a per-channel
    # grouping reconstructs this exactly (a per-token grouping would not)
    rng = np.random.default_rng(3)
    d = 128
    col = rng.standard_normal(d).astype(np.float32)
    X = np.tile(col, (64, 1))
    codes, s, z, R = orc.encode_rows(X, None, is_key=True)
    assert s.shape == (1, d) and np.all(s == 0)
    assert np.array_equal(R, X)
    # the same data as values (per token over 64 channels) is not exact
    _, _, _, Rv = orc.encode_rows(X, None, is_key=False)
    assert not np.array_equal(Rv, X)


def test_values_are_grouped_per_token(orc):
    rng = np.random.default_rng(4)
    d = 128
    row = rng.standard_normal(64).astype(np.float32)
    # rows constant within each 64-channel group, different per row and per group
    X = np.concatenate([np.repeat(row[:, None], 64, 1), np.repeat(row[::-1, None], 64, 1)], 1)
    codes, s, z, R = orc.encode_rows(X, None, is_key=False)
    assert s.shape == (64, 2) and np.all(s == 0)
    assert np.array_equal(R, X)
    assert np.array_equal(z[:, 0], row) and np.array_equal(z[:, 1], row[::-1])
    _, _, _, Rk = orc.encode_rows(X, None, is_key=True)
    assert not np.array_equal(Rk, X)


def test_key_groups_follow_stored_rows(orc):
    # 100 stored rows -> groups rows [0,64) and [64,100); an outlier in row 10 of
    # channel 3 widens only group 0's channel-3 scale
    rng = np.random.default_rng(5)
    X = rng.standard_normal((100, 64)).astype(np.float32)
    X[10, 3] = 1000.0
    codes, s, z, R = orc.encode_rows(X, None, is_key=True)
    assert s.shape == (2, 64)
    assert s[0, 3] > 60 and s[1, 3] < 1.0
    # group 1 is quantized from rows 64..99 alone
    c1, s1, z1 = orc.quantize_group(X[64:, 7])
    assert s[1, 7] == s1 and z[1, 7] == z1 and np.array_equal(codes[64:, 7], c1)


def test_residual_against_reconstruction_error_feedback(orc):
    # loop 2 stores X2 - Xhat1; its error is bounded by loop 2's own half step,
    # it does not carry loop 1's quantization error
    rng = np.random.default_rng(6)
    X1 = rng.standard_normal((64, 128)).astype(np.float32)
    X2 = (X1 + 0.05 * rng.standard_normal((64, 128))).astype(np.float32)
    for is_key in (True, False):
        _, s1, _, R1 = orc.encode_rows(X1, None, is_key)
        _, s2, _, R2 = orc.encode_rows(X2, R1, is_key)
        err1 = np.abs(R1.astype(np.float64) - X1)
        err2 = np.abs(R2.astype(np.float64) - X2)
        half2 = (np.repeat(s2, 64, axis=1) if not is_key else np.broadcast_to(s2, (64, 128))) / 2
        assert np.all(err2 <= half2 * (1 + 1e-5) + 1e-6)
        assert err2.max() < 0.5 * err1.max()
        # the stored residual plus the previous reconstruction is the new reconstruction
        assert np.all(np.isfinite(R2))


def test_loop1_is_plain_quantization(orc):
    rng = np.random.default_rng(7)
    X = rng.standard_normal((64, 64)).astype(np.float32)
    codes, s, z, R = orc.encode_rows(X, None, True)
    for ch in (0, 17, 63):
        c, sc, zc = orc.quantize_group(X[:, ch])
        assert np.array_equal(codes[:, ch], c) and s[0, ch] == sc and z[0, ch] == zc
        assert np.array_equal(R[:, ch], orc.dequant(c, sc, zc))
