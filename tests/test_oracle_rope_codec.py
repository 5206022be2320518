"""Pins for the oracle's RoPE and int4 codec (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import brute, codec, rope


# ----------------------------------------------------------------------------- RoPE

def test_rope_two_dims_is_plane_rotation():
    """d_h = 2: theta_0 = 1, so RoPE is the plane rotation by the position angle."""
    x = np.array([0.3, -1.7])
    for pos in (0, 1, 5, 1000):
        c, s = np.cos(pos), np.sin(pos)
        np.testing.assert_allclose(rope.rope(x, pos, 1e4), [c * x[0] - s * x[1], s * x[0] + c * x[1]],
                                   atol=1e-12)


def test_rope_freqs():
    f = rope.freqs(128, 1e4)
    assert f[0] == 1.0
    assert abs(f[1] - 1e4 ** (-2 / 128)) < 1e-16
    assert abs(f[63] - 1e4 ** (-126 / 128)) < 1e-18


def test_rope_preserves_norm_and_relative_position():
    rng = np.random.default_rng(0)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for base in (1e4, 5e5):
        assert abs(np.linalg.norm(rope.rope(k, 777, base)) - np.linalg.norm(k)) < 1e-12
        ref = rope.rope(q, 50, base) @ rope.rope(k, 20, base)
        for shift in (1, 999, 65000):
            got = rope.rope(q, 50 + shift, base) @ rope.rope(k, 20 + shift, base)
            assert abs(got - ref) < 1e-9


def test_rope_inverse_and_identity():
    """The explicit inverse of the Shard post (section 5) recovers the key exactly."""
    rng = np.random.default_rng(1)
    k = rng.standard_normal((9, 64))
    pos = np.arange(9) * 1234
    np.testing.assert_allclose(rope.unrope(rope.rope(k, pos, 1e4), pos, 1e4), k, atol=1e-12)
    np.testing.assert_array_equal(rope.rope(k, pos, 0), k)
    np.testing.assert_allclose(rope.rope(k, 0, 1e4), k, atol=0)


def test_rope_matches_brute_force():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(8)
    for pos in (0, 3, 17):
        np.testing.assert_allclose(rope.rope(x, pos, 1e4), brute.rope_vec(list(x), pos, 1e4), atol=1e-13)


# ----------------------------------------------------------------------------- int4 codec

def _group(values, amax=7.0):
    g = np.zeros(32, np.float32)
    g[0] = amax
    g[1:1 + len(values)] = values
    return g


def test_int4_ties_round_half_even():
    # amax 7 -> s32 = 1 exactly -> s16 = 1, so x/s16 = x
    g = _group([2.5, 3.5, -2.5, 0.5, 1.5, 6.5, -6.5, -0.5, 4.5])
    codes, scales = codec.quantize(g[None])
    assert scales[0, 0] == np.float16(1.0)
    assert list(codes[0, :10]) == [7, 2, 4, -2, 0, 2, 6, -6, 0, 4]


def test_int4_ties_with_inexact_scale():
    # amax 1 -> s32 = fp32(1/7) -> s16 = fp16(that); ties are k + 1/2 of s16 itself
    s16 = np.float16(np.float32(1.0) / np.float32(7.0))
    vals = [np.float32(np.float64(s16) * (k + 0.5)) for k in (0, 1, 2, 3, -1, -4)]
    g = _group(vals, amax=1.0)
    codes, scales = codec.quantize(g[None])
    assert scales[0, 0] == s16
    exact = [float(Fraction(float(v)) / Fraction(float(s16))) for v in vals]
    assert exact == [0.5, 1.5, 2.5, 3.5, -0.5, -3.5]        # really ties
    assert list(codes[0, 1:7]) == [0, 2, 2, 4, 0, -4]


def test_int4_matches_exact_rational_rounding():
    """Brute force with exact rationals: code = round-half-even(x / s16), clamped."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((200, 64)) * rng.uniform(0.01, 50, (200, 1))).astype(np.float32)
    # plant near-ties and exact ties
    codes, scales = codec.quantize(x)
    for i in range(0, 200, 7):
        for j in range(64):
            s = Fraction(float(scales[i, j // 32]))
            q = Fraction(float(x[i, j])) / s if s else Fraction(0)
            fl = q.numerator // q.denominator
            rem = q - fl
            k = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)
            k = max(-7, min(7, k)) if s else 0
            assert codes[i, j] == k


def test_int4_scale_rule_and_bounds():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((500, 32)) * 3).astype(np.float32)
    codes, scales = codec.quantize(x)
    amax = np.abs(x).max(axis=1)
    np.testing.assert_array_equal(scales[:, 0], (amax / np.float32(7)).astype(np.float32).astype(np.float16))
    xhat = codec.dequantize(codes, scales)
    assert np.all(np.abs(x - xhat) <= scales.astype(np.float32) / 2 * (1 + 1e-6) + 1e-30)
    arg = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(codes[np.arange(500), arg]) == 7)
    assert codes.min() >= -7 and codes.max() <= 7


def test_int4_degenerate_groups():
    x = np.zeros((3, 32), np.float32)
    x[1, 5] = -0.75                                 # single nonzero element
    x[2, 0] = 1e6                                   # scale overflows fp16 -> saturate
    codes, scales = codec.quantize(x)
    assert scales[0, 0] == 0 and not codes[0].any()
    assert codes[1, 5] == -7 and np.count_nonzero(codes[1]) == 1
    assert scales[2, 0] == np.float16(65504.0)
    assert codes[2, 0] == 7                          # 1e6 / 65504 = 15.3 -> clamp


def test_int4_pack_layout():
    codes = np.array([[1, -1, -8, 7, 0, -2]], np.int8)
    packed = codec.pack(codes)
    assert list(packed[0]) == [0xF1, 0x78, 0xE0]
    np.testing.assert_array_equal(codec.unpack(packed), codes)
    rng = np.random.default_rng(5)
    c = rng.integers(-7, 8, (10, 64)).astype(np.int8)
    np.testing.assert_array_equal(codec.unpack(codec.pack(c)), c)


def test_int4_dequant_exact():
    codes = np.arange(-7, 8, dtype=np.int8)[None].repeat(1, 0)
    codes = np.concatenate([codes, np.zeros((1, 17), np.int8)], axis=1)
    s = np.array([[np.float16(0.3333)]])
    out = codec.dequantize(codes, s)
    assert np.array_equal(out[0, :15], np.arange(-7, 8).astype(np.float32) * np.float32(np.float16(0.3333)))


def test_int4_rejects_bad_width():
    with pytest.raises(ValueError):
        codec.quantize(np.zeros((2, 48), np.float32))
