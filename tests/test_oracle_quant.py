"""Pins for the oracle's NVFP4 quantizer and weight QDQ (CPU only).

Pins used: brute force over all 16 codes in exact rational arithmetic,
exactly representable inputs (the quantizer must be the identity on the
NVFP4 grid), closed-form scale bounds, and QDQ idempotence.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import synthetic as S


def _levels():
    return [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def test_tensor_scale_closed_form():
    rng = np.random.default_rng(21)
    for _ in range(50):
        x = (rng.standard_normal((8, 32)) * np.exp2(rng.uniform(-20, 20))).astype(np.float32)
        g = O.tensor_scale(x)
        a = np.abs(x).max()
        # g is a/2688 rounded once to fp32
        assert abs(Fraction(float(g)) - Fraction(float(a)) / 2688) <= Fraction(float(g)) * Fraction(1, 2 ** 24)
    assert O.tensor_scale(np.zeros((2, 16), np.float32)) == np.float32(1.0)


def test_quantizer_brute_force_codes():
    """P8: each code is the one of 16 minimizing |x - level·d| exactly, with
    ties to the even magnitude index and the sign bit of x; scales satisfy the
    E4M3 rounding bound of amax_b/(6g)."""
    rng = np.random.default_rng(22)
    x = rng.standard_normal((6, 64)).astype(np.float32)
    x[:, 5] *= 25
    x[2, 16:32] = 0.0
    x[3, 40] = -0.0
    q = O.quantize_nvfp4(x)
    code = O.unpack_nibbles(q.codes)
    L = _levels()
    g = Fraction(float(q.g))
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 16):
            blk = x[r, 16 * b:16 * b + 16]
            s = int(q.scales[r, b])
            ds = Fraction(float(O.e4m3_decode(s)))
            # scale is the nearest E4M3 value to amax/(6g) (within fp32 rounding of the quotient)
            s_real = Fraction(float(np.abs(blk).max())) / 6 / g
            spacing = Fraction(float(O.E4M3_VALUES[min(s + 1, 126)] - O.E4M3_VALUES[s])) if s < 126 else Fraction(64)
            assert abs(ds - s_real) <= spacing * Fraction(1, 2) * (1 + Fraction(1, 2 ** 20)) or s == 0x7E
            d = Fraction(float(np.float32(np.float32(O.e4m3_decode(s)) * q.g)))
            for i, xv in enumerate(blk):
                c = int(code[r, 16 * b + i])
                assert (c >> 3) == int(np.signbit(xv))
                if d == 0:
                    assert c & 7 == 0
                    continue
                ax = abs(Fraction(float(xv)))
                dist = [abs(ax - lv * d) for lv in L]
                m = min(dist)
                cands = [k for k in range(8) if dist[k] == m]
                exp = cands[0] if len(cands) == 1 else [k for k in cands if k % 2 == 0][0]
                assert (c & 7) == exp, (r, b, i, float(xv))


def _grid_tensor(rng, rows, cols, g):
    """Values level·dec(s)·g with every block holding a 6 so its amax is
    6·dec(s)·g: exactly representable, so quantization must return it."""
    lv = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    sc = O.E4M3_VALUES[rng.integers(40, 126, (rows, cols // 16))]
    sc[:, 0] = 448.0  # tensor amax = 6·448·g, so tensor_scale(x) == g
    m = lv[rng.integers(0, 8, (rows, cols))] * np.where(rng.random((rows, cols)) < 0.5, -1, 1)
    m[:, ::16] = 6.0
    x = m * np.repeat(sc, 16, axis=1) * g
    return x.astype(np.float32), sc


def test_quantizer_identity_on_grid():
    """P13 (first half): an exactly representable tensor quantizes to itself,
    so ΔX = 0 and every channel score is 0."""
    rng = np.random.default_rng(23)
    g = np.float32(2.0 ** -7)
    x, sc = _grid_tensor(rng, 12, 128, g)
    q = O.quantize_nvfp4(x)
    assert q.g == g
    assert np.array_equal(O.e4m3_decode(q.scales), sc)
    assert np.array_equal(q.dq, x)
    assert np.array_equal(O.dequant_exact(q.codes, q.scales, q.g), x.astype(np.float64))
    assert (O.rac_scores(x, q) == 0).all()


def test_dequant_f32_matches_quantizer_dq():
    rng = np.random.default_rng(24)
    x = rng.standard_normal((9, 48)).astype(np.float32)
    q = O.quantize_nvfp4(x)
    assert np.array_equal(O.dequant_f32(q.codes, q.scales, q.g), q.dq)
    # exact and fp32 dequant agree to fp32 rounding
    ex = O.dequant_exact(q.codes, q.scales, q.g)
    assert np.allclose(ex, q.dq, rtol=2 ** -23, atol=0)


def test_zero_and_signed_zero():
    x = np.zeros((2, 16), np.float32)
    x[1, 3] = -0.0
    q = O.quantize_nvfp4(x)
    code = O.unpack_nibbles(q.codes)
    assert q.g == 1.0 and (q.scales == 0).all()
    assert code[1, 3] == 8 and code[0, 3] == 0


def test_qdq_idempotent_fixed_g():
    """P4: with g held fixed, Q(QDQ(W)) reproduces codes and scales bit-exactly
    and QDQ(QDQ(W)) == QDQ(W), for fp32 and bf16 masters."""
    rng = np.random.default_rng(25)
    for bf16 in (False, True):
        w = S.weights(rng, (64, 256), 0.02, bf16=bf16).f32
        b1, q1 = O.weight_qdq(w)
        # precondition: no deep-subnormal block scales
        blk = np.abs(w).reshape(64, 16, 16).max(2)
        assert ((blk == 0) | (blk / 6 / q1.g > 5 * 2 ** -10)).all()
        w1 = O.f32_from_bf16_bits(b1) if bf16 else q1.dq
        b2, q2 = O.weight_qdq(w1, g=q1.g)
        assert np.array_equal(q2.codes, q1.codes)
        assert np.array_equal(q2.scales, q1.scales)
        assert np.array_equal(b2, b1)


def test_qdq_recomputed_g_keeps_codes():
    rng = np.random.default_rng(26)
    w = S.weights(rng, (32, 512), 0.02, bf16=True).f32
    b1, q1 = O.weight_qdq(w)
    b2, q2 = O.weight_qdq(O.f32_from_bf16_bits(b1))
    assert np.array_equal(q2.codes, q1.codes)
    assert np.array_equal(q2.scales, q1.scales)
    d = np.abs(O.f32_from_bf16_bits(b2).astype(np.float64) - O.f32_from_bf16_bits(b1))
    assert (d <= np.abs(O.f32_from_bf16_bits(b1)) * 2 ** -8).all()


def test_qdq_matches_quantizer():
    """P11: the QDQ path's codes/scales/g are the quantizer's; its values are
    bf16(dq)."""
    rng = np.random.default_rng(27)
    w = S.weights(rng, (16, 64), 0.02, bf16=True).f32
    b, qq = O.weight_qdq(w)
    q = O.quantize_nvfp4(w)
    assert np.array_equal(qq.codes, q.codes) and np.array_equal(qq.scales, q.scales) and qq.g == q.g
    assert np.array_equal(b, O.bf16_bits_from_f32(q.dq))


def test_quantize_rejects_bad_shapes():
    with pytest.raises(ValueError):
        O.quantize_nvfp4(np.zeros((2, 10), np.float32))
    with pytest.raises(ValueError):
        O.quantize_nvfp4(np.full((1, 16), np.inf, np.float32))
