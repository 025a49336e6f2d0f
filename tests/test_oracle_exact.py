"""Exact pins of the oracle's FP32 / FP16 step sequences (CPU only).

The merged RAC operand and the FP32 dequantized value are fixed step by step
(which products and sums are rounded, to which format, in which order), so
they are pinned by re-evaluating each step in exact rational arithmetic
(``tests/exact_float.py``) with the element values decoded from the E2M1 and
E4M3 bit fields -- no NumPy float arithmetic and no oracle helper takes part
in the expected values.  For each plausible mistake in the rounding sequence
(rounding both terms to fp16 before the sum, forming R'*g_r before dividing
by g_x, contracting the product into the sum, truncating instead of rounding
to nearest-even), a case is constructed on which that variant gives
different bits from the definition, so a mutated oracle fails the pin.

Definitions (the correction is added to the quantized activation before the
GEMM: AI-Wiki "Methodology"; the residual of the masked channels is
quantized a second time and added to the quantized path: gist.science
"Technische Samenvatting: QUADS" section 2.2-B):
  ratio = fl32(g_r / g_x)
  merged[r, sel_j] = fp16( fl32( X'[r, sel_j] + fl32(R'[r, j] * ratio) ) )
  merged[r, c]     = X'[r, c] for unselected c
  dequant_f32      = sign * fl32(level * fl32(dec(s) * g))
"""
from fractions import Fraction

import numpy as np

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import synthetic as S
from tests.exact_float import (e2m1_value, e4m3_value, f16_bits, frac, nvfp4_element, rnd16, rnd32)

# ---------------------------------------------------------------------------
# the definitions, evaluated exactly (signed zeros tracked per IEEE 754 RNE)
# ---------------------------------------------------------------------------


def _code(codes, r, c):
    byte = int(codes[r, c // 2])
    return byte & 0xF if c % 2 == 0 else byte >> 4


def _add(a, a_neg, b, b_neg):
    """Exact sum of two signed-zero-aware values -> (value, sign of a zero)."""
    s = a + b
    if s != 0:
        return s, s < 0
    if a == 0 and b == 0:
        return s, a_neg and b_neg
    return s, False  # x + (-x) = +0 under round-to-nearest


def _bits16(v, neg_zero):
    if v == 0:
        return 0x8000 if neg_zero else 0
    return f16_bits(v)


def merged_element(xv, x_neg, rv, r_neg, ratio, variant="definition"):
    """fp16 bits of one selected element of the merged operand.  xv, rv:
    exact X' and R' values; x_neg, r_neg: their sign bits (for zeros)."""
    if variant == "fp16_terms":  # fp16(X') + fp16(cor), summed in fp16
        cor = rnd32(rv * ratio)
        cor_neg = r_neg if cor == 0 else cor < 0
        a, b = rnd16(xv), rnd16(cor)
        s, neg = _add(a, x_neg if a == 0 else a < 0, b, cor_neg if b == 0 else b < 0)
        out = rnd16(s)
        return _bits16(out, neg if out == 0 else out < 0)
    if variant == "contracted":  # X' + R' * ratio with the product unrounded
        exact, s_neg = _add(xv, x_neg, rv * ratio, r_neg)
        s = rnd32(exact)
        s_neg = s_neg if s == 0 else s < 0
    else:
        if variant == "product_first":  # fl32(fl32(R' * g_r) / g_x)
            cor = rnd32(rnd32(rv * ratio[0]) / ratio[1])
        else:
            cor = rnd32(rv * ratio)
        cor_neg = r_neg if cor == 0 else cor < 0
        exact, s_neg = _add(xv, x_neg, cor, cor_neg)
        s = rnd32(exact)
        s_neg = s_neg if s == 0 else s < 0
    out = rnd16(s, "trunc" if variant == "truncate" else "rne")
    return _bits16(out, s_neg if out == 0 else out < 0)


def merged_pin(q, r, sel, nsel, variant="definition"):
    """uint16 [rows, cols]: the merged operand from the definition (or a
    named variant of it), element by element in exact arithmetic."""
    rows, cols = q.codes.shape[0], q.codes.shape[1] * 2
    gx, gr = frac(np.float32(q.g)), frac(np.float32(r.g))
    ratio = (gr, gx) if variant == "product_first" else rnd32(gr / gx)
    pos = {int(c): j for j, c in enumerate(sel[:nsel])}
    out = np.empty((rows, cols), dtype=np.uint16)
    for i in range(rows):
        for c in range(cols):
            xv = nvfp4_element(q.codes, q.scales, i, c)
            x_neg = bool(_code(q.codes, i, c) & 8)
            if c in pos:
                j = pos[c]
                rv = nvfp4_element(r.codes, r.scales, i, j)
                r_neg = bool(_code(r.codes, i, j) & 8)
                out[i, c] = merged_element(xv, x_neg, rv, r_neg, ratio, variant)
            else:
                out[i, c] = _bits16(rnd16(xv), x_neg)
    return out


def _bits(a16):
    return np.asarray(a16, dtype=np.float16).view(np.uint16)


# ---------------------------------------------------------------------------
# the oracle equals the definition
# ---------------------------------------------------------------------------


def test_merged_operand_equals_exact_definition():
    """Seeded activations with outlier channels (k = 25, 50, 100, one nsel not
    a multiple of 16): every element of the oracle's merged operand has the
    bits of the exactly evaluated definition."""
    rng = np.random.default_rng(91)
    for M, K, k in ((24, 256, 50), (16, 128, 100), (20, 256, 25), (12, 208, 33)):
        x = S.activation(rng, M, K, 3, 20.0, bf16=False).f32
        q = O.quantize_nvfp4(x)
        sel, n = O.rac_select(O.rac_scores(x, q), k)
        r = O.rac_quantize_residual(x, q, sel, n)
        got = _bits(O.rac_merged_operand(q, r, sel, n))
        assert np.array_equal(got, merged_pin(q, r, sel, n)), (M, K, k)


# ---------------------------------------------------------------------------
# each rounding mistake is caught
# ---------------------------------------------------------------------------

_MUTATIONS = ("fp16_terms", "product_first", "contracted", "truncate")


def _hand_tensors(rng, reps):
    """A handcrafted NVFP4 activation X' and residual R' (one 16-block per
    row, every channel selected): residual rows run through every nonzero
    E4M3 scale byte with all 14 nonzero E2M1 codes and both zeros; the
    activation codes and scales are seeded random."""
    rows = 126 * reps
    rcode = np.tile(np.array([1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15, 0, 8], np.uint8), (rows, 1))
    rscale = np.tile(np.arange(1, 127, dtype=np.uint8), reps)[:, None]
    xcode = rng.integers(0, 16, (rows, 16)).astype(np.uint8)
    xscale = rng.integers(1, 127, (rows, 1)).astype(np.uint8)
    return O.pack_nibbles(xcode), xscale, O.pack_nibbles(rcode), rscale


def _np_values(codes, scales):
    """float64 values e2m1 * e4m3 via the bit-field decoders (search only)."""
    c = O.unpack_nibbles(codes)
    lv = np.vectorize(lambda v: float(e2m1_value(int(v))))(c)
    sv = np.vectorize(lambda v: float(e4m3_value(int(v))))(scales)
    return lv * np.repeat(sv, 16, axis=1)


def _np_variant(xv, rv, gx, gr, variant):
    """Fast float evaluation of a variant, used only to find candidate cases
    (IEEE float32 operations on float32 operands are correctly rounded; the
    candidates are then re-checked exactly)."""
    f32 = np.float32
    ratio = f32(f32(gr) / f32(gx))
    x32, r32 = xv.astype(f32), rv.astype(f32)
    if variant == "product_first":
        cor = ((r32 * f32(gr)).astype(f32) / f32(gx)).astype(f32)
    else:
        cor = (r32 * ratio).astype(f32)
    if variant == "contracted":
        s = (xv + rv * np.float64(ratio)).astype(f32)  # exact in float64 for these magnitudes, one rounding
    elif variant == "fp16_terms":
        return (x32.astype(np.float16) + cor.astype(np.float16)).astype(np.float16)
    else:
        s = (x32 + cor).astype(f32)
    return s.astype(np.float16)


def test_merged_pin_rejects_rounding_mutations():
    """For every mutation a seeded search over tensor scales finds a case on
    which the mutation's bits differ from the definition's (checked in exact
    arithmetic), while the oracle still equals the definition on that case."""
    rng = np.random.default_rng(92)
    xc, xs, rc, rs = _hand_tensors(rng, 4)
    xv, rv = _np_values(xc, xs), _np_values(rc, rs)
    sel = np.arange(16, dtype=np.int32)
    found = {}
    for trial in range(4000):
        gx = np.float32(rng.uniform(1e-3, 1.0))
        gr = np.float32(rng.uniform(1e-4, 1e-1) * gx)
        ref = _np_variant(xv, rv, gx, gr, "definition")
        for m in _MUTATIONS:
            if m in found:
                continue
            if m == "truncate":
                rows = np.arange(min(8, xv.shape[0]))  # truncation differs on about half the elements
            else:
                diff = np.nonzero((_np_variant(xv, rv, gx, gr, m).view(np.uint16) != ref.view(np.uint16)).any(1))[0]
                if diff.size == 0:
                    continue
                rows = diff[:4]
            q = O.NVFP4(xc[rows], xs[rows], gx, None, None, None)
            r = O.NVFP4(rc[rows], rs[rows], gr, None, None, None)
            want = merged_pin(q, r, sel, 16)
            if not np.array_equal(merged_pin(q, r, sel, 16, m), want):
                found[m] = (q, r, want)
        if len(found) == len(_MUTATIONS):
            break
    assert sorted(found) == sorted(_MUTATIONS), f"no distinguishing case for {set(_MUTATIONS) - set(found)}"
    for m, (q, r, want) in found.items():
        assert np.array_equal(_bits(O.rac_merged_operand(q, r, sel, 16)), want), m


# ---------------------------------------------------------------------------
# dequant_f32
# ---------------------------------------------------------------------------


def _f32_bits(v, neg):
    if v == 0:
        return 0x80000000 if neg else 0
    return int(np.array(float(v), dtype=np.float32).view(np.uint32))


def test_dequant_f32_exact_sequence():
    """dequant_f32 = sign * fl32(level * fl32(dec(s) * g)) for every code and
    every finite scale byte (subnormal scales included) under seeded tensor
    scales, evaluated exactly from the bit fields; with g = 1 both roundings
    are exact and it equals dequant_exact."""
    rng = np.random.default_rng(93)
    codes = np.tile(np.arange(16, dtype=np.uint8), (127, 1))  # row b: scale byte b, all 16 codes
    scales = np.arange(0, 127, dtype=np.uint8)[:, None]
    packed = O.pack_nibbles(codes)
    for g in [np.float32(1.0)] + [np.float32(v) for v in rng.uniform(1e-6, 3.0, 6)] + [np.float32(2.0 ** -100)]:
        got = O.dequant_f32(packed, scales, g).view(np.uint32)
        gq = frac(g)
        for b in range(127):
            d = rnd32(e4m3_value(b) * gq)
            for c in range(16):
                lvl = abs(e2m1_value(c))
                m = rnd32(lvl * d)
                want = _f32_bits(-m if c & 8 else m, bool(c & 8))
                assert got[b, c] == want, (float(g), b, c)
        if g == 1:
            ex = O.dequant_exact(packed, scales, g)
            assert np.array_equal(O.dequant_f32(packed, scales, g).astype(np.float64), ex)
