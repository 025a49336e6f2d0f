"""Pins for the oracle's number formats (CPU only).

Each test checks the oracle against something other than itself: the OCP
format tables stored under tests/golden (with their sources), an independent
closed-form rounding formula, torch's float8_e4m3fn / bfloat16 casts, and
exhaustive enumeration.
"""
import os

import numpy as np
import pytest
import torch

from oracle import quads_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


# P1 -- the E2M1 level set (eight magnitudes per sign)
def test_e2m1_decode_matches_format_table():
    rows = _rows("e2m1_levels.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = O.e2m1_decode(int(code))
        assert float(got) == float(val)
        assert np.signbit(got) == val.startswith("-")
    mags = sorted({abs(float(O.e2m1_decode(c))) for c in range(16)})
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_tie_table():
    for vin, lvl, code in _rows("e2m1_ties.txt"):
        idx = int(O.e2m1_round_magnitude(np.array([float(vin)]))[0])
        assert idx == int(code), vin
        assert O.E2M1_MAGNITUDES[idx] == float(lvl)


def _e2m1_rne_closed_form(v):
    """Independent formula: round-half-even to the binade's spacing
    (0.5 below 2, then 2^(e-1)), saturating at 6."""
    v = np.asarray(v, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(v, 1e-300)))
    e = np.clip(e, 1, 2)            # spacing 0.5 for v<2 (binades [0,1) and [1,2))
    spacing = np.where(v < 2, 0.5, 2.0 ** (e - 1))
    q = np.rint(v / spacing) * spacing  # numpy rint is round-half-even
    q = np.minimum(q, 6.0)
    levels = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    idx = np.searchsorted(levels, q)
    assert np.array_equal(levels[idx], q)
    return idx


@pytest.mark.slow
def test_e2m1_round_exhaustive_binades():
    """P2: every fp32 value with exponent in [-4, 3] (i.e. [1/16, 16)) plus 0,
    compared with the independent closed form."""
    for ex in range(-4, 4):
        base = np.uint32((ex + 127) << 23)
        bits = base + np.arange(1 << 23, dtype=np.uint32)
        v = bits.view(np.float32)
        got = O.e2m1_round_magnitude(v)
        ref = _e2m1_rne_closed_form(v)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (ex, v[bad[:5]], got[bad[:5]], ref[bad[:5]])
    assert O.e2m1_round_magnitude(np.array([0.0, 1e-30, 0.0624]))[()].tolist() == [0, 0, 0]


def test_e2m1_round_near_ties():
    """Every tie and its fp32 neighbours (±1..3 ulp)."""
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    vals = []
    for t in ties:
        b = np.array([t], dtype=np.float32).view(np.uint32)[0]
        for d in range(-3, 4):
            vals.append(np.array([b + np.uint32(d) if d >= 0 else b - np.uint32(-d)], dtype=np.uint32).view(np.float32)[0])
    vals = np.array(vals, dtype=np.float32)
    assert np.array_equal(O.e2m1_round_magnitude(vals), _e2m1_rne_closed_form(vals))


# P3 -- E4M3
def test_e4m3_points_fixture():
    for vin, code in _rows("e4m3_points.txt"):
        assert int(O.e4m3_encode(np.array([float(vin)]))[0]) == int(code, 16), vin


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(127, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(O.e4m3_decode(codes), ref)


def test_e4m3_encode_vs_torch_dense():
    """Dense sweep over [0, 448]: all fp32 values near every E4M3 value and
    midpoint, plus 2M log-uniform random values, against torch's RNE cast."""
    rng = np.random.default_rng(11)
    t = O.E4M3_VALUES
    mids = (t[:-1] + t[1:]) / 2
    pts = np.concatenate([t, mids]).astype(np.float32)
    b = pts.view(np.uint32).astype(np.int64)
    near = (b[:, None] + np.arange(-4, 5)[None, :]).clip(0).astype(np.uint32).view(np.float32).reshape(-1)
    rnd = np.exp2(rng.uniform(-13, np.log2(448.0), 2_000_000)).astype(np.float32)
    v = np.concatenate([near, rnd, np.array([0.0], np.float32)])
    v = v[(v >= 0) & (v <= 448)]
    got = O.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (v[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_e4m3_saturates():
    v = np.array([448.0, 449.0, 464.0, 470.0, 480.0, 1e30], dtype=np.float64)
    assert (O.e4m3_encode(v) == 0x7E).all()


def test_e4m3_encode_brute_force_nearest():
    """Brute force: nearest of the 127 finite codes with ties to the even code."""
    rng = np.random.default_rng(12)
    v = np.exp2(rng.uniform(-12, 9, 20000))
    got = O.e4m3_encode(v)
    for x, c in zip(v[:3000], got[:3000]):
        d = np.abs(O.E4M3_VALUES - x)
        m = d.min()
        cands = np.nonzero(d == m)[0]
        exp = cands[0] if len(cands) == 1 else [c2 for c2 in cands if c2 % 2 == 0][0]
        if x >= 448:
            exp = 0x7E
        assert c == exp


# bf16 rounding used by the QDQ output
def test_bf16_rounding_vs_torch():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal(1_000_000) * np.exp2(rng.uniform(-30, 30, 1_000_000))).astype(np.float32)
    b = x.view(np.uint32)
    ties = ((b & 0xFFFF0000) | 0x8000).view(np.float32)  # exact halfway cases
    x = np.concatenate([x, ties])
    got = O.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_pack_nibbles_roundtrip_and_order():
    code = np.arange(32, dtype=np.uint8).reshape(2, 16) & 0xF
    p = O.pack_nibbles(code)
    assert p[0, 0] == (0 | (1 << 4))
    assert np.array_equal(O.unpack_nibbles(p), code)
