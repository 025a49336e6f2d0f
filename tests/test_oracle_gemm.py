"""Pins for the oracle's W4A4 (+RAC) GEMM reference (CPU only).

Pins: an exact rational triple loop over the NVFP4 definitions (catches a
transposed operand, a dropped residual term or a wrong scale); the
exactly-representable special case, where the whole path must reduce to the
textbook product X·Wᵀ; the k=0 reduction to plain W4A4; and the output-level
error comparison of RAC vs plain W4A4 on the seeded workloads.
"""
from fractions import Fraction

import numpy as np

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import synthetic as S


def _frac_dequant(codes, scales, g):
    lv = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    rows, half = codes.shape
    out = []
    for r in range(rows):
        row = []
        for c in range(half * 2):
            b = int(codes[r, c // 2])
            nib = (b >> (4 * (c % 2))) & 0xF
            v = lv[nib & 7] * Fraction(float(O.e4m3_decode(int(scales[r, c // 16])))) * Fraction(float(g))
            row.append(-v if nib & 8 else v)
        out.append(row)
    return out


def test_gemm_exact_triple_loop():
    """P8: 3x32 activations, 4x32 weights, k=50 -- Y from a Fraction triple
    loop over the NVFP4 definitions equals the oracle's float64 GEMM to
    float64 rounding."""
    rng = np.random.default_rng(51)
    x = rng.standard_normal((3, 32)).astype(np.float32)
    x[:, 7] *= 20
    w = (rng.standard_normal((4, 32)) * 0.02).astype(np.float32)
    qw = O.quantize_nvfp4(w)
    out = O.rac_linear(x, O.dequant_exact(qw.codes, qw.scales, qw.g)[None], 50)
    q, r, sel, n = out["q"], out["r"], out["sel"], out["nsel"]
    X = _frac_dequant(q.codes, q.scales, q.g)
    W = _frac_dequant(qw.codes, qw.scales, qw.g)
    R = _frac_dequant(r.codes, r.scales, r.g)
    for i in range(3):
        for j in range(4):
            acc = sum(W[j][k] * X[i][k] for k in range(32))
            acc += sum(W[j][int(sel[t])] * R[i][t] for t in range(len(sel)))
            assert abs(float(acc) - out["y"][i, j]) <= 1e-15 * max(1.0, abs(float(acc)))


def test_grid_inputs_reduce_to_textbook_matmul():
    """P13: if X and W lie on the NVFP4 grid, quantization is the identity, the
    residual is zero and Y == X·Wᵀ exactly, for any k."""
    rng = np.random.default_rng(52)
    lv = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)

    def grid(rows, cols, g):
        sc = O.E4M3_VALUES[rng.integers(48, 120, (rows, cols // 16))]
        sc[0, 0] = 448.0
        m = lv[rng.integers(0, 8, (rows, cols))] * np.where(rng.random((rows, cols)) < 0.5, -1, 1)
        m[:, ::16] = 6.0
        return (m * np.repeat(sc, 16, axis=1) * g).astype(np.float32)

    x = grid(16, 64, 2.0 ** -9)
    w = grid(24, 64, 2.0 ** -14)
    qw = O.quantize_nvfp4(w)
    assert np.array_equal(qw.dq, w)
    for k in (0, 50, 100):
        out = O.rac_linear(x, O.dequant_exact(qw.codes, qw.scales, qw.g)[None], k)
        assert (out["scores"] == 0).all()
        ref = x.astype(np.float64) @ w.astype(np.float64).T
        assert np.array_equal(out["y"], ref)


def test_k0_equals_plain_w4a4():
    """P5 at the GEMM level: with k=0 the RAC path is the plain W4A4 product."""
    wl = S.dense_small()
    qw = O.quantize_nvfp4(wl.w.f32)
    we = O.dequant_exact(qw.codes, qw.scales, qw.g)
    out = O.rac_linear(wl.x.f32, we[None], 0)
    xe = O.dequant_exact(out["q"].codes, out["q"].scales, out["q"].g)
    assert np.array_equal(out["y"], xe @ we.T)


def test_rac_error_not_larger_than_plain_on_seeded_dense():
    """P7 (output level; not a theorem): on the seeded dense workload, the
    Frobenius distance of Y to the unquantized-activation product does not
    grow with RAC at k in {25, 50, 100}."""
    wl = S.dense_small()
    qw = O.quantize_nvfp4(wl.w.f32)
    we = O.dequant_exact(qw.codes, qw.scales, qw.g)
    yt = wl.x.f32.astype(np.float64) @ we.T
    e_plain = np.linalg.norm(O.rac_linear(wl.x.f32, we[None], 0)["y"] - yt)
    prev = e_plain
    for k in (25, 50, 100):
        e = np.linalg.norm(O.rac_linear(wl.x.f32, we[None], k)["y"] - yt)
        assert e <= e_plain
        assert e <= prev * 1.0001
        prev = e


def test_grouped_rows_and_experts():
    """Grouped GEMM reference: row i uses activation row row_token[i] and the
    weights of the expert whose offset range holds i."""
    rng = np.random.default_rng(53)
    x = rng.standard_normal((5, 32)).astype(np.float32)
    w = (rng.standard_normal((3, 8, 32)) * 0.02).astype(np.float32)
    _, _, _, we = O.quantize_weights(w)
    rt = np.array([4, 0, 0, 2, 3, 1, 4], np.int32)
    offs = np.array([0, 3, 3, 7], np.int32)  # expert 1 empty
    out = O.rac_linear(x, we, 50, rt, offs)
    full = O.rac_linear(x, we[0:1], 50)  # same activation quantization
    assert np.array_equal(out["y"][0:3], full["y"][rt[0:3]])
    full2 = O.rac_linear(x, we[2:3], 50)
    assert np.array_equal(out["y"][3:7], full2["y"][rt[3:7]])
