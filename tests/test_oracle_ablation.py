"""Pins for the oracle's ablation variants (CPU only).

The technical summary's ablations (section 4) compare the asymmetric W4A16
trainer with symmetric W4A4 QAT, which fake-quantizes the trainer's
activations as well (section 2.1). The survey's ablation list adds one RAC
channel mask per expert as an alternative to one mask per input tensor.
Pins:
- a single expert reduces the per-expert function to the global one;
- k=0 reduces it to plain W4A4;
- the column max decomposes over row groups;
- each expert's mask is the brute-force top-k of its own rows' residual;
- the activation error still never grows;
- activations on the NVFP4 grid pass the symmetric fake-quant unchanged.
"""
import numpy as np

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import synthetic as S


def _grouped(seed, counts, K=64, N=24, outliers=2):
    rng = np.random.default_rng(seed)
    rows = int(sum(counts))
    x = S.activation(rng, rows, K, outliers, 30.0, bf16=True).f32
    w = S.weights(rng, (len(counts), N, K), bf16=True).f32
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    _, _, _, we = O.quantize_weights(w)
    return x, we, offs


def test_single_expert_equals_global_mask():
    x, we, offs = _grouped(201, [45])
    for k in (25, 50, 100):
        pe = O.rac_linear_per_expert(x, we, k, offs)
        gl = O.rac_linear(x, we, k, None, offs)
        e0 = pe["experts"][0]
        assert np.array_equal(e0["sel"], gl["sel"]) and e0["nsel"] == gl["nsel"]
        assert np.array_equal(e0["r"].codes, gl["r"].codes)
        assert np.array_equal(e0["r"].scales, gl["r"].scales) and e0["r"].g == gl["r"].g
        assert np.array_equal(pe["y"], gl["y"])


def test_k0_is_plain_w4a4():
    x, we, offs = _grouped(202, [7, 0, 30, 1])
    pe = O.rac_linear_per_expert(x, we, 0, offs)
    plain = O.rac_linear(x, we, 0, None, offs)
    assert np.array_equal(pe["y"], plain["y"])
    assert pe["experts"][1] is None


def test_scores_decompose_over_experts_and_codes_match_global():
    """The column max over all rows is the max of the per-expert column
    maxima, and quantizing an expert's rows with the tensor's scale gives the
    same codes as the tensor-wide quantization."""
    x, we, offs = _grouped(203, [12, 5, 20, 9], K=96)
    pe = O.rac_linear_per_expert(x, we, 50, offs)
    gl = O.rac_linear(x, we, 50, None, offs)
    per = np.stack([e["scores"] for e in pe["experts"]])
    assert np.array_equal(per.max(axis=0), gl["scores"])
    for e, ex in enumerate(pe["experts"]):
        a, b = offs[e], offs[e + 1]
        assert np.array_equal(ex["q"].codes, gl["q"].codes[a:b])
        assert np.array_equal(ex["q"].scales, gl["q"].scales[a:b])


def test_expert_mask_is_brute_force_top_k_of_its_rows():
    """Each expert's mask is the top nsel channels of max |x - dq| over that
    expert's rows, ranked by (score desc, index asc). Here dq comes from the
    tensor-wide quantization and the ranking is an explicit sort."""
    x, we, offs = _grouped(204, [6, 11, 3], K=32)
    gl = O.quantize_nvfp4(x)
    for k in (10, 50, 90):
        pe = O.rac_linear_per_expert(x, we, k, offs)
        for e, ex in enumerate(pe["experts"]):
            a, b = offs[e], offs[e + 1]
            score = np.abs(x[a:b].astype(np.float64) - gl.dq[a:b]).max(axis=0)
            nsel = (32 * k) // 100
            ranked = sorted(range(32), key=lambda c: (-score[c], c))[:nsel]
            assert ex["nsel"] == nsel
            assert list(ex["sel"][:nsel]) == sorted(ranked)


def test_per_expert_activation_error_never_grows():
    """P7 at the activation level holds mask by mask: with each expert's own
    mask the compensated activation is never farther from x than the plain
    dequantized one (up to one fp32 rounding)."""
    x, we, offs = _grouped(205, [20, 31, 13], K=128)
    pe = O.rac_linear_per_expert(x, we, 50, offs)
    for e, ex in enumerate(pe["experts"]):
        a, b = offs[e], offs[e + 1]
        xe = x[a:b]
        comp = O.rac_compensated_activation(xe, ex["q"], ex["r"], ex["sel"], ex["nsel"])
        e0 = np.abs(xe.astype(np.float64) - ex["q"].dq)
        e1 = np.abs(xe.astype(np.float64) - comp)
        ulp = np.spacing(np.abs(comp).astype(np.float32)).astype(np.float64)
        assert (e1 <= e0 + ulp).all()


def test_fake_quant_activation_identity_on_grid():
    """Activations that lie on the NVFP4 grid are returned unchanged by the
    symmetric scheme's fake quantization. One block per row reaches the
    tensor's amax, so the tensor scale is reproduced exactly."""
    rng = np.random.default_rng(206)
    lv = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    g = 2.0 ** -8
    sc = O.E4M3_VALUES[rng.integers(48, 120, (8, 4))]
    sc[0, 0] = 448.0
    m = lv[rng.integers(0, 8, (8, 64))] * np.where(rng.random((8, 64)) < 0.5, -1, 1)
    m[:, ::16] = 6.0
    x = (m * np.repeat(sc, 16, axis=1) * g).astype(np.float32)
    bits = O.fake_quant_activation(x)
    assert np.array_equal(O.f32_from_bf16_bits(bits), x)
