"""GPU parity of the ablation variants, through the C ABI. The variants are
the asymmetric W4A16 trainer, the symmetric W4A4 QAT trainer, the rollout's
plain W4A4, and RAC with one mask per tensor or one mask per expert. The
grouped layers include an empty expert and ragged experts. The oracle
decides:
- bit-exact QDQ bits, per-expert masks and residuals;
- GEMM outputs within 1e-3 of its float64 products;
- the P7 output-level ordering on the seeded layers."""
import numpy as np
import pytest
import torch

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import _lib as Q
from fp4_quantized_moe_amd import ablation as A
from fp4_quantized_moe_amd import synthetic as S
from tests.gpu_util import dev_act, host, log, rel_err

pytestmark = pytest.mark.gpu


def _setup(seed, counts, K=256, N=128):
    rng = np.random.default_rng(seed)
    R = int(sum(counts))
    xa = S.activation(rng, R, K, 3, 30.0, bf16=True)
    wa = S.weights(rng, (len(counts), N, K))
    offs = [0] + [int(v) for v in np.cumsum(counts)]
    return xa, wa, offs


def _grouped(xm, wm, offs):
    y = np.zeros((xm.shape[0], wm.shape[1]), np.float64)
    for e in range(wm.shape[0]):
        a, b = offs[e], offs[e + 1]
        y[a:b] = xm[a:b] @ wm[e].T
    return y


def _bits(t):
    return host(t.contiguous().view(torch.int16)).view(np.uint16)


def test_ablation_variants_match_oracle():
    counts = (37, 0, 64, 21)
    log(f"[ablation] variants, experts {counts}, K=256, N=128")
    xa, wa, offs = _setup(301, counts)
    x, w = dev_act(xa), dev_act(wa)
    out = A.grouped_linear_variants(x, w, offs, k_list=(0, 25, 50, 100), per_expert_k=(50, 100))
    E = len(counts)
    wq_bits = np.stack([O.weight_qdq(wa.f32[e])[0] for e in range(E)])
    xq_bits = O.fake_quant_activation(xa.f32)
    assert np.array_equal(_bits(Q.weight_qdq(w)[0]), wq_bits)
    assert np.array_equal(_bits(Q.weight_qdq(x)[0]), xq_bits)
    x64 = xa.f32.astype(np.float64)
    wq64 = O.f32_from_bf16_bits(wq_bits).astype(np.float64)
    ref = {"bf16": _grouped(x64, wa.f32.astype(np.float64), offs),
           "w4a16": _grouped(x64, wq64, offs),
           "w4a4_sym": _grouped(O.f32_from_bf16_bits(xq_bits).astype(np.float64), wq64, offs)}
    _, _, _, we = O.quantize_weights(wa.f32)
    for k in (0, 25, 50, 100):
        ref[f"rac{k}"] = O.rac_linear(xa.f32, we, k, None, np.array(offs))["y"]
    ref["w4a4"] = ref["rac0"]
    for k in (50, 100):
        ref[f"rac{k}_pe"] = O.rac_linear_per_expert(xa.f32, we, k, np.array(offs))["y"]
    for name, r in ref.items():
        err = rel_err(host(out[name]), r)
        log(f"  {name}: rel err {err:.2e}")
        assert err <= 1e-3, name


@pytest.mark.parametrize("k", [25, 50, 100])
def test_per_expert_masks_bit_exact(k):
    counts = (50, 16, 0, 9, 33)
    log(f"[ablation] per-expert masks k={k}, experts {counts}")
    xa, wa, offs = _setup(302, counts, K=512, N=256)
    x, w = dev_act(xa), dev_act(wa)
    _, wq = Q.weight_qdq(w, export=True)
    q, _ = Q.quantize_nvfp4(x)
    _, _, _, we = O.quantize_weights(wa.f32)
    y, parts = A.per_expert_rac(x, q, wq, offs, k)
    ref = O.rac_linear_per_expert(xa.f32, we, k, np.array(offs))
    for e, (p, r) in enumerate(zip(parts, ref["experts"])):
        if r is None:
            assert p is None
            continue
        sel, res, nsel = p
        assert nsel == r["nsel"], e
        assert np.array_equal(host(sel), r["sel"]), e
        assert np.array_equal(host(res.codes), r["r"].codes), e
        assert np.array_equal(host(res.scales), r["r"].scales), e
        assert host(res.gscale)[0] == np.float32(r["r"].g), e
    assert rel_err(host(y), ref["y"]) <= 1e-3


def test_error_ordering_on_seeded_layer():
    """P7 at the output level, on the GPU's results for a seeded layer: the
    reference is the float64 product of the unquantized activation and the
    exactly dequantized weights. RAC at every k, with either mask, is no
    farther from it than plain W4A4. Against the masters' product, the
    symmetric trainer is farther than the asymmetric one."""
    counts = (40, 70, 0, 25)
    log(f"[ablation] error ordering, experts {counts}, K=512, N=256")
    xa, wa, offs = _setup(303, counts, K=512, N=256)
    x, w = dev_act(xa), dev_act(wa)
    out = A.grouped_linear_variants(x, w, offs, k_list=(25, 50, 100), per_expert_k=(25, 50, 100))
    _, _, _, we = O.quantize_weights(wa.f32)
    yt = _grouped(xa.f32.astype(np.float64), we, offs)
    fro = {n: float(np.linalg.norm(host(y).astype(np.float64) - yt)) for n, y in out.items()}
    log("  " + ", ".join(f"{n} {v:.4g}" for n, v in fro.items()))
    for k in (25, 50, 100):
        assert fro[f"rac{k}"] <= fro["w4a4"], k
        assert fro[f"rac{k}_pe"] <= fro["w4a4"], k
    err = A.errors(out, A.reference_fp64(x, w, offs))
    assert err["w4a16"]["rel_fro"] < err["w4a4_sym"]["rel_fro"]
    assert err["bf16"]["rel_max"] < 1e-5
