"""GPU parity: NVFP4 quantization, RAC scores / mask / residual and weight QDQ
through the C ABI vs the oracle -- bit-exact on codes, scale bytes, tensor
scales, scores and selected indices."""
import numpy as np
import pytest
import torch

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import _lib as Q
from fp4_quantized_moe_amd import synthetic as S
from tests.gpu_util import dev_act, host, log, nvfp4_host

pytestmark = pytest.mark.gpu


def _check_quant(x_act, tag):
    log(f"[quant] {tag} shape={x_act.f32.shape} bf16={x_act.is_bf16}")
    x = dev_act(x_act)
    q, scores = Q.quantize_nvfp4(x, want_scores=True)
    ref = O.quantize_nvfp4(x_act.f32)
    codes, scales, g = nvfp4_host(q)
    assert g[0] == ref.g, (g[0], ref.g)
    assert np.array_equal(scales, ref.scales), np.argwhere(scales != ref.scales)[:5]
    bad = np.argwhere(codes != ref.codes)
    assert bad.size == 0, bad[:5]
    sref = O.rac_scores(x_act.f32, ref)
    assert np.array_equal(host(scores).view(np.uint32), sref.view(np.uint32))
    return x, q, scores, ref, sref


def test_quantize_dense_small_fp32():
    _check_quant(S.dense_small().x, "dense_small")


def test_quantize_expert_gemm_bf16():
    _check_quant(S.expert_gemm().x, "expert_gemm")


def test_quantize_ragged_and_special():
    rng = np.random.default_rng(7)
    for rows, cols in [(1, 16), (3, 48), (17, 80), (129, 784), (257, 1040)]:
        a = S.activation(rng, rows, cols, min(2, cols // 16), 50.0, bf16=bool(rows % 2))
        a.f32[0, :16] = 0.0  # an all-zero block
        if a.bits is not None:
            a.bits[0, :16] = 0
        _check_quant(a, f"ragged {rows}x{cols}")


def test_quantize_all_zero_and_signed_zero():
    x = torch.zeros(4, 32, dtype=torch.float32, device="cuda")
    x[1, 3] = -0.0
    q, _ = Q.quantize_nvfp4(x)
    codes, scales, g = nvfp4_host(q)
    assert g[0] == 1.0 and (scales == 0).all()
    ref = O.quantize_nvfp4(host(x))
    assert np.array_equal(codes, ref.codes)


def test_quantize_gscale_given_and_batched():
    rng = np.random.default_rng(8)
    w = S.weights(rng, (6, 64, 128), 0.02, bf16=True)
    wd = dev_act(w)
    q, _ = Q.quantize_nvfp4(wd)
    codes, scales, g = nvfp4_host(q)
    for b in range(6):
        r = O.quantize_nvfp4(w.f32[b])
        assert g[b] == r.g and np.array_equal(codes[b], r.codes) and np.array_equal(scales[b], r.scales)
    # given tensor scale: doubled g
    g2 = torch.from_numpy(g * 2).cuda()
    q2, _ = Q.quantize_nvfp4(wd, gscale=g2)
    c2, s2, gg = nvfp4_host(q2)
    for b in range(6):
        r = O.quantize_nvfp4(w.f32[b], g=np.float32(g[b] * 2))
        assert gg[b] == np.float32(g[b] * 2) and np.array_equal(c2[b], r.codes) and np.array_equal(s2[b], r.scales)


@pytest.mark.parametrize("k", [0, 25, 50, 100])
def test_rac_select_and_residual_expert_gemm(k):
    wl = S.expert_gemm()
    x, q, scores, ref, sref = _check_quant(wl.x, f"expert_gemm k={k}")
    log(f"[rac] expert_gemm k={k}")
    sel, res, nsel = Q.rac_select(x, q, scores, k)
    rsel, rn = O.rac_select(sref, k)
    assert nsel == rn
    assert np.array_equal(host(sel), rsel)
    rres = O.rac_quantize_residual(wl.x.f32, ref, rsel, rn)
    rc, rs, rg = nvfp4_host(res)
    assert rg[0] == rres.g
    if rsel.size:
        assert np.array_equal(rs, rres.scales)
        assert np.array_equal(rc, rres.codes)


def test_rac_select_ties_and_ragged():
    """Scores with many exact ties (constructed input) and nsel not a multiple of 16."""
    rng = np.random.default_rng(9)
    xv = np.round(rng.standard_normal((40, 256)) * 4).astype(np.float32) / 4
    a = S.Activation(xv, None)
    x, q, scores, ref, sref = _check_quant(a, "ties")
    for k in (1, 10, 33, 77):
        sel, res, nsel = Q.rac_select(x, q, scores, k)
        rsel, rn = O.rac_select(sref, k)
        assert np.array_equal(host(sel), rsel), k
        rres = O.rac_quantize_residual(xv, ref, rsel, rn)
        rc, rs, rg = nvfp4_host(res)
        assert rg[0] == rres.g and np.array_equal(rc, rres.codes) and np.array_equal(rs, rres.scales)


@pytest.mark.parametrize("cols", [256, 1024, 2048])
def test_rac_select_ties_bf16_one_launch(cols):
    """bf16 rows with many exactly tied scores, few rows (each workgroup of the
    row kernel finds the mask itself: one launch), nsel not a multiple of
    16, both RAC entry points: mask, residual and g_r bit-exact."""
    rng = np.random.default_rng(19 + cols)
    xv = np.round(rng.standard_normal((37, cols)) * 4).astype(np.float32) / 4
    a = S.Activation(xv, O.bf16_bits_from_f32(xv))
    x, q, scores, ref, sref = _check_quant(a, f"ties bf16 {cols}")
    for k in (1, 10, 33, 77, 100):
        for merged in (False, True):
            sel, res, nsel = Q.SelectCall(x, q, scores, k, merged=merged)()
            rsel, rn = O.rac_select(sref, k)
            assert nsel == rn and np.array_equal(host(sel), rsel), (k, merged)
            rres = O.rac_quantize_residual(xv, ref, rsel, rn)
            rc, rs, rg = nvfp4_host(res)
            assert rg[0] == rres.g and np.array_equal(rc, rres.codes) and np.array_equal(rs, rres.scales), (k, merged)


def test_weight_qdq_bit_exact():
    rng = np.random.default_rng(10)
    w = S.weights(rng, (5, 96, 256), 0.02, bf16=True)
    wd = dev_act(w)
    out, q = Q.weight_qdq(wd, export=True)
    o = host(out.view(torch.int16)).view(np.uint16)
    codes, scales, g = nvfp4_host(q)
    for b in range(5):
        bits, r = O.weight_qdq(w.f32[b])
        assert np.array_equal(o[b], bits)
        assert g[b] == r.g and np.array_equal(codes[b], r.codes) and np.array_equal(scales[b], r.scales)
    # shared path: the QDQ export equals the quantizer on the same weights
    q2, _ = Q.quantize_nvfp4(wd)
    assert torch.equal(q2.codes, q.codes) and torch.equal(q2.scales, q.scales) and torch.equal(q2.gscale, q.gscale)


def test_determinism():
    wl = S.expert_gemm(M=512)
    x = dev_act(wl.x)
    outs = []
    for _ in range(2):
        q, s = Q.quantize_nvfp4(x, want_scores=True)
        sel, res, _ = Q.rac_select(x, q, s, 50)
        outs.append([host(t).tobytes() for t in (q.codes, q.scales, s, sel, res.codes, res.scales, res.gscale)])
    assert outs[0] == outs[1]


def test_quantize_near_ties_random_scales():
    """Elements placed at every E2M1 rounding tie t*d and +-1..3 ulp around it,
    for many random tensor scales and block scales: the device quotient and
    rounding must match the oracle's IEEE division bit for bit."""
    rng = np.random.default_rng(11)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float64)
    blocks = []
    for _ in range(4096):
        g = np.float32(np.exp2(rng.uniform(-20, 10)))
        s = int(rng.integers(1, 127))
        ds = O.E4M3_VALUES[s]
        amax = np.float32(6.0 * ds * np.float64(g))
        d = np.float32(np.float32(ds) * g)
        t = ties[rng.integers(0, len(ties), 15)]
        base = (t * np.float64(d)).astype(np.float32)
        off = rng.integers(-3, 4, 15)
        vals = (base.view(np.int32) + off.astype(np.int32)).view(np.float32) * np.where(rng.random(15) < 0.5, -1, 1).astype(np.float32)
        blk = np.concatenate([[amax], vals]).astype(np.float32)
        blocks.append((g, blk))
    # one row per tensor scale: [rows=4096, cols=16] with per-row g is not expressible,
    # so quantize each block as its own 1-row tensor through the batched entry point
    gs = np.array([b[0] for b in blocks], np.float32)
    x = np.stack([b[1] for b in blocks])[:, None, :]  # [batch, 1, 16]
    xd = torch.from_numpy(x).cuda()
    q, _ = Q.quantize_nvfp4(xd, gscale=torch.from_numpy(gs).cuda())
    codes, scales, _ = nvfp4_host(q)
    for i in range(len(blocks)):
        r = O.quantize_nvfp4(x[i], g=gs[i])
        assert codes[i].tobytes() == r.codes.tobytes() and scales[i].tobytes() == r.scales.tobytes(), i


@pytest.mark.parametrize("cols,k", [(2048, 50), (768, 25), (64, 100)])
def test_empty_activation(cols, k):
    """No rows: the tensor scale is 1 and every channel score 0 (the oracle's
    reading: the largest of no magnitudes is 0), then the mask is the first
    nsel channels and the residual's tensor scale is 1, with the plain and the
    merged select.  Outputs start out poisoned, so each is seen written."""
    log(f"[quant] empty activation cols={cols} k={k}")
    x = torch.empty(0, cols, dtype=torch.bfloat16, device="cuda")
    qc = Q.QuantizeCall(x, want_scores=True)
    qc.q.gscale.fill_(7.0)
    qc.scores.fill_(float("nan"))
    q, scores = qc()
    empty = np.zeros((0, cols), np.float32)
    ref = O.quantize_nvfp4(empty)
    sref = O.rac_scores(empty, ref)
    assert host(q.gscale)[0] == ref.g == np.float32(1.0)
    assert np.array_equal(host(scores).view(np.uint32), sref.view(np.uint32))
    osel, on = O.rac_select(sref, k)
    for merged in (False, True):
        call = Q.SelectCall(x, q, scores, k, merged=merged)
        call.sel.fill_(-1)
        call.res.gscale.fill_(7.0)
        sel, res, nsel = call()
        assert nsel == on and np.array_equal(host(sel), osel)
        assert host(res.gscale)[0] == O.rac_quantize_residual(empty, ref, osel, on).g == np.float32(1.0)
