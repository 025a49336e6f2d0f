"""GPU parity of the trainer forward with the weight QDQ fused into the GEMM
(QUADS_OPERANDS_BF16_QDQ: bf16 masters fake-quantized in registers on their
way to the matrix cores; gist.science "Technische Samenvatting: QUADS"
section 2.2-A: every forward pass sees the discretized weights, the
optimizer updates the BF16 masters).

* QUADS_SCALES_ONLY gives the tensor scales quads_weight_qdq exports, and the
  oracle's, bit for bit;
* both fused forms -- the masters fake-quantized in registers
  (QUADS_OPERANDS_BF16_QDQ) and their NVFP4 encoding decoded to QDQ values
  (QUADS_OPERANDS_BF16_W4) -- equal quads_weight_qdq followed by the
  bf16-operand GEMM bit for bit (same tile schedule, identical weight
  values), on grouped and SwiGLU shapes, a K tail, zero blocks and matrices
  small enough that the block scales fall below FP32's normal range, and on
  a full trainer layer;
* against the oracle (its own weight QDQ, float64 product) within 1e-3;
* the quantizer's codes stay bit-exact for extreme blocks (given tensor
  scales far too small for the data, tiny matrices)."""
import numpy as np
import pytest
import torch

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import _lib as Q
from fp4_quantized_moe_amd import synthetic as S
from tests.gpu_util import dev_act, host, log, rel_err

pytestmark = pytest.mark.gpu


def _bits(t):
    return host(t.contiguous().view(torch.int16)).view(np.uint16)


def _masters(rng, E, N, K, n_seg, tiny_matrix=None, zero_rows=True):
    """bf16 masters [E, N, K] ~N(0, 0.02); optionally one whole (expert,
    segment) matrix scaled down to ~1e-33 (block scales below FP32's normal
    range after the tensor scale) and a few all-zero 16-blocks."""
    w = (rng.standard_normal((E, N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    if tiny_matrix is not None:
        # ~1e-33 values (tensor scale ~2^-119); two rows 1e-5 smaller still,
        # whose block scales are E4M3 subnormals (d below 2^-125), and one
        # row 1e-7 smaller, whose block scales flush to zero
        e, sg = tiny_matrix
        seg = N // n_seg
        m = w[e, sg * seg:(sg + 1) * seg]
        m *= np.float32(5e-32)
        m[1:3] *= np.float32(1e-5)
        m[4] *= np.float32(1e-7)
    if zero_rows:
        w[0, 3, 16:48] = 0.0
        w[-1, -1, :16] = 0.0
    bits, vals = S.to_bf16(w)
    return S.Activation(vals, bits)


def _fused_and_unfused(xa, wa, offs, rt, n_seg, epilogue):
    E, N, K = wa.f32.shape
    x = dev_act(xa)
    w = dev_act(wa)
    g = Q.weight_scales(w.view(E * n_seg, N // n_seg, K))
    wq, q = Q.weight_qdq(w.view(E * n_seg, N // n_seg, K), export=True)
    assert np.array_equal(host(g).view(np.uint32), host(q.gscale).view(np.uint32)), "scales-only != exported g"
    R = int(offs[-1])
    kw = dict(N=N, K=K, expert_offsets=torch.from_numpy(offs).cuda(), num_rows=R, x_bf16=x,
              row_token=None if rt is None else torch.from_numpy(rt).cuda(), epilogue=epilogue, n_seg=n_seg)
    y_unf = Q.moe_w4a4_gemm(w_bf16=wq.view(E, N, K), **kw)
    y_fus = Q.moe_w4a4_gemm(w_bf16=w, w_gscale=g, qdq=True, **kw)
    # the masters' NVFP4 encoding decoded to QDQ values inside the GEMM
    wn, _ = Q.quantize_nvfp4(w.view(E * n_seg, N // n_seg, K))
    y_w4 = Q.moe_w4a4_gemm(w_codes=wn.codes.view(E, N, K // 2), w_scales=wn.scales.view(E, N, K // 16),
                           w_gscale=wn.gscale, **kw)
    same = y_w4.view(torch.int16) if y_w4.dtype == torch.bfloat16 else y_w4.view(torch.int32)
    ref = y_unf.view(torch.int16) if y_unf.dtype == torch.bfloat16 else y_unf.view(torch.int32)
    assert torch.equal(same, ref), "NVFP4-decoded forward != QDQ + bf16 GEMM"
    return y_fus, y_unf, host(g)


def _oracle_y(xa, wa, offs, rt, n_seg, g_dev):
    E, N, K = wa.f32.shape
    seg = N // n_seg
    xs = xa.f32.astype(np.float64)
    rows_all = np.arange(int(offs[-1])) if rt is None else rt
    y = np.zeros((int(offs[-1]), N))
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        parts = []
        for sgi in range(n_seg):
            bits, q = O.weight_qdq(wa.f32[e, sgi * seg:(sgi + 1) * seg])
            assert np.float32(q.g) == np.float32(g_dev[e * n_seg + sgi])
            parts.append(O.f32_from_bf16_bits(bits).astype(np.float64))
        if a < b:
            y[a:b] = xs[rows_all[a:b]] @ np.concatenate(parts).T
    return y


def test_fused_qdq_grouped_bit_identical_and_oracle():
    rng = np.random.default_rng(801)
    counts = [130, 0, 257, 64, 1, 300]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    for K in (512, 528):  # 528: a K tail of one 16-block past the last 64-element step
        xa = S.activation(rng, 400, K, 4, 30.0, bf16=True)
        wa = _masters(rng, len(counts), 256, K, 1, tiny_matrix=(3, 0))
        rt = rng.integers(0, 400, int(offs[-1])).astype(np.int32)
        log(f"[qdq-fused] grouped experts {counts} N=256 K={K} (one tiny matrix, zero blocks)")
        y_fus, y_unf, g = _fused_and_unfused(xa, wa, offs, rt, 1, Q.EPI_NONE)
        assert np.array_equal(host(y_fus).view(np.uint32), host(y_unf).view(np.uint32))
        ref = _oracle_y(xa, wa, offs, rt, 1, g)
        err = rel_err(host(y_fus), ref)
        log(f"  rel err {err:.2e}")
        assert err <= 1e-3


def test_fused_qdq_swiglu_large_tiles_bit_identical():
    """Many rows per expert (the ping-pong 256 x 256 kernel), gate and up
    with their own scales, SwiGLU epilogue."""
    rng = np.random.default_rng(802)
    counts = [700, 0, 1100, 513]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    xa = S.activation(rng, 1500, 1024, 10, 30.0, bf16=True)
    wa = _masters(rng, len(counts), 512, 1024, 2, tiny_matrix=(2, 1))
    rt = rng.integers(0, 1500, int(offs[-1])).astype(np.int32)
    log(f"[qdq-fused] SwiGLU experts {counts} N=2x256 K=1024")
    h_fus, h_unf, g = _fused_and_unfused(xa, wa, offs, rt, 2, Q.EPI_SWIGLU)
    assert np.array_equal(_bits(h_fus), _bits(h_unf))
    y = _oracle_y(xa, wa, offs, rt, 2, g)
    h_ref = O.swiglu(y[:, :256], y[:, 256:])
    hf = host(h_fus.float())
    tol = 2.0 ** -8 * np.abs(h_ref) + 2e-3 * np.abs(y).max() * (np.abs(y[:, 256:]) + np.abs(y[:, :256]) + 1)
    assert (np.abs(hf - h_ref) <= tol).all()


def test_fused_qdq_full_trainer_layer_bit_identical():
    """One full trainer layer (8192 tokens, 128 experts, top-8; gate_up
    2048 -> 2 x 1024 with SwiGLU, down 1024 -> 2048) in the launch
    configuration the benchmark times: the fused forward equals QDQ + bf16
    GEMM bit for bit, and the scales-only pass equals the exported scales."""
    T, H, E, I, top = 8192, 2048, 128, 1024, 8
    rng = np.random.default_rng(5)
    x = dev_act(S.activation(rng, T, H, 0, 1.0, bf16=True))
    logits = S.gaussian_logits(rng, T, E)
    gu_m, dn_m = S.trainer_layer_weights_device(5, 0, E, H, I)
    _, _, offs, rt, _ = Q.moe_route(torch.from_numpy(logits).cuda(), top)
    R = T * top
    log("[qdq-fused] full trainer layer: scales, QDQ, unfused and fused forward")
    g_gu, g_dn = Q.weight_scales(gu_m), Q.weight_scales(dn_m)
    wq_gu, qgu = Q.weight_qdq(gu_m, export=True)
    wq_dn, qdn = Q.weight_qdq(dn_m, export=True)
    assert np.array_equal(host(g_gu).view(np.uint32), host(qgu.gscale).view(np.uint32))
    assert np.array_equal(host(g_dn).view(np.uint32), host(qdn.gscale).view(np.uint32))
    h_unf = Q.moe_w4a4_gemm(N=2 * I, K=H, expert_offsets=offs, num_rows=R, row_token=rt, x_bf16=x,
                            w_bf16=wq_gu.view(E, 2 * I, H), epilogue=Q.EPI_SWIGLU)
    h_fus = Q.moe_w4a4_gemm(N=2 * I, K=H, expert_offsets=offs, num_rows=R, row_token=rt, x_bf16=x,
                            w_bf16=gu_m.view(E, 2 * I, H), w_gscale=g_gu, qdq=True, n_seg=2,
                            epilogue=Q.EPI_SWIGLU)
    assert np.array_equal(_bits(h_fus), _bits(h_unf))
    y_unf = Q.moe_w4a4_gemm(N=H, K=I, expert_offsets=offs, num_rows=R, x_bf16=h_unf, w_bf16=wq_dn)
    y_fus = Q.moe_w4a4_gemm(N=H, K=I, expert_offsets=offs, num_rows=R, x_bf16=h_fus, w_bf16=dn_m, w_gscale=g_dn,
                            qdq=True)
    assert np.array_equal(host(y_fus).view(np.uint32), host(y_unf).view(np.uint32))
    log("[qdq-fused] full trainer layer: NVFP4-decoded forward")
    qg, _ = Q.quantize_nvfp4(gu_m)
    qd, _ = Q.quantize_nvfp4(dn_m)
    h_w4 = Q.moe_w4a4_gemm(N=2 * I, K=H, expert_offsets=offs, num_rows=R, row_token=rt, x_bf16=x,
                           w_codes=qg.codes.view(E, 2 * I, H // 2), w_scales=qg.scales.view(E, 2 * I, H // 16),
                           w_gscale=qg.gscale, n_seg=2, epilogue=Q.EPI_SWIGLU)
    assert np.array_equal(_bits(h_w4), _bits(h_unf))
    y_w4 = Q.moe_w4a4_gemm(N=H, K=I, expert_offsets=offs, num_rows=R, x_bf16=h_unf, w_codes=qd.codes,
                           w_scales=qd.scales, w_gscale=qd.gscale)
    assert np.array_equal(host(y_w4).view(np.uint32), host(y_unf).view(np.uint32))


def test_quantizer_extreme_blocks_bit_exact():
    """Codes and scales against the oracle where the division takes its
    rescaled or capped form: a tensor scale given far too small for the data
    (block scales saturate at 448 and quotients exceed 8 or FP32's range), a
    matrix of ~1e-33 values (block scales below FP32's normal range), and a
    given scale so large that block scales flush to zero."""
    rng = np.random.default_rng(803)
    x = rng.standard_normal((64, 256), dtype=np.float32)
    x[5] *= np.float32(1e10)
    tiny = (rng.standard_normal((64, 256), dtype=np.float32) * np.float32(1e-33)).astype(np.float32)
    tiny[3:9] *= np.float32(1e-5)  # FP32 subnormal inputs; block scales with d below 2^-125
    tiny[10] *= np.float32(1e-7)   # block scales that flush to zero
    sub = (rng.standard_normal((64, 256), dtype=np.float32) * np.float32(1e-40)).astype(np.float32)
    # every intermediate stays finite (the oracle's domain): the given scales
    # only push block scales to saturation (quotients far above 8), below
    # FP32's normal range, or to zero
    cases = [("given g too small", x, np.float32(1e-20)), ("tiny matrix", tiny, None),
             ("FP32-subnormal data, given subnormal g", sub, np.float32(2.0 ** -140)),
             ("given g huge", x, np.float32(1e35))]
    for tag, xv, g in cases:
        log(f"[quant] extreme blocks: {tag}")
        xd = torch.from_numpy(np.ascontiguousarray(xv)).cuda()
        q, _ = Q.quantize_nvfp4(xd, gscale=None if g is None else torch.tensor([g], device="cuda"))
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            oq = O.quantize_nvfp4(xv, g)
        assert np.array_equal(host(q.codes), oq.codes), tag
        assert np.array_equal(host(q.scales), oq.scales), tag
