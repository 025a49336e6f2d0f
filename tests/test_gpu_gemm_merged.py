"""GPU parity of both formulations of the RAC correction in the grouped GEMM,
chosen per call with the rac_form argument:
- exact (QUADS_RAC_FORM_EXACT): the correction as an extended contraction,
  exact up to FP32 accumulation;
- merged (QUADS_RAC_FORM_MERGED): the correction added to the activation as
  one fp16 operand, with one more rounding per corrected element.
Both are checked against the oracle's float64 extended-K reference at the
1e-3 bar (the exact form also at the accumulation-only bar EXACT_TOL):
dense and grouped shapes, ragged rows, a gathered row order, the SwiGLU
epilogue, the few-rows (decode) shape in both forms, K tails (K % 64 != 0,
an odd number of 64-wide steps) on both tile shapes, and the full-size
expert-GEMM workload through the caller-built merged operand."""
import numpy as np
import pytest
import torch

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import _lib as Q
from fp4_quantized_moe_amd import synthetic as S
from tests.gpu_util import dev_act, host, log, quantize_weights_gpu, rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-3
# The exact form differs from the float64 reference by FP32 accumulation only.
EXACT_TOL = 2e-5
FORMS = {"exact": Q.RAC_FORM_EXACT, "merged": Q.RAC_FORM_MERGED}


def _grouped(seed, counts, T, K, N, n_seg=1):
    rng = np.random.default_rng(seed)
    xa = S.activation(rng, T, K, max(1, K // 100), 30.0, bf16=True)
    wa = S.weights(rng, (len(counts), N, K))
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rt = rng.integers(0, T, int(offs[-1])).astype(np.int32)
    return xa, wa, offs, rt


def _run(xa, wa, offs, rt, k, n_seg=1, epilogue=Q.EPI_NONE, rac_form=Q.RAC_FORM_AUTO):
    x = dev_act(xa)
    E, N, K = wa.f32.shape
    wc, ws_, wg = quantize_weights_gpu(dev_act(wa), n_seg)
    q, scores = Q.quantize_nvfp4(x, want_scores=True)
    sel, res, nsel = Q.rac_select(x, q, scores, k)
    R = int(offs[-1])
    return Q.moe_w4a4_gemm(w_codes=wc, w_scales=ws_, w_gscale=wg, n_seg=n_seg, N=N, K=K,
                           expert_offsets=torch.from_numpy(offs).cuda(), num_rows=R, x=q,
                           res=res if nsel else None, sel_idx=sel,
                           row_token=None if rt is None else torch.from_numpy(rt).cuda(), epilogue=epilogue,
                           rac_form=rac_form)


def _check(y, ref, mode):
    err = rel_err(y, ref)
    log(f"  rel err {err:.2e}")
    assert err <= (EXACT_TOL if mode == "exact" else TOL)


@pytest.mark.parametrize("mode", ["exact", "merged"])
@pytest.mark.parametrize("k", [25, 50, 100])
def test_dense_both_formulations(mode, k):
    wl = S.expert_gemm(M=1024)
    log(f"[gemm-rac] dense 1024x2048x1536 k={k} {mode}")
    offs = np.array([0, 1024], np.int32)
    y = host(_run(wl.x, S.Activation(wl.w.f32[None], wl.w.bits[None]), offs, None, k, rac_form=FORMS[mode]))
    _, _, _, we = O.quantize_weights(wl.w.f32[None], 1)
    _check(y, O.rac_linear(wl.x.f32, we, k)["y"], mode)


@pytest.mark.parametrize("mode", ["exact", "merged"])
def test_grouped_gathered_both_formulations(mode):
    counts = [300, 0, 257, 511, 64, 1, 200, 129]
    xa, wa, offs, rt = _grouped(601, counts, 700, 768, 512)
    log(f"[gemm-rac] grouped experts {counts} K=768 N=512 k=50 {mode}")
    y = host(_run(xa, wa, offs, rt, 50, rac_form=FORMS[mode]))
    _, _, _, we = O.quantize_weights(wa.f32, 1)
    _check(y, O.rac_linear(xa.f32, we, 50, rt, offs)["y"], mode)


@pytest.mark.parametrize("counts,K,N", [
    ([300, 0, 257, 130], 784, 512),   # K % 64 != 0
    ([300, 0, 257, 130], 832, 512),   # odd step count
    ([4096, 4000], 832, 2048),        # 256x256 tiles, odd step count
])
def test_merged_k_tails(counts, K, N):
    """K tails of the merged operand's GEMM: K % 64 != 0 (a ragged last
    step whose blocks past K are zeroed) and an odd count of 64-wide steps
    (the pipeline pads one all-zero step), on both tile shapes."""
    xa, wa, offs, rt = _grouped(611, counts, 700, K, N)
    log(f"[gemm-rac] merged experts {counts} K={K} N={N} k=50")
    y = host(_run(xa, wa, offs, rt, 50, rac_form=Q.RAC_FORM_MERGED))
    _, _, _, we = O.quantize_weights(wa.f32, 1)
    _check(y, O.rac_linear(xa.f32, we, 50, rt, offs)["y"], "merged")


@pytest.mark.parametrize("mode", ["exact", "merged"])
def test_decode_shape_both_formulations(mode):
    """Few rows per expert (the decode shape, which defaults to the merged
    operand on the few-rows kernel): the exact form runs on the many-rows
    kernels and reaches the accumulation-only bar."""
    counts = [16, 0, 9, 16, 31, 1, 16, 12, 16, 16, 3, 16, 20, 16, 16, 8]
    xa, wa, offs, rt = _grouped(607, counts, 200, 512, 256)
    log(f"[gemm-rac] decode shape experts {counts} K=512 N=256 k=50 {mode}")
    y = host(_run(xa, wa, offs, rt, 50, rac_form=FORMS[mode]))
    _, _, _, we = O.quantize_weights(wa.f32, 1)
    _check(y, O.rac_linear(xa.f32, we, 50, rt, offs)["y"], mode)


def test_grouped_swiglu_merged():
    """gate/up stacked along N with two tensor scales, SwiGLU epilogue, merged
    operand: h against silu(gate) * up of the oracle's float64 product."""
    counts = [400, 333, 0, 291]
    xa, wa, offs, rt = _grouped(602, counts, 600, 512, 512)
    log(f"[gemm-rac] grouped SwiGLU experts {counts} K=512 N=512 merged")
    h = host(_run(xa, wa, offs, rt, 50, n_seg=2, epilogue=Q.EPI_SWIGLU, rac_form=Q.RAC_FORM_MERGED).float())
    _, _, _, we = O.quantize_weights(wa.f32, 2)
    y = O.rac_linear(xa.f32, we, 50, rt, offs)["y"]
    I = y.shape[1] // 2
    h_ref = O.swiglu(y[:, :I], y[:, I:])
    tol = 2.0 ** -8 * np.abs(h_ref) + 2e-3 * np.abs(y).max() * (np.abs(y[:, I:]) + np.abs(y[:, :I]) + 1)
    assert (np.abs(h - h_ref) <= tol).all()


@pytest.mark.parametrize("case", [("bf16", 300, 2048, 50), ("bf16", 300, 2048, 100), ("bf16", 77, 768, 25),
                                  ("f32", 64, 256, 50), ("bf16", 40, 512, 0),
                                  # more than 1024 four-row groups: workgroups walk several groups
                                  ("bf16", 6001, 768, 50), ("bf16", 5000, 2048, 25),
                                  # wide rows: four load slots, one row per group, LDS beyond 64 KiB
                                  ("bf16", 5, 16384, 100), ("f32", 7, 8208, 50), ("bf16", 33, 9984, 25)])
def test_rac_select_merged_bit_exact(case):
    """quads_rac_select_merged's fp16 operand equals the oracle's
    rac_merged_operand bit for bit (same fp32 operations, one rounding); the
    mask and residual match as for quads_rac_select."""
    dt, M, K, k = case
    log(f"[rac-merged] {dt} M={M} K={K} k={k}")
    rng = np.random.default_rng(603 + M + k)
    xa = S.activation(rng, M, K, max(1, K // 100), 30.0, bf16=(dt == "bf16"))
    x = dev_act(xa)
    q, scores = Q.quantize_nvfp4(x, want_scores=True)
    call = Q.SelectCall(x, q, scores, k, merged=True)
    sel, res, nsel = call()
    oq = O.quantize_nvfp4(xa.f32)
    osel, on = O.rac_select(O.rac_scores(xa.f32, oq), k)
    assert nsel == on and np.array_equal(host(sel), osel)
    if on == 0:
        return  # nothing selected: the merged operand is not written
    orr = O.rac_quantize_residual(xa.f32, oq, osel, on)
    assert np.array_equal(host(res.codes), orr.codes) and np.array_equal(host(res.scales), orr.scales)
    want = O.rac_merged_operand(oq, orr, osel, on)
    got = host(call.merged)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("shape", ["dense", "grouped", "decode", "dense_wide", "grouped_wide"])
def test_gemm_with_caller_merged_operand(shape):
    """The GEMM reads the operand quads_rac_select_merged wrote (no merge pass
    of its own) on the DMA-tile, large-tile and few-rows shapes; the *_wide
    shapes (N = 1536, about 30 row tiles, more tiles than CUs) add a ragged
    last row tile and, grouped, gathered rows and an empty expert."""
    if shape == "dense":
        wl = S.expert_gemm(M=512)
        xa, wa = wl.x, S.Activation(wl.w.f32[None], wl.w.bits[None])
        offs, rt = np.array([0, 512], np.int32), None
    elif shape == "dense_wide":
        wl = S.expert_gemm(M=4000)
        xa, wa = wl.x, S.Activation(wl.w.f32[None], wl.w.bits[None])
        offs, rt = np.array([0, 4000], np.int32), None
    elif shape == "grouped_wide":
        xa, wa, offs, rt = _grouped(609, [1100, 0, 777, 1123], 1500, 768, 1536)
    elif shape == "grouped":
        xa, wa, offs, rt = _grouped(604, [300, 0, 257, 511, 64, 1, 200, 129], 700, 768, 512)
    else:
        counts = [16, 0, 9, 16, 31, 1, 16, 12, 16, 16, 3, 16, 20, 16, 16, 8]
        xa, wa, offs, rt = _grouped(605, counts, 200, 512, 256)
    log(f"[gemm-rac] caller-merged operand, {shape}")
    x = dev_act(xa)
    E, N, K = wa.f32.shape
    wc, ws_, wg = quantize_weights_gpu(dev_act(wa), 1)
    q, scores = Q.quantize_nvfp4(x, want_scores=True)
    call = Q.SelectCall(x, q, scores, 50, merged=True)
    sel, res, nsel = call()
    R = int(offs[-1])
    y = Q.moe_w4a4_gemm(w_codes=wc, w_scales=ws_, w_gscale=wg, N=N, K=K, expert_offsets=torch.from_numpy(offs).cuda(),
                        num_rows=R, x=q, res=res, sel_idx=sel, x_merged=call.merged,
                        row_token=None if rt is None else torch.from_numpy(rt).cuda())
    _, _, _, we = O.quantize_weights(wa.f32, 1)
    ref = O.rac_linear(xa.f32, we, 50, rt, offs)["y"]
    err = rel_err(host(y), ref)
    log(f"  rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("k", [25, 50, 100])
def test_expert_gemm_full_size_merged_pipeline(k):
    """The expert-GEMM workload at full size (X 4096 x 2048 bf16, W 1536 x 2048)
    through the calls and launch configuration the throughput benchmark
    times: quads_rac_select_merged, then the GEMM on the caller's merged
    operand (128x128 register-staged tiles, merged steps). The operand is
    bit-exact against the oracle's rac_merged_operand and Y is within 1e-3
    of its float64 extended-K product."""
    wl = S.expert_gemm()
    M, K = wl.x.f32.shape
    N = wl.w.f32.shape[0]
    log(f"[gemm-rac] full-size merged pipeline {M}x{K}x{N} k={k}")
    x = dev_act(wl.x)
    wc, ws_, wg = quantize_weights_gpu(dev_act(wl.w)[None], 1)
    q, scores = Q.quantize_nvfp4(x, want_scores=True)
    call = Q.SelectCall(x, q, scores, k, merged=True)
    sel, res, nsel = call()
    y = Q.moe_w4a4_gemm(w_codes=wc, w_scales=ws_, w_gscale=wg, N=N, K=K,
                        expert_offsets=torch.tensor([0, M], dtype=torch.int32, device="cuda"), num_rows=M,
                        x=q, res=res, sel_idx=sel, x_merged=call.merged)
    oq = O.quantize_nvfp4(wl.x.f32)
    osel, on = O.rac_select(O.rac_scores(wl.x.f32, oq), k)
    assert nsel == on and np.array_equal(host(sel), osel)
    orr = O.rac_quantize_residual(wl.x.f32, oq, osel, on)
    want = O.rac_merged_operand(oq, orr, osel, on)
    assert np.array_equal(host(call.merged).view(np.uint16), want.view(np.uint16))
    _, _, _, we = O.quantize_weights(wl.w.f32[None], 1)
    err = rel_err(host(y), O.rac_linear(wl.x.f32, we, k)["y"])
    log(f"  rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("K", [2048, 8448])
def test_gemm_merge_step_operand_bit_exact(K):
    """The GEMM's own merge step (residual handed over, rac_form MERGED, no
    x_merged) builds the operand with the same row kernel as
    quads_rac_select_merged: its copy in the workspace (after the tile list,
    at byte align256(4 * (E + 1)), [act_rows, K] fp16) equals the oracle's
    rac_merged_operand bit for bit, for rows of at most 512 blocks and wider
    ones (K = 8448: four load slots per thread, one row per group), and Y
    is within the bar.  Decode-shaped counts: the few-rows kernel."""
    counts = [16, 9, 0, 31, 16, 1, 12, 16]
    T = 120
    xa, wa, offs, rt = _grouped(611 + K, counts, T, K, 256)
    log(f"[gemm-rac] merge step K={K} rows={T} k=50")
    x = dev_act(xa)
    E, N, _ = wa.f32.shape
    wc, ws_, wg = quantize_weights_gpu(dev_act(wa), 1)
    q, scores = Q.quantize_nvfp4(x, want_scores=True)
    sel, res, nsel = Q.rac_select(x, q, scores, 50)
    call = Q.GemmCall(w_codes=wc, w_scales=ws_, w_gscale=wg, N=N, K=K, expert_offsets=torch.from_numpy(offs).cuda(),
                      num_rows=int(offs[-1]), x=q, res=res, sel_idx=sel, row_token=torch.from_numpy(rt).cuda(),
                      rac_form=Q.RAC_FORM_MERGED)
    call.prepare()
    torch.cuda.synchronize()
    off = (4 * (E + 1) + 255) // 256 * 256
    got = call.ws[off:off + T * K * 2].view(torch.int16).cpu().numpy().view(np.uint16).reshape(T, K)
    oq = O.quantize_nvfp4(xa.f32)
    osel, on = O.rac_select(O.rac_scores(xa.f32, oq), 50)
    orr = O.rac_quantize_residual(xa.f32, oq, osel, on)
    want = O.rac_merged_operand(oq, orr, osel, on)
    assert np.array_equal(got, want.view(np.uint16)), np.argwhere(got != want.view(np.uint16))[:5]
    call.run()
    _, _, _, we = O.quantize_weights(wa.f32, 1)
    _check(host(call.y), O.rac_linear(xa.f32, we, 50, rt, offs)["y"], "merged")


@pytest.mark.parametrize("M,K,k", [(6001, 768, 50), (5000, 2048, 25), (3, 16384, 100), (9, 8208, 50)])
def test_rac_select_many_rows_bit_exact(M, K, k):
    """quads_rac_select (no merged operand) with more rows than 1024 row
    groups, and on the widest rows: mask, residual codes, scales and g_r
    bit-exact against the oracle."""
    log(f"[rac] many rows M={M} K={K} k={k}")
    rng = np.random.default_rng(606 + M)
    xa = S.activation(rng, M, K, max(1, K // 100), 30.0, bf16=True)
    x = dev_act(xa)
    q, scores = Q.quantize_nvfp4(x, want_scores=True)
    sel, res, nsel = Q.rac_select(x, q, scores, k)
    oq = O.quantize_nvfp4(xa.f32)
    osel, on = O.rac_select(O.rac_scores(xa.f32, oq), k)
    assert nsel == on and np.array_equal(host(sel), osel)
    orr = O.rac_quantize_residual(xa.f32, oq, osel, on)
    assert np.array_equal(host(res.codes), orr.codes) and np.array_equal(host(res.scales), orr.scales)
    assert host(res.gscale)[0] == np.float32(orr.g)
