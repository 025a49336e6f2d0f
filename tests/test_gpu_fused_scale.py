"""GPU parity of the output tensor scale formed inside the grouped GEMM
(quads_moe_gemm_args.y_gscale): on every kernel family that writes a bf16
output -- the large register-staged tiles (prefill gate_up, SwiGLU on the
merged RAC operand), the 128 x 128 DMA tiles and the few-rows kernel (decode
gate_up) -- y_gscale equals the oracle's tensor scale of the GPU's own
output h bit for bit, and quantizing h with that scale given
(QUADS_GSCALE_GIVEN) yields the same codes, scales and channel scores as the
quantizer's own amax pass.  Workgroups with empty tiles, repeated main-only
calls (the fold clears the gathered amax) and an all-zero output (g = 1)
are covered.  The fusion is the gist.science "Technische Samenvatting:
QUADS" section 2.2-B note that fused kernels keep the RAC overhead small."""
import numpy as np
import pytest
import torch

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import _lib as Q
from fp4_quantized_moe_amd import synthetic as S
from tests.gpu_util import dev_act, host, log, quantize_weights_gpu

pytestmark = pytest.mark.gpu


def _setup(seed, counts, T, K, N, zero_x=False):
    rng = np.random.default_rng(seed)
    xa = S.activation(rng, T, K, max(1, K // 100), 30.0, bf16=True)
    if zero_x:
        xa = S.Activation(np.zeros_like(xa.f32), np.zeros_like(xa.bits))
    wa = S.weights(rng, (len(counts), N, K))
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rt = rng.integers(0, T, int(offs[-1])).astype(np.int32)
    return xa, wa, offs, rt


def _gemm(xa, wa, offs, rt, n_seg, epilogue, merged, k=50, y_dtype=torch.float32, own_merge=False):
    x = dev_act(xa)
    E, N, K = wa.f32.shape
    wc, ws_, wg = quantize_weights_gpu(dev_act(wa), n_seg)
    q, scores = Q.quantize_nvfp4(x, want_scores=True)
    sel = res = xm = None
    if merged:
        sc = Q.SelectCall(x, q, scores, k, merged=True)
        sel, res, _ = sc()
        xm = None if own_merge else sc.merged
    gs = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    call = Q.GemmCall(w_codes=wc, w_scales=ws_, w_gscale=wg, n_seg=n_seg, N=N, K=K,
                      expert_offsets=torch.from_numpy(offs).cuda(), num_rows=int(offs[-1]), x=q, res=res,
                      sel_idx=sel, x_merged=xm, row_token=torch.from_numpy(rt).cuda(), epilogue=epilogue,
                      y_dtype=y_dtype, rac_form=Q.RAC_FORM_MERGED if merged else Q.RAC_FORM_AUTO, y_gscale=gs)
    return call, gs


def _check(call, gs, tag):
    h = host(call.y.view(torch.int16)).view(np.uint16)
    hf = O.f32_from_bf16_bits(h)
    g_gpu = host(gs)[0]
    g_ref = O.tensor_scale(hf)
    log(f"  {tag}: y_gscale {g_gpu!r} oracle {g_ref!r}")
    assert np.float32(g_gpu).view(np.uint32) == np.float32(g_ref).view(np.uint32)
    # the quantizer with that scale given = the quantizer's own amax pass
    y = call.y
    q_own, s_own = Q.quantize_nvfp4(y, want_scores=True)
    qc = Q.QuantizeCall(y, want_scores=True, gscale_given=True)
    qc.q.gscale.copy_(gs)
    q_giv, s_giv = qc()
    assert host(q_own.gscale)[0] == host(q_giv.gscale)[0]
    assert np.array_equal(host(q_own.codes), host(q_giv.codes))
    assert np.array_equal(host(q_own.scales), host(q_giv.scales))
    assert np.array_equal(host(s_own).view(np.uint32), host(s_giv).view(np.uint32))


def test_y_gscale_prefill_swiglu_large_tiles():
    """Gate_up with SwiGLU on the caller's merged operand, 8 experts (one
    empty) over 16384 routed rows: the 256 x 256 register-staged kernel."""
    counts = [4000, 0, 3100, 2600, 1900, 2300, 1500, 984]
    xa, wa, offs, rt = _setup(701, counts, 4096, 2048, 1536)
    log(f"[fused-g] prefill-shaped gate_up {counts} K=2048 N=1536 SwiGLU merged")
    call, gs = _gemm(xa, wa, offs, rt, 2, Q.EPI_SWIGLU, True)
    call()
    _check(call, gs, "large tiles")


def test_y_gscale_decode_swiglu_few_rows():
    """Decode-shaped gate_up (few rows per expert, some experts empty) with
    the GEMM's own merge step: the few-rows kernel."""
    counts = [16, 0, 9, 16, 31, 1, 16, 12, 0, 16, 3, 16, 20, 16, 16, 8]
    xa, wa, offs, rt = _setup(702, counts, 200, 1024, 512)
    log(f"[fused-g] decode-shaped gate_up {counts} K=1024 N=512 SwiGLU")
    call, gs = _gemm(xa, wa, offs, rt, 2, Q.EPI_SWIGLU, True, own_merge=True)
    call()
    _check(call, gs, "few rows")


@pytest.mark.parametrize("merged", [False, True])
def test_y_gscale_dma_tiles_bf16_output(merged):
    """bf16 output without epilogue on the 128 x 128 DMA tiles (plain W4A4
    and the merged operand); the grid has empty trailing tiles."""
    counts = [700, 300]
    xa, wa, offs, rt = _setup(703, counts, 900, 512, 256)
    log(f"[fused-g] DMA tiles bf16 y merged={merged}")
    call, gs = _gemm(xa, wa, offs, rt, 1, Q.EPI_NONE, merged, y_dtype=torch.bfloat16)
    call()
    _check(call, gs, "DMA tiles")


def test_y_gscale_repeated_main_calls_and_zero_output():
    """After one prepare, main-only calls keep returning the same scale (the
    fold clears the gathered amax), and an all-zero output gives 1."""
    counts = [16, 0, 9, 16, 31, 1, 16, 12]
    xa, wa, offs, rt = _setup(704, counts, 120, 512, 256)
    call, gs = _gemm(xa, wa, offs, rt, 2, Q.EPI_SWIGLU, False)
    call.prepare()
    got = []
    for _ in range(3):
        gs.fill_(float("nan"))
        call.run()
        got.append(np.float32(host(gs)[0]).view(np.uint32))
    log(f"[fused-g] repeated main calls: {[hex(int(v)) for v in got]}")
    assert got[0] == got[1] == got[2]
    _check(call, gs, "repeated")
    xz, wz, oz, rz = _setup(705, [40, 0, 17], 64, 512, 256, zero_x=True)
    callz, gz = _gemm(xz, wz, oz, rz, 2, Q.EPI_SWIGLU, False)
    callz()
    assert host(gz)[0] == np.float32(1.0)
    _check(callz, gz, "zero output")
