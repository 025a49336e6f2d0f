"""GPU parity: the W4A4 (+RAC) grouped expert GEMM and its bf16-operand
(trainer W4A16) mode through the C ABI vs the oracle's float64 reference.
Bar: max|Y - Y_ref| / max|Y_ref| <= 1e-3 with Y in FP32, where Y_ref
accumulates the same exactly dequantized operands in float64 (the operand
codes themselves are checked bit-exactly in test_gpu_quant_rac)."""
import numpy as np
import pytest
import torch

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import _lib as Q
from fp4_quantized_moe_amd import synthetic as S
from tests.gpu_util import dev_act, host, log, quantize_weights_gpu, rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _dense_case(x_act, w_act, k, row_token=None):
    """Run quantize -> RAC -> GEMM on the GPU for one expert; return (Y_gpu, Y_ref)."""
    x = dev_act(x_act)
    wd = dev_act(w_act)
    N, K = w_act.f32.shape
    wc, ws_, wg = quantize_weights_gpu(wd[None], 1)
    q, scores = Q.quantize_nvfp4(x, want_scores=True)
    sel, res, nsel = Q.rac_select(x, q, scores, k)
    M = x_act.f32.shape[0] if row_token is None else len(row_token)
    offs = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    rt = None if row_token is None else torch.from_numpy(np.asarray(row_token, np.int32)).cuda()
    y = Q.moe_w4a4_gemm(w_codes=wc, w_scales=ws_, w_gscale=wg, N=N, K=K, expert_offsets=offs, num_rows=M,
                        x=q, res=res if nsel else None, sel_idx=sel, row_token=rt)
    _, _, _, we = O.quantize_weights(w_act.f32[None], 1)
    ref = O.rac_linear(x_act.f32, we, k, row_token, None if row_token is None else np.array([0, M]))
    return host(y), ref["y"]


def test_gemm_dense_small_k50():
    wl = S.dense_small()
    log("[gemm] dense_small k=50")
    y, yr = _dense_case(wl.x, wl.w, 50)
    assert rel_err(y, yr) <= TOL


@pytest.mark.parametrize("k", [0, 25, 50, 100])
def test_gemm_expert_gemm(k):
    wl = S.expert_gemm()
    log(f"[gemm] expert_gemm 4096x2048x1536 k={k}")
    y, yr = _dense_case(wl.x, wl.w, k)
    e = rel_err(y, yr)
    log(f"  rel err {e:.3e}")
    assert e <= TOL


def test_k0_bit_exact_equals_plain():
    """k=0 selects nothing: the RAC call must produce exactly the plain W4A4 output."""
    wl = S.expert_gemm(M=384)
    x = dev_act(wl.x)
    wd = dev_act(wl.w)
    N, K = wl.w.f32.shape
    wc, ws_, wg = quantize_weights_gpu(wd[None], 1)
    q, scores = Q.quantize_nvfp4(x, want_scores=True)
    sel, res, nsel = Q.rac_select(x, q, scores, 0)
    assert nsel == 0
    offs = torch.tensor([0, 384], dtype=torch.int32, device="cuda")
    y0 = Q.moe_w4a4_gemm(w_codes=wc, w_scales=ws_, w_gscale=wg, N=N, K=K, expert_offsets=offs, num_rows=384,
                         x=q, res=res, sel_idx=sel)
    yp = Q.moe_w4a4_gemm(w_codes=wc, w_scales=ws_, w_gscale=wg, N=N, K=K, expert_offsets=offs, num_rows=384,
                         x=q)
    assert torch.equal(y0, yp)


def test_gemm_ragged_shapes():
    """Rows not a multiple of the 128-row tile, K with a partial 64-wide step,
    nsel not a multiple of 16 (zero-padded residual), and a gathered row order."""
    rng = np.random.default_rng(71)
    for M, K, N, k in [(1, 16, 128, 50), (77, 80, 128, 33), (200, 272, 256, 10), (129, 1040, 384, 77)]:
        log(f"[gemm] ragged M={M} K={K} N={N} k={k}")
        xa = S.activation(rng, M, K, 1, 20.0, bf16=True)
        wa = S.weights(rng, (N, K), 0.02, bf16=True)
        y, yr = _dense_case(xa, wa, k)
        assert rel_err(y, yr) <= TOL, (M, K, N, k)
        rt = rng.integers(0, M, size=2 * M + 3)
        y, yr = _dense_case(xa, wa, k, row_token=rt)
        assert rel_err(y, yr) <= TOL, ("gather", M, K, N, k)


def _grouped_setup(seed=72, T=300, H=256, E=8, I=128, top=2):
    rng = np.random.default_rng(seed)
    xa = S.activation(rng, T, H, 3, 30.0, bf16=True)
    logits = S.zipf_logits(rng, T, E)
    logits[:, 5] = -1e4  # expert 5 receives no rows
    wgu = S.weights(rng, (E, 2 * I, H))
    return xa, logits, wgu, top


def test_grouped_gemm_row_gather_and_empty_expert():
    xa, logits, wgu, top = _grouped_setup()
    T, H = xa.f32.shape
    E, N, _ = wgu.f32.shape
    ids, w, offs, rt, inv = O.route(logits, top)
    assert offs[6] == offs[5]
    x = dev_act(xa)
    wc, ws_, wg = quantize_weights_gpu(dev_act(wgu), 2)
    q, scores = Q.quantize_nvfp4(x, want_scores=True)
    sel, res, nsel = Q.rac_select(x, q, scores, 50)
    offs_d = torch.from_numpy(offs).cuda()
    rt_d = torch.from_numpy(rt).cuda()
    log("[gemm] grouped E=8 gather, EPI_NONE")
    y = Q.moe_w4a4_gemm(w_codes=wc, w_scales=ws_, w_gscale=wg, n_seg=2, N=N, K=H, expert_offsets=offs_d,
                        num_rows=len(rt), x=q, res=res, sel_idx=sel, row_token=rt_d)
    _, _, _, we = O.quantize_weights(wgu.f32, 2)
    ref = O.rac_linear(xa.f32, we, 50, rt, offs)
    assert rel_err(host(y), ref["y"]) <= TOL
    log("[gemm] grouped E=8 gather, EPI_SWIGLU")
    h = Q.moe_w4a4_gemm(w_codes=wc, w_scales=ws_, w_gscale=wg, n_seg=2, N=N, K=H, expert_offsets=offs_d,
                        num_rows=len(rt), x=q, res=res, sel_idx=sel, row_token=rt_d, epilogue=Q.EPI_SWIGLU)
    I = N // 2
    h_ref = O.swiglu(ref["y"][:, :I], ref["y"][:, I:])
    hh = host(h.float())
    # bf16 output (2^-9 relative) on top of the FP32 GEMM error (1e-3 of max|Y|, amplified by <= max|Y| via silu')
    ymax = np.abs(ref["y"]).max()
    tol = 2.0 ** -8 * np.abs(h_ref) + 2e-3 * ymax * (np.abs(ref["y"][:, I:]) + np.abs(ref["y"][:, :I]) + 1)
    assert (np.abs(hh - h_ref) <= tol).all()


def test_bf16_operand_mode_trainer_forward():
    """W4A16 forward: QDQ'd bf16 weights times bf16 activations."""
    rng = np.random.default_rng(73)
    T, H, E, I, top = 260, 256, 4, 128, 2
    xa = S.activation(rng, T, H, 0, 1.0, bf16=True)
    logits = S.gaussian_logits(rng, T, E)
    wgu = S.weights(rng, (E, 2 * I, H))
    ids, w, offs, rt, inv = O.route(logits, top)
    wq, _ = Q.weight_qdq(dev_act(wgu).reshape(E * 2, I, H))
    wq = wq.reshape(E, 2 * I, H)
    log("[gemm] bf16 operand mode")
    y = Q.moe_w4a4_gemm(N=2 * I, K=H, expert_offsets=torch.from_numpy(offs).cuda(), num_rows=len(rt),
                        row_token=torch.from_numpy(rt).cuda(), x_bf16=dev_act(xa), w_bf16=wq)
    wqh = host(wq.float()).astype(np.float64)
    ref = np.zeros((len(rt), 2 * I))
    for e in range(E):
        a, b = offs[e], offs[e + 1]
        ref[a:b] = xa.f32[rt[a:b]].astype(np.float64) @ wqh[e].T
    assert rel_err(host(y), ref) <= TOL
    # the QDQ'd weights are the oracle's
    for e in range(E):
        for s in range(2):
            bits, _ = O.weight_qdq(wgu.f32[e, s * I:(s + 1) * I])
            got = host(wq[e, s * I:(s + 1) * I].contiguous().view(torch.int16)).view(np.uint16)
            assert np.array_equal(got, bits)


@pytest.fixture(scope="module")
def experts_1024():
    """1024 experts (the largest count) of [128, 256] weights, quantized once."""
    rng = np.random.default_rng(95)
    wa = S.weights(rng, (1024, 128, 256), 0.02, bf16=True)
    _, _, _, we = O.quantize_weights(wa.f32, 1)
    xa = S.activation(rng, 4096, 256, 3, 30.0, bf16=True)
    return wa, we, xa


@pytest.mark.parametrize("rows,form", [(3000, "merged"), (36000, "exact"), (36000, "merged")])
def test_grouped_gemm_1024_experts(experts_1024, rows, form):
    """The largest expert count: Zipf-skewed rows with every seventh expert
    empty, gathered token rows.  3000 rows run the few-rows kernel, 36000
    rows (more than 32 per expert) the 128-row kernels over a tile list of
    1024 experts; both RAC forms."""
    wa, we, xa = experts_1024
    E, N, K = wa.f32.shape
    T = xa.f32.shape[0]
    rng = np.random.default_rng(96 + rows)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p[::7] = 0.0
    counts = rng.multinomial(rows, rng.permutation(p / p.sum()))
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rt = rng.integers(0, T, rows).astype(np.int32)
    log(f"[gemm] E=1024 rows={rows} ({int((counts == 0).sum())} empty experts) {form}")
    x = dev_act(xa)
    wc, ws_, wg = quantize_weights_gpu(dev_act(wa), 1)
    q, scores = Q.quantize_nvfp4(x, want_scores=True)
    sel, res, nsel = Q.rac_select(x, q, scores, 50)
    y = Q.moe_w4a4_gemm(w_codes=wc, w_scales=ws_, w_gscale=wg, N=N, K=K, expert_offsets=torch.from_numpy(offs).cuda(),
                        num_rows=rows, x=q, res=res, sel_idx=sel, row_token=torch.from_numpy(rt).cuda(),
                        rac_form=Q.RAC_FORM_MERGED if form == "merged" else Q.RAC_FORM_EXACT)
    err = rel_err(host(y), O.rac_linear(xa.f32, we, 50, rt, offs)["y"])
    log(f"  rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("rows,form", [(40, "merged"), (300, "exact"), (300, "merged")])
def test_grouped_gemm_largest_k(rows, form):
    """K = 16384, the largest contraction the RAC select and the merge step
    stage (k = 50: 8192 residual channels): 40 rows over two experts run the
    few-rows kernel, 300 rows the 128-row kernels; both RAC forms."""
    E, N, K, T = 2, 128, 16384, 200
    rng = np.random.default_rng(97 + rows)
    wa = S.weights(rng, (E, N, K), 0.02, bf16=True)
    xa = S.activation(rng, T, K, K // 100, 30.0, bf16=True)
    offs = np.array([0, rows // 3, rows], np.int32)
    rt = rng.integers(0, T, rows).astype(np.int32)
    log(f"[gemm] K={K} E={E} rows={rows} {form}")
    x = dev_act(xa)
    wc, ws_, wg = quantize_weights_gpu(dev_act(wa), 1)
    q, scores = Q.quantize_nvfp4(x, want_scores=True)
    sel, res, nsel = Q.rac_select(x, q, scores, 50)
    y = Q.moe_w4a4_gemm(w_codes=wc, w_scales=ws_, w_gscale=wg, N=N, K=K, expert_offsets=torch.from_numpy(offs).cuda(),
                        num_rows=rows, x=q, res=res, sel_idx=sel, row_token=torch.from_numpy(rt).cuda(),
                        rac_form=Q.RAC_FORM_MERGED if form == "merged" else Q.RAC_FORM_EXACT)
    _, _, _, we = O.quantize_weights(wa.f32, 1)
    err = rel_err(host(y), O.rac_linear(xa.f32, we, 50, rt, offs)["y"])
    log(f"  rel err {err:.2e}")
    assert err <= TOL
