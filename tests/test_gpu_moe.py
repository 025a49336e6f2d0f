"""GPU parity: MoE routing / permutation (bit-exact indices), combine, and an
end-to-end W4A4+RAC MoE layer checked stage by stage against the oracle."""
import numpy as np
import pytest
import torch

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import _lib as Q
from fp4_quantized_moe_amd import synthetic as S
from tests.gpu_util import dev_act, host, log, quantize_weights_gpu, rel_err

pytestmark = pytest.mark.gpu


def _check_route(logits, top, tag):
    log(f"[route] {tag} T={logits.shape[0]} E={logits.shape[1]} top={top}")
    ids, w, offs, rt, inv = Q.moe_route(torch.from_numpy(logits).cuda(), top)
    rids, rw, roffs, rrt, rinv = O.route(logits, top)
    assert np.array_equal(host(ids), rids)
    assert np.array_equal(host(offs), roffs)
    assert np.array_equal(host(rt), rrt)
    assert np.array_equal(host(inv), rinv)
    assert np.allclose(host(w), rw, rtol=2e-6, atol=1e-9)
    return ids, w, offs, rt, inv, (rids, rw, roffs, rrt, rinv)


def test_route_decode_and_prefill_shapes():
    _check_route(S.moe_decode().logits, 8, "decode")
    wl = S.moe_prefill(T=4096, H=32, I=16)
    _check_route(wl.logits, 8, "prefill-zipf")


def test_route_ties_and_edge_shapes():
    rng = np.random.default_rng(81)
    lg = np.round(rng.standard_normal((700, 37)) * 2).astype(np.float32)
    _check_route(lg, 5, "ties")
    _check_route(rng.standard_normal((1, 16)).astype(np.float32), 16, "top=E")
    _check_route(rng.standard_normal((513, 1024)).astype(np.float32), 8, "E=1024")
    # both top-k kernels (ranking: E <= 64, or up to 256 experts with at
    # least 2048 tokens; argmax rounds otherwise): -inf logits, +0 / -0 ties,
    # rounded-value ties, E not a multiple of 4
    for T in (300, 2048):
        lg = rng.standard_normal((T, 130)).astype(np.float32)
        lg[:, 5] = -np.inf
        lg[::3, 7] = 0.0
        lg[::3, 9] = -0.0
        lg[::3, 11] = 0.0
        _check_route(lg, 8, f"E=130 T={T} -inf and signed-zero ties")
    for T in (257, 2100):
        _check_route(np.round(rng.standard_normal((T, 200)) * 2).astype(np.float32), 8, f"E=200 T={T} ties")
    _check_route(np.round(rng.standard_normal((64, 63)) * 3).astype(np.float32), 6, "E=63 ties")
    _check_route(np.round(rng.standard_normal((2048, 100)) * 2).astype(np.float32), 8, "E=100 T=2048 ties")
    _check_route(np.round(rng.standard_normal((100, 300)) * 2).astype(np.float32), 8, "E=300 ties")


def test_route_nan_logits():
    """Rows with NaN logits, fewer real logits than top, NaN mixed with -inf:
    every id is a valid expert and the ids, offsets and rows equal the
    oracle's (its stable descending sort puts NaN after -inf, ties to the
    lower index).  Covers the argmax-round kernel (E=128 T=256, E=300) and
    the ranking kernel (E=64 T=2048).  Weights of NaN rows are unspecified
    and not compared."""
    rng = np.random.default_rng(83)
    for T, E in ((256, 128), (100, 300), (2048, 64), (2048, 130)):
        lg = rng.standard_normal((T, E)).astype(np.float32)
        lg[::2, :] = np.nan                      # whole rows NaN
        lg[1::4, 3:] = np.nan                    # three real logits, then NaN
        lg[3::4, ::2] = np.nan                   # NaN interleaved with -inf and reals
        lg[3::4, 1::3] = -np.inf
        lg[5::8, :E - 2] = -np.inf               # two reals, the rest -inf
        log(f"[route] NaN rows T={T} E={E}")
        ids, w, offs, rt, inv = Q.moe_route(torch.from_numpy(lg).cuda(), 8)
        rids, rw, roffs, rrt, rinv = O.route(lg, 8)
        h = host(ids)
        assert h.min() >= 0 and h.max() < E
        assert np.array_equal(h, rids)
        assert np.array_equal(host(offs), roffs)
        assert np.array_equal(host(rt), rrt)
        assert np.array_equal(host(inv), rinv)
        fin = np.isfinite(lg).all(axis=1)
        if fin.any():
            assert np.allclose(host(w)[fin], rw[fin], rtol=2e-6, atol=1e-9)


@pytest.mark.parametrize("top", [8, 4])
def test_combine(top):
    """Combine against the oracle's float64 sum, and bit for bit against the
    FP32 sum in slot order (each product rounded, then added), the kernel's
    stated operation order (top 8 has its own kernel with all loads hoisted)."""
    rng = np.random.default_rng(82 + top)
    T, N = 123, 256
    logits = S.gaussian_logits(rng, T, 16)
    *_, (rids, rw, roffs, rrt, rinv) = _check_route(logits, top, "combine")
    y = rng.standard_normal((T * top, N)).astype(np.float32)
    w32 = rw.astype(np.float32)
    out = host(Q.moe_combine(torch.from_numpy(y).cuda(), torch.from_numpy(rinv).cuda(),
                             torch.from_numpy(w32).cuda()))
    ref = O.combine(y, rinv, w32.astype(np.float64))
    assert rel_err(out, ref) <= 1e-6
    acc = np.zeros((T, N), np.float32)
    for j in range(top):
        acc = (acc + (w32[:, j:j + 1] * y[rinv[:, j]]).astype(np.float32)).astype(np.float32)
    assert np.array_equal(out.view(np.uint32), acc.view(np.uint32))


def _layer_setup(seed=83, T=192, H=256, E=16, I=128, top=4):
    rng = np.random.default_rng(seed)
    xa = S.activation(rng, T, H, 3, 30.0, bf16=True)
    logits = S.zipf_logits(rng, T, E)
    wgu = S.weights(rng, (E, 2 * I, H))
    wdn = S.weights(rng, (E, H, I))
    return rng, xa, logits, wgu, wdn, top


def test_moe_down_stage_on_seeded_h():
    """Down projection stage on a seeded bf16 h (identity rows, per-expert
    offsets from the routing): codes, mask and residual bit-exact; Y within 1e-3."""
    rng, xa, logits, wgu, wdn, top = _layer_setup()
    E, H, I = wdn.f32.shape
    T = xa.f32.shape[0]
    ids, w, offs, rt, inv, oref = _check_route(logits, top, "down-stage")
    roffs = oref[2]
    ha = S.activation(rng, T * top, I, 2, 8.0, bf16=True)
    h = dev_act(ha)
    dnc, dns, dng = quantize_weights_gpu(dev_act(wdn), 1)
    hq, hsc = Q.quantize_nvfp4(h, want_scores=True)
    hsel, hres, _ = Q.rac_select(h, hq, hsc, 50)
    y = Q.moe_w4a4_gemm(w_codes=dnc, w_scales=dns, w_gscale=dng, n_seg=1, N=H, K=I, expert_offsets=offs,
                        num_rows=T * top, x=hq, res=hres, sel_idx=hsel)
    _, _, _, dne = O.quantize_weights(wdn.f32, 1)
    rd = O.rac_linear(ha.f32, dne, 50, None, roffs)
    assert np.array_equal(host(hq.codes), rd["q"].codes)
    assert np.array_equal(host(hsel), rd["sel"])
    assert np.array_equal(host(hres.codes), rd["r"].codes)
    assert rel_err(host(y), rd["y"]) <= 1e-3


def test_moe_layer_end_to_end_small():
    """Route -> quantize+RAC -> gate_up (SwiGLU) -> quantize+RAC on h -> down ->
    combine on the GPU vs the oracle's own chain.  The gate_up stage is held to
    the stage tolerance; the chained output is compared at 2e-2 of max|out|:
    h differs from the oracle's by FP32-vs-FP64 accumulation and a bf16 rounding,
    which can move a few requantized codes by one E2M1 step.  The stage-wise
    tests hold each step to the exact/1e-3 bar."""
    rng, xa, logits, wgu, wdn, top = _layer_setup()
    T, H = xa.f32.shape
    E, _, I = wdn.f32.shape
    k = 50
    ids, w, offs, rt, inv, _ = _check_route(logits, top, "layer")
    x = dev_act(xa)
    guc, gus, gug = quantize_weights_gpu(dev_act(wgu), 2)
    dnc, dns, dng = quantize_weights_gpu(dev_act(wdn), 1)
    q, sc = Q.quantize_nvfp4(x, want_scores=True)
    sel, res, _ = Q.rac_select(x, q, sc, k)
    R = T * top
    h = Q.moe_w4a4_gemm(w_codes=guc, w_scales=gus, w_gscale=gug, n_seg=2, N=2 * I, K=H, expert_offsets=offs,
                        num_rows=R, x=q, res=res, sel_idx=sel, row_token=rt, epilogue=Q.EPI_SWIGLU)
    hq, hsc = Q.quantize_nvfp4(h, want_scores=True)
    hsel, hres, _ = Q.rac_select(h, hq, hsc, k)
    y = Q.moe_w4a4_gemm(w_codes=dnc, w_scales=dns, w_gscale=dng, n_seg=1, N=H, K=I, expert_offsets=offs,
                        num_rows=R, x=hq, res=hres, sel_idx=hsel)
    out = Q.moe_combine(y, inv, w)
    _, _, _, gue = O.quantize_weights(wgu.f32, 2)
    _, _, _, dne = O.quantize_weights(wdn.f32, 1)
    ref = O.moe_layer(xa.f32, logits, gue, dne, k, top)
    assert rel_err(host(h.float()), ref["h"]) <= 1e-2
    assert rel_err(host(out), ref["out"]) <= 2e-2


def test_prefill_layer_full_size_sampled_experts():
    """The prefill-shaped layer at full size (16384 tokens, hidden 2048, 64
    experts with Zipf-skewed top-8 routing, intermediate 768, k=50) as the
    benchmark launches it; the oracle recomputes the rows of the largest,
    smallest and one random non-empty expert of the gate_up GEMM (FP32 and
    SwiGLU outputs) and of the down GEMM on a seeded h; the RAC of that h
    (131072 x 768) is checked bit for bit, with and without the merged
    operand."""
    wl = S.moe_prefill()
    T, H = wl.x.f32.shape
    E, N2, _ = wl.w_gate_up.f32.shape
    I = N2 // 2
    k = wl.k_percent
    log(f"[moe] prefill full size T={T} E={E} H={H} I={I} k={k}")
    ids, w, offs, rt, inv = Q.moe_route(torch.from_numpy(wl.logits).cuda(), wl.top)
    _, _, roffs, rrt, _ = O.route(wl.logits, wl.top)
    assert np.array_equal(host(offs), roffs) and np.array_equal(host(rt), rrt)
    R = int(roffs[-1])
    x = dev_act(wl.x)
    guc, gus, gug = quantize_weights_gpu(dev_act(wl.w_gate_up), 2)
    q, sc = Q.quantize_nvfp4(x, want_scores=True)
    sel, res, nsel = Q.rac_select(x, q, sc, k)
    args = dict(w_codes=guc, w_scales=gus, w_gscale=gug, n_seg=2, N=N2, K=H, expert_offsets=offs, num_rows=R,
                x=q, res=res, sel_idx=sel, row_token=rt)
    y = host(Q.moe_w4a4_gemm(**args))
    h = host(Q.moe_w4a4_gemm(epilogue=Q.EPI_SWIGLU, **args).float())
    xq = O.quantize_nvfp4(wl.x.f32)
    xsel, xn = O.rac_select(O.rac_scores(wl.x.f32, xq), k)
    xr = O.rac_quantize_residual(wl.x.f32, xq, xsel, xn)
    assert np.array_equal(host(q.codes), xq.codes) and np.array_equal(host(sel), xsel)
    assert np.array_equal(host(res.codes), xr.codes)
    xe = O.dequant_exact(xq.codes, xq.scales, xq.g)
    re = O.dequant_exact(xr.codes, xr.scales, xr.g)
    cnt = np.diff(roffs)
    nz = np.flatnonzero(cnt)
    pick = sorted({int(nz[np.argmax(cnt[nz])]), int(nz[np.argmin(cnt[nz])]),
                   int(np.random.default_rng(97).choice(nz))})
    for e in pick:
        a, b = int(roffs[e]), int(roffs[e + 1])
        _, _, _, we = O.quantize_weights(wl.w_gate_up.f32[e:e + 1], 2)
        yr = O.gemm_ref(xe[rrt[a:b]], we[0], re[rrt[a:b]], xsel)
        err = rel_err(y[a:b], yr)
        log(f"  gate_up expert {e} rows {b - a}: rel err {err:.2e}")
        assert err <= 1e-3, e
        hr = O.swiglu(yr[:, :I], yr[:, I:])
        ymax = np.abs(yr).max()
        tol = 2.0 ** -8 * np.abs(hr) + 2e-3 * ymax * (np.abs(yr[:, I:]) + np.abs(yr[:, :I]) + 1)
        assert (np.abs(h[a:b] - hr) <= tol).all(), e

    rng = np.random.default_rng(98)
    ha = S.activation(rng, R, I, 2, 8.0, bf16=True)
    hd = dev_act(ha)
    dnc, dns, dng = quantize_weights_gpu(dev_act(wl.w_down), 1)
    hq, hsc = Q.quantize_nvfp4(hd, want_scores=True)
    hsel, hres, _ = Q.rac_select(hd, hq, hsc, k)
    yd = host(Q.moe_w4a4_gemm(w_codes=dnc, w_scales=dns, w_gscale=dng, n_seg=1, N=H, K=I, expert_offsets=offs,
                              num_rows=R, x=hq, res=hres, sel_idx=hsel))
    oq = O.quantize_nvfp4(ha.f32)
    osel, on = O.rac_select(O.rac_scores(ha.f32, oq), k)
    orr = O.rac_quantize_residual(ha.f32, oq, osel, on)
    assert np.array_equal(host(hsel), osel) and np.array_equal(host(hres.codes), orr.codes)
    # the same h through quads_rac_select_merged: 131072 rows of 768 channels,
    # many row groups per workgroup (each workgroup finds the mask itself)
    mcall = Q.SelectCall(hd, hq, hsc, k, merged=True)
    msel, mres, _ = mcall()
    assert np.array_equal(host(msel), osel) and np.array_equal(host(mres.codes), orr.codes)
    assert np.array_equal(host(mres.scales), orr.scales) and host(mres.gscale)[0] == np.float32(orr.g)
    want = O.rac_merged_operand(oq, orr, osel, on)
    assert np.array_equal(host(mcall.merged).view(np.uint16), want.view(np.uint16))
    del want
    he = O.dequant_exact(oq.codes, oq.scales, oq.g)
    hre = O.dequant_exact(orr.codes, orr.scales, orr.g)
    for e in pick:
        a, b = int(roffs[e]), int(roffs[e + 1])
        _, _, _, we = O.quantize_weights(wl.w_down.f32[e:e + 1], 1)
        yr = O.gemm_ref(he[a:b], we[0], hre[a:b], osel)
        err = rel_err(yd[a:b], yr)
        log(f"  down expert {e} rows {b - a}: rel err {err:.2e}")
        assert err <= 1e-3, e


def test_prefill_merged_pipeline_full_size_sampled_experts():
    """The prefill layer's gate_up exactly as the benchmark launches it
    (16384 tokens, 64 Zipf-routed experts, k=50): quads_rac_select_merged
    writes the corrected fp16 activation, bit-exact against the oracle's
    rac_merged_operand on every element, and the grouped GEMM reads it as
    x_merged on 256 x 256 tiles (MODE 2), with FP32 output and with the
    SwiGLU epilogue; the largest, smallest and one random non-empty expert
    are checked against the oracle's float64 extended-K product."""
    wl = S.moe_prefill()
    T, H = wl.x.f32.shape
    E, N2, _ = wl.w_gate_up.f32.shape
    I = N2 // 2
    k = wl.k_percent
    log(f"[moe] prefill merged pipeline full size T={T} E={E} H={H} I={I} k={k}")
    ids, w, offs, rt, inv = Q.moe_route(torch.from_numpy(wl.logits).cuda(), wl.top)
    _, _, roffs, rrt, _ = O.route(wl.logits, wl.top)
    assert np.array_equal(host(offs), roffs) and np.array_equal(host(rt), rrt)
    R = int(roffs[-1])
    x = dev_act(wl.x)
    guc, gus, gug = quantize_weights_gpu(dev_act(wl.w_gate_up), 2)
    q, sc = Q.quantize_nvfp4(x, want_scores=True)
    call = Q.SelectCall(x, q, sc, k, merged=True)
    sel, res, nsel = call()
    xq = O.quantize_nvfp4(wl.x.f32)
    xsel, xn = O.rac_select(O.rac_scores(wl.x.f32, xq), k)
    xr = O.rac_quantize_residual(wl.x.f32, xq, xsel, xn)
    assert nsel == xn and np.array_equal(host(sel), xsel)
    want = O.rac_merged_operand(xq, xr, xsel, xn)
    assert np.array_equal(host(call.merged).view(np.uint16), want.view(np.uint16))
    args = dict(w_codes=guc, w_scales=gus, w_gscale=gug, n_seg=2, N=N2, K=H, expert_offsets=offs, num_rows=R,
                x=q, res=res, sel_idx=sel, row_token=rt, x_merged=call.merged, rac_form=Q.RAC_FORM_MERGED)
    y = host(Q.moe_w4a4_gemm(**args))
    h = host(Q.moe_w4a4_gemm(epilogue=Q.EPI_SWIGLU, **args).float())
    xe = O.dequant_exact(xq.codes, xq.scales, xq.g)
    re = O.dequant_exact(xr.codes, xr.scales, xr.g)
    cnt = np.diff(roffs)
    nz = np.flatnonzero(cnt)
    pick = sorted({int(nz[np.argmax(cnt[nz])]), int(nz[np.argmin(cnt[nz])]),
                   int(np.random.default_rng(98).choice(nz))})
    for e in pick:
        a, b = int(roffs[e]), int(roffs[e + 1])
        _, _, _, we = O.quantize_weights(wl.w_gate_up.f32[e:e + 1], 2)
        yr = O.gemm_ref(xe[rrt[a:b]], we[0], re[rrt[a:b]], xsel)
        err = rel_err(y[a:b], yr)
        log(f"  expert {e} rows {b - a}: gate_up rel err {err:.2e}")
        assert err <= 1e-3
        hr = O.swiglu(yr[:, :I], yr[:, I:])
        tol = 2.0 ** -8 * np.abs(hr) + 2e-3 * np.abs(yr).max() * (np.abs(yr[:, I:]) + np.abs(yr[:, :I]) + 1)
        assert (np.abs(h[a:b] - hr) <= tol).all()


def test_moe_layer_no_tokens():
    """A layer call with no tokens: routing writes all-zero expert offsets,
    the activation's tensor scale is 1 and its scores 0, the select keeps the
    first nsel channels, the GEMM (few-rows kernel at K = 256, 128-row
    kernels at K = 272) writes only the output tensor scale (1) and combine
    nothing; every call returns OK with empty (NULL) row buffers."""
    E, I, top = 16, 256, 8
    rng = np.random.default_rng(91)
    ids, tw, offs, rt, inv = Q.moe_route(torch.empty(0, E, dtype=torch.float32, device="cuda"), top)
    assert host(offs).tolist() == [0] * (E + 1)
    for H in (256, 272):
        log(f"[moe] no tokens E={E} H={H} I={I}")
        x = torch.empty(0, H, dtype=torch.bfloat16, device="cuda")
        q, scores = Q.quantize_nvfp4(x, want_scores=True)
        assert host(q.gscale)[0] == np.float32(1.0) and not host(scores).any()
        sel, res, nsel = Q.SelectCall(x, q, scores, 50, merged=True)()
        assert np.array_equal(host(sel)[:nsel], np.arange(nsel))
        wgu = S.weights(rng, (E, 2 * I, H), 0.02, bf16=True)
        guc, gus, gug = quantize_weights_gpu(dev_act(wgu), 2)
        g_h = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
        h = Q.moe_w4a4_gemm(w_codes=guc, w_scales=gus, w_gscale=gug, n_seg=2, N=2 * I, K=H, expert_offsets=offs,
                            num_rows=0, x=q, res=res, sel_idx=sel, row_token=rt, epilogue=Q.EPI_SWIGLU, y_gscale=g_h)
        assert tuple(h.shape) == (0, I) and host(g_h)[0] == np.float32(1.0)
        out = Q.moe_combine(torch.empty(0, H, dtype=torch.float32, device="cuda"), inv, tw)
        torch.cuda.synchronize()
        assert tuple(out.shape) == (0, H)
