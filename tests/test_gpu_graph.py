"""The hot path captured in a HIP graph (as the benchmark runs it) gives the
eager results bit for bit on every replay, with eager work and device
synchronisation between replays; and the eager results themselves match the
oracle (codes, scales and mask bit-exact, Y within 1e-3)."""
import numpy as np
import pytest
import torch

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import _lib as Q
from fp4_quantized_moe_amd import synthetic as S
from tests.gpu_util import dev_act, host, log, nvfp4_host, quantize_weights_gpu, rel_err

pytestmark = pytest.mark.gpu


def _outputs(q, scores, sel, res, y):
    # sel is an output only when channels are selected (its buffer has one
    # unused element at k=0)
    ts = (q.codes, q.scales, q.gscale, scores, res.codes, res.scales, res.gscale, y) + ((sel,) if res.cols else ())
    return [t.clone() for t in ts]


@pytest.mark.parametrize("k,merged", [(0, False), (50, False), (50, True)])
def test_graph_replay_matches_eager(k, merged):
    """merged: quads_rac_select_merged and the GEMM on that operand (the
    benchmark's default pipeline); otherwise the extended-K form."""
    wl = S.expert_gemm(M=1024)
    log(f"[graph] expert_gemm M=1024 k={k} merged={merged}")
    x, wd = dev_act(wl.x), dev_act(wl.w)
    M, K = wl.x.f32.shape
    N = wl.w.f32.shape[0]
    wc, wsc, wg = quantize_weights_gpu(wd[None], 1)
    offs = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    qc = Q.QuantizeCall(x, want_scores=True)
    q, scores = qc()
    sc = Q.SelectCall(x, q, scores, k, merged=merged)
    sel, res, nsel = sc()
    gc = Q.GemmCall(w_codes=wc, w_scales=wsc, w_gscale=wg, N=N, K=K, expert_offsets=offs, num_rows=M,
                    x=q, res=res if nsel else None, sel_idx=sel, x_merged=sc.merged if merged else None)
    gc()
    torch.cuda.synchronize()
    extra = (sc.merged,) if merged else ()
    eager = _outputs(q, scores, sel, res, gc.y) + [t.clone() for t in extra]

    # the eager results are the oracle's
    ref = O.quantize_nvfp4(wl.x.f32)
    codes, scales, g = nvfp4_host(q)
    assert g[0] == ref.g and np.array_equal(codes, ref.codes) and np.array_equal(scales, ref.scales)
    rsel, rn = O.rac_select(O.rac_scores(wl.x.f32, ref), k)
    assert nsel == rn and np.array_equal(host(sel)[:rn], rsel[:rn])
    _, _, _, we = O.quantize_weights(wl.w.f32[None], 1)
    yref = O.rac_linear(wl.x.f32, we, k)["y"]
    assert rel_err(host(gc.y), yref) <= 1e-3

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qc()
        sc()
        gc()
    other = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    for rep in range(3):
        for t in (q.codes, q.scales, res.codes, res.scales, sel):
            t.fill_(0x5A if t.dtype == torch.uint8 else -7)
        for t in (q.gscale, scores, res.gscale, gc.y) + extra:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(q, scores, sel, res, gc.y) + list(extra)
        for a, b in zip(eager, got):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rep
        # eager work between replays: the same calls on other data, then back
        Q.quantize_nvfp4(other, want_scores=True)
        torch.cuda.synchronize()


def test_graph_replay_decode_layer():
    """The decode-shaped RAC layer (route, quantize + RAC of x, few-rows gate_up
    with SwiGLU and its dense-residual prepare, quantize + RAC of h, down,
    combine) captured in one graph: every replay gives the eager output bit
    for bit, with eager work between replays."""
    wl = S.moe_decode()
    T, H = wl.x.f32.shape
    E, N2, _ = wl.w_gate_up.f32.shape
    I = N2 // 2
    k = wl.k_percent
    log(f"[graph] decode layer T={T} E={E} H={H} I={I} k={k}")
    x = dev_act(wl.x)
    logits = torch.from_numpy(wl.logits).cuda()
    guc, gus, gug = quantize_weights_gpu(dev_act(wl.w_gate_up), 2)
    dnc, dns, dng = quantize_weights_gpu(dev_act(wl.w_down), 1)
    rc = Q.RouteCall(logits, wl.top)
    ids, w, offs, rt, inv = rc()
    R = T * wl.top
    qx = Q.QuantizeCall(x, want_scores=True)
    xq, xs = qx()
    sx = Q.SelectCall(x, xq, xs, k)
    xsel, xres, _ = sx()
    g1 = Q.GemmCall(w_codes=guc, w_scales=gus, w_gscale=gug, n_seg=2, N=N2, K=H, expert_offsets=offs, num_rows=R,
                    x=xq, res=xres, sel_idx=xsel, row_token=rt, epilogue=Q.EPI_SWIGLU)
    g1()
    qh = Q.QuantizeCall(g1.y, want_scores=True)
    hq, hs = qh()
    sh = Q.SelectCall(g1.y, hq, hs, k)
    hsel, hres, _ = sh()
    g2 = Q.GemmCall(w_codes=dnc, w_scales=dns, w_gscale=dng, n_seg=1, N=H, K=I, expert_offsets=offs, num_rows=R,
                    x=hq, res=hres, sel_idx=hsel)
    g2()
    cc = Q.CombineCall(g2.y, inv, w)
    out = cc()
    torch.cuda.synchronize()
    eager = out.clone()
    assert torch.isfinite(eager).all()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rc()
        qx()
        sx()
        g1()
        qh()
        sh()
        g2()
        cc()
    other = torch.randn(T, H, device="cuda").to(torch.bfloat16)
    for rep in range(3):
        for t in (g1.y, g2.y, cc.out):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(cc.out.view(torch.int32), eager.view(torch.int32)), rep
        Q.quantize_nvfp4(other, want_scores=True)
        torch.cuda.synchronize()
