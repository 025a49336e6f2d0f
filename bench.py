#!/usr/bin/env python3
"""Benchmark of the QUADS rollout hot path on one MI355X (gfx950).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--k 50]

Prints ONE JSON line.  A step is one pass of the hot path over one batch of
synthetic, seeded input already resident in HBM:

  expert_gemm (default): one expert-sized linear, X bf16 4096 x 2048 with 1%
      outlier channels, W 1536 x 2048 NVFP4 (quantized once, outside the
      step): quantize X + RAC channel scores -> top-k% mask + second-pass
      residual quantization -> tile list + selected-column gather -> grouped
      W4A4+RAC GEMM (FP32 out).  The plain W4A4 step (quantize + GEMM) is timed
      beside it for the RAC overhead.
  moe_prefill: 16384 tokens, hidden 2048, 64 experts, top-8 Zipf-skewed
      routing, SwiGLU 2048->768->2048: route -> quantize+RAC(X) -> gate_up
      (SwiGLU epilogue) -> quantize+RAC(h) -> down -> combine.
  moe_decode: the same layer at 256 tokens, 128 experts, intermediate 1024.
  trainer_qdq: per layer, NVFP4 QDQ of 128 experts x (gate, up, down) bf16
      master weights, then the bf16 grouped forward on 8192 tokens.
  trainer_bwd: one layer's W4A16 QAT backward at the trainer shape (8192
      tokens, 128 experts, top-8, gate_up 2048 -> 2048, down 1024 -> 2048):
      per projection, transpose of W_qdq, dX grouped GEMM (+ per-token sum for
      gate_up) and the dW grouped GEMM (FP32), from synthetic output gradients.
  ablation: not a throughput run.  Output error of every trainer and rollout
      variant (bf16, asymmetric W4A16, symmetric W4A4 QAT, W4A4, RAC with one
      mask per tensor or per expert) against the float64 product of the
      masters, and the trainer/rollout output mismatch with a drifted rollout
      activation, on the expert-GEMM shape and on the decode-shaped down
      projection (128 experts, routed rows of 256 tokens x top-8, 1024 -> 2048).

`value` is tokens per second of the whole step; `roofline` describes the
dominant kernel (its average duration from HIP events recorded on the
stream it runs on, inside the timed steps): `achieved` counts the
algorithmic work of the survey's per-unit figures (2*M*N*(K+nsel) flops for
a RAC GEMM, bytes for a bandwidth-bound kernel) and `executed` the MFMA work
the kernel really issues; `cpu_baseline` is the CPU oracle timed on a
bounded sample of the same workload on the host cores.

The default run also measures the prefill-shaped (moe_prefill) and
decode-shaped (moe_decode) MoE layers and one trainer layer's weight QDQ,
each in its own block under `workloads` with its step time, tokens/s, RAC
overhead over plain W4A4, roofline and CPU baseline (--no-moe skips them).
Bandwidth-bound stages report algorithmic GB/s twice: back to back (20 calls
in a HIP graph; inputs may sit in the 256 MB Infinity Cache) and cold (one
call between HIP events after a 1 GiB write evicts the cache).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE W4A4+RAC expert-GEMM tokens/s & TFLOPS; % of MFMA peak; RAC overhead %"
PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 MFMA
PEAK_HBM_GBS = 8000.0
CPU_BASELINE_MIN_S = 10.0  # repeat the oracle sample until at least this much CPU time
# RAC steps write the merged fp16 activation (quads_rac_select_merged) and the
# GEMMs read it; --rac-form exact times the extended-K formulation instead.
MERGED_RAC = True


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="expert_gemm",
                    choices=["expert_gemm", "moe_prefill", "moe_decode", "trainer_qdq", "trainer_bwd", "ablation"])
    ap.add_argument("--k", type=int, default=50, help="RAC k percent")
    ap.add_argument("--layers", type=int, default=48, help="trainer_qdq: layers per step")
    ap.add_argument("--qdq", choices=["separate", "in_gemm", "codes"], default="separate",
                    help="trainer_qdq: weight QDQ as a separate pass, inside the GEMMs (QUADS_OPERANDS_BF16_QDQ), "
                         "or as an NVFP4 encoding the GEMMs decode (QUADS_OPERANDS_BF16_W4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-plain", action="store_true", help="skip the plain W4A4 comparison run")
    ap.add_argument("--graph", action="store_true", help="replay the non-dominant stages as HIP graphs")
    ap.add_argument("--no-moe", action="store_true",
                    help="expert_gemm: skip the prefill, decode and QDQ blocks")
    ap.add_argument("--rac-form", choices=["merged", "exact"], default="merged",
                    help="RAC correction: merged fp16 operand from quads_rac_select_merged, or the exact "
                         "extended-K contraction (QUADS_RAC_FORM_EXACT)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# workloads: each returns a dict with the step's stages and accounting
# ---------------------------------------------------------------------------

def _dev(a):
    import torch
    if a.bits is not None:
        return torch.from_numpy(a.bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a.f32)).cuda()


def _weights_nvfp4(Q, w_dev, n_seg):
    E, N, K = w_dev.shape
    q, _ = Q.quantize_nvfp4(w_dev.reshape(E * n_seg, N // n_seg, K))
    return q.codes.reshape(E, N, K // 2), q.scales.reshape(E, N, K // 16), q.gscale


def _act_bytes(rows, K, kpad, merged):
    """Algorithmic bytes of the bandwidth-bound activation stages on a bf16
    [rows, K] activation: quantize with scores reads x (2 B) and writes codes
    (0.5 B) and block scales (1/16 B) per element, plus the K fp32 scores;
    RAC re-reads x, codes and scales and writes the residual NVFP4 tensor
    (0.5625 B per selected element) and, in the merged form, the fp16
    corrected activation (2 B per element)."""
    q = rows * K * 2.5625 + 4.0 * K
    rac = rows * K * 2.5625 + 4.0 * K + rows * kpad * 0.5625 + (rows * K * 2.0 if merged else 0.0)
    return q, rac


def setup_expert_gemm(Q, S, k):
    import torch
    wl = S.expert_gemm()
    x, w = _dev(wl.x), _dev(wl.w)
    M, K = wl.x.f32.shape
    N = wl.w.f32.shape[0]
    wc, wsc, wg = _weights_nvfp4(Q, w[None], 1)
    offs = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    qc = Q.QuantizeCall(x, want_scores=True)
    q, scores = qc()
    merged = MERGED_RAC and k > 0
    scall = Q.SelectCall(x, q, scores, k, merged=merged)
    sel, res, nsel = scall()
    gc = Q.GemmCall(w_codes=wc, w_scales=wsc, w_gscale=wg, N=N, K=K, expert_offsets=offs, num_rows=M,
                    x=q, res=res if nsel else None, sel_idx=sel, x_merged=scall.merged if merged else None,
                    rac_form=Q.RAC_FORM_MERGED if merged else Q.RAC_FORM_EXACT)
    # Algorithmic work of the RAC GEMM: the extended contraction, 2*M*N*(K +
    # nsel).  MFMA work it executes: one contraction over K on the merged
    # operand (the correction is summed into it), K + nsel otherwise.
    flops_alg = 2.0 * M * N * (K + nsel)
    flops_exec = 2.0 * M * N * (K + (0 if merged else nsel))
    stages = [("quantize_scores", qc), ("rac_select_residual", scall), ("gemm_prepare", gc.prepare),
              ("gemm", gc.run)]
    qp = Q.QuantizeCall(x, want_scores=False)
    qpl, _ = qp()
    gp = Q.GemmCall(w_codes=wc, w_scales=wsc, w_gscale=wg, N=N, K=K, expert_offsets=offs, num_rows=M, x=qpl)
    plain = [("quantize", qp), ("gemm_prepare", gp.prepare), ("gemm", gp.run)]
    qb, rb = _act_bytes(M, K, res.cols, merged)
    cfg = {"workload": "expert_gemm", "tokens": M, "K": K, "N": N, "k_percent": k, "nsel": nsel,
           "x": "bf16 N(0,1), 1% outlier channels x30", "w": "bf16 N(0,0.02) -> NVFP4 (offline)",
           "rac_gemm": ("merged fp16 operand from quads_rac_select_merged (executes 2*M*N*K)" if merged else
                        "extended K (executes 2*M*N*(K+nsel))")}

    def cpu_baseline():
        """The oracle's quantize + RAC + fp64 GEMM over all M tokens (the same
        step), repeated until CPU_BASELINE_MIN_S have passed."""
        from oracle import quads_oracle as O
        qw = O.quantize_nvfp4(wl.w.f32)
        we = O.dequant_exact(qw.codes, qw.scales, qw.g)[None]
        reps, t0 = 0, time.perf_counter()
        while True:
            O.rac_linear(wl.x.f32, we, k)
            reps += 1
            secs = time.perf_counter() - t0
            if secs >= CPU_BASELINE_MIN_S:
                break
        return M * reps / secs, secs, (f"the whole step ({M} tokens, K={K}, N={N}, k={k}%) x {reps} repetitions: "
                                       "oracle quantize + RAC + fp64 GEMM (weights quantized beforehand)")

    kern = ("k_gemm<Cfg<128, 128, 2, 2, 2>, 2, 0, false> (merged RAC operand x NVFP4 weights, 128x128 "
            "register-staged tiles)" if merged else "k_gemm_dma<2, 0, true> (W4A4 + RAC segment, 128x128 DMA-staged tiles)")
    summary = (f"k_gemm_merged_expert_gemm_k{k}_traffic.txt" if merged else f"k_gemm_dma_expert_gemm_k{k}_traffic.txt")
    return dict(stages=stages, plain=plain, tokens=M, flops=flops_alg, dominant="gemm", bound="mfma",
                dominant_work=flops_alg, dominant_exec=flops_exec, dominant_kernel=kern, config=cfg,
                cpu_baseline=cpu_baseline, traffic_summary=os.path.join(ROOT, "profiles", summary),
                stage_bytes={"quantize_scores": qb, "rac_select_residual": rb},
                plain_stage_bytes={"quantize": M * K * 2.5625})


def cpu_baseline_moe(wl, k, every):
    """The oracle on a bounded sample of one MoE layer step: routing, and
    quantize + scores + mask + residual of the whole X (one mask per batch),
    timed in full; gate_up (fp64 GEMM with the RAC correction), SwiGLU
    rounded to bf16, quantize + RAC of those rows of h and the down GEMM,
    timed for every `every`-th expert and scaled to all routed rows by row
    count (the combine is not included).  Weights of the sampled experts are
    quantized beforehand, as on the GPU.  Returns (tokens/s, seconds, sample)."""
    from oracle import quads_oracle as O
    T, H = wl.x.f32.shape
    E = wl.logits.shape[1]
    I = wl.w_down.f32.shape[2]
    sample = list(range(0, E, every))
    wgu = {e: O.quantize_weights(wl.w_gate_up.f32[e:e + 1], 2)[3][0] for e in sample}
    wdn = {e: O.quantize_weights(wl.w_down.f32[e:e + 1], 1)[3][0] for e in sample}
    t0 = time.perf_counter()
    ids, wts, offs, rt, inv = O.route(wl.logits, wl.top)
    t_route = time.perf_counter() - t0
    t0 = time.perf_counter()
    x = wl.x.f32
    q = O.quantize_nvfp4(x)
    sel, nsel = O.rac_select(O.rac_scores(x, q), k)
    r = O.rac_quantize_residual(x, q, sel, nsel)
    xe = O.dequant_exact(q.codes, q.scales, q.g)
    re = O.dequant_exact(r.codes, r.scales, r.g) if nsel else None
    t_x = time.perf_counter() - t0
    # the sampled experts are cycled until CPU_BASELINE_MIN_S of row work
    # has been timed (at least one pass)
    rows_done, passes, t0 = 0, 0, time.perf_counter()
    for e in sample * 1000:
        if e == sample[0] and rows_done and time.perf_counter() - t0 >= CPU_BASELINE_MIN_S:
            break
        passes += e == sample[0]
        a, b = int(offs[e]), int(offs[e + 1])
        if a == b:
            continue
        rows = rt[a:b]
        y = O.gemm_ref(xe[rows], wgu[e], None if re is None else re[rows], sel if nsel else None)
        h = O.swiglu(y[:, :I], y[:, I:])
        hb = O.f32_from_bf16_bits(O.bf16_bits_from_f32(h.astype(np.float32)))
        hq = O.quantize_nvfp4(hb)
        hsel, hn = O.rac_select(O.rac_scores(hb, hq), k)
        hr = O.rac_quantize_residual(hb, hq, hsel, hn)
        O.gemm_ref(O.dequant_exact(hq.codes, hq.scales, hq.g), wdn[e],
                   O.dequant_exact(hr.codes, hr.scales, hr.g) if hn else None, hsel if hn else None)
        rows_done += b - a
    t_rows = time.perf_counter() - t0
    R = T * wl.top
    est = t_route + t_x + t_rows * R / max(rows_done, 1)
    return T / est, t_route + t_x + t_rows, (
        f"routing and quantize + RAC of X ({T}x{H}) in full ({t_route + t_x:.1f} s); gate_up + SwiGLU + "
        f"quantize/RAC of h + down for experts {sample[0]}, {sample[0] + every}, ... ({len(sample)} of {E}, "
        f"{passes} passes, {rows_done} routed rows of the layer's {R}, {t_rows:.1f} s) scaled by rows to the "
        f"full layer ({est:.1f} s estimated); combine not included")


def setup_moe(Q, S, k, decode):
    import torch
    wl = S.moe_decode(k=k) if decode else S.moe_prefill(k=k)
    T, H = wl.x.f32.shape
    E, N2, _ = wl.w_gate_up.f32.shape
    I = N2 // 2
    x = _dev(wl.x)
    logits = torch.from_numpy(wl.logits).cuda()
    guc, gus, gug = _weights_nvfp4(Q, _dev(wl.w_gate_up), 2)
    dnc, dns, dng = _weights_nvfp4(Q, _dev(wl.w_down), 1)
    R = T * wl.top
    rc = Q.RouteCall(logits, wl.top)
    ids, w, offs, rt, inv = rc()
    qx = Q.QuantizeCall(x, want_scores=True)
    q, sc = qx()
    mr = MERGED_RAC and k > 0
    sx = Q.SelectCall(x, q, sc, k, merged=mr)
    sel, res, nsel_x = sx()
    form = Q.RAC_FORM_MERGED if mr else Q.RAC_FORM_EXACT
    # Prefill: h's NVFP4 tensor scale is formed by the gate_up GEMM while it
    # writes h (y_gscale), so quantize_h runs with it given and skips its
    # amax pass over h (about 200 MB).  Decode keeps the quantizer's own amax
    # pass: on a 4 MB h the fold and zeroing launches cost more than it.
    fuse = not decode
    hq_out = Q.empty_nvfp4(1, R, I, x.device)
    g1 = Q.GemmCall(w_codes=guc, w_scales=gus, w_gscale=gug, n_seg=2, N=N2, K=H, expert_offsets=offs, num_rows=R,
                    x=q, res=res if nsel_x else None, sel_idx=sel, row_token=rt, epilogue=Q.EPI_SWIGLU,
                    x_merged=sx.merged if mr else None, rac_form=form, y_gscale=hq_out.gscale if fuse else None)
    h = g1()
    qh = Q.QuantizeCall(h, want_scores=True, out=hq_out, gscale_given=fuse)
    hq, hsc = qh()
    sh = Q.SelectCall(h, hq, hsc, k, merged=mr)
    hsel, hres, nsel_h = sh()
    g2 = Q.GemmCall(w_codes=dnc, w_scales=dns, w_gscale=dng, n_seg=1, N=H, K=I, expert_offsets=offs, num_rows=R,
                    x=hq, res=hres if nsel_h else None, sel_idx=hsel, x_merged=sh.merged if mr else None,
                    rac_form=form)
    cc = Q.CombineCall(g2.y, inv, w)
    stages = [("route", rc), ("quantize_x", qx), ("rac_x", sx), ("gate_up_prepare", g1.prepare),
              ("gate_up", g1.run), ("quantize_h", qh), ("rac_h", sh), ("down_prepare", g2.prepare),
              ("down", g2.run), ("combine", cc)]
    # Algorithmic GEMM work: the extended contraction (K + nsel).  Executed
    # MFMA work: one contraction over K on the merged operand, unless
    # --rac-form exact forces the extended contraction.
    f1 = 2.0 * R * N2 * (H + nsel_x)
    f2 = 2.0 * R * H * (I + nsel_h)
    f1x = 2.0 * R * N2 * (H + (0 if mr else nsel_x))
    # plain W4A4 layer
    qxp = Q.QuantizeCall(x)
    qp, _ = qxp()
    hqp_out = Q.empty_nvfp4(1, R, I, x.device)
    g1p = Q.GemmCall(w_codes=guc, w_scales=gus, w_gscale=gug, n_seg=2, N=N2, K=H, expert_offsets=offs, num_rows=R,
                     x=qp, row_token=rt, epilogue=Q.EPI_SWIGLU, y_gscale=hqp_out.gscale if fuse else None)
    g1p()
    qhp = Q.QuantizeCall(g1p.y, out=hqp_out, gscale_given=fuse)
    hqp, _ = qhp()
    g2p = Q.GemmCall(w_codes=dnc, w_scales=dns, w_gscale=dng, n_seg=1, N=H, K=I, expert_offsets=offs, num_rows=R,
                     x=hqp)
    ccp = Q.CombineCall(g2p.y, inv, w)
    plain = [("route", rc), ("quantize_x", qxp), ("gate_up_prepare", g1p.prepare), ("gate_up", g1p.run),
             ("quantize_h", qhp), ("down_prepare", g2p.prepare), ("down", g2p.run), ("combine", ccp)]
    cnt = np.diff(offs.cpu().numpy())
    cfg = {"workload": wl.name, "tokens": T, "hidden": H, "experts": E, "top": wl.top, "intermediate": I,
           "k_percent": k, "nsel_x": nsel_x, "nsel_h": nsel_h,
           "rac_gemm": "merged fp16 operand (executes 2*R*N*K)" if mr else "extended K (executes 2*R*N*(K+nsel))",
           "h_tensor_scale": ("quantizer's own amax pass" if decode else
                              "formed in the gate_up epilogue (y_gscale); quantize_h has no amax pass"),
           "rows_per_expert": {"min": int(cnt.min()), "max": int(cnt.max()), "mean": float(cnt.mean())}}
    wbytes = {"gate_up": E * N2 * H * 0.5625, "down": E * H * I * 0.5625}
    qxb, rxb = _act_bytes(T, H, res.cols, mr)
    qhb, rhb = _act_bytes(R, I, hres.cols, mr)
    sb = {"quantize_x": qxb, "rac_x": rxb, "quantize_h": qhb, "rac_h": rhb}
    if decode:
        # HBM-bound: the gate_up launch streams every expert's NVFP4 weights
        # once, reads its routed rows of the fp16 activation operand and
        # writes h (bf16).
        gu_bytes = wbytes["gate_up"] + R * H * (2.0 if mr else 0.5625) + R * I * 2.0
        dom = dict(bound="hbm", dominant_work=gu_bytes, dominant_exec=gu_bytes,
                   dominant_kernel="k_gemm_small<1, true> (gate_up, SwiGLU, merged RAC operand, few rows per expert)",
                   layer_floor_bytes=wbytes["gate_up"] + wbytes["down"])
    else:
        dom = dict(bound="mfma", dominant_work=f1, dominant_exec=f1x,
                   dominant_kernel=("k_gemm<Cfg<256, 256, 2, 4, 1>, 2, 1, false> (gate_up, SwiGLU, merged RAC operand)"
                                    if mr else "k_gemm<Cfg<256, 256, 2, 4, 1>, 0, 1, true> (gate_up, SwiGLU, extended K)"))
    tname = (f"k_gemm_small_gate_up_moe_decode_k{k}_traffic.txt" if decode else
             f"k_gemm_gate_up_moe_prefill_k{k}_traffic.txt")
    return dict(stages=stages, plain=plain, tokens=T, flops=f1 + f2, dominant="gate_up", config=cfg,
                traffic_summary=os.path.join(ROOT, "profiles", tname) if mr else None,
                cpu_baseline=lambda: cpu_baseline_moe(wl, k, 8 if decode else 16), weight_bytes=wbytes,
                stage_bytes=sb, plain_stage_bytes={"quantize_x": T * H * 2.5625, "quantize_h": R * I * 2.5625},
                **dom)


def setup_qdq_layer(Q, S):
    """One trainer layer's weight QDQ (128 experts x gate, up and down bf16
    masters of 2048 x 1024, 1.61 GB in and out): the bandwidth-bound step of
    the trainer-side W4A16 QAT forward."""
    E, H, I = 128, 2048, 1024
    gu_m, dn_m = S.trainer_layer_weights_device(5, 0, E, H, I)
    q1, q2 = Q.QdqCall(gu_m), Q.QdqCall(dn_m)
    elems = gu_m.numel() + dn_m.numel()

    def cpu_baseline():
        from oracle import quads_oracle as O
        mats = [gu_m[i].float().cpu().numpy() for i in (0, 1, 2, 3)] + [dn_m[i].float().cpu().numpy() for i in (0, 1)]
        n, reps, t0 = 0, 0, time.perf_counter()
        while True:
            for m in mats:
                O.weight_qdq(m)
                n += m.size
            reps += 1
            secs = time.perf_counter() - t0
            if secs >= CPU_BASELINE_MIN_S / 2:
                break
        return n * 4.0 / secs / 1e9, secs, (f"oracle weight QDQ of 4 gate/up and 2 down master matrices of layer 0 "
                                            f"x {reps} repetitions, as GB/s of bf16 in + out")

    return dict(stages=[("qdq_gate_up", q1), ("qdq_down", q2)], bytes=4.0 * elems, elems=elems,
                cpu_baseline=cpu_baseline, keep=(gu_m, dn_m))


def setup_trainer(Q, S, layers, qdq="separate"):
    """Trainer-side W4A16 QAT forward: per layer, NVFP4 QDQ of the bf16 master
    weights of 128 experts x (gate, up, down) into one reused bf16 buffer,
    then the bf16 grouped forward of 8192 tokens (top-8 routing computed once
    per step; every layer sees the same synthetic input, so no cast kernel
    sits between layers).  qdq="in_gemm": the QDQ happens inside the GEMMs
    (QUADS_OPERANDS_BF16_QDQ), per layer only the masters' tensor scales are
    computed first (QUADS_SCALES_ONLY); qdq="codes": per layer the masters
    are quantized to NVFP4 and the GEMMs decode the codes to their QDQ values
    (QUADS_OPERANDS_BF16_W4).  Either way W_qdq is never written."""
    import torch
    T, H, E, I, top = 8192, 2048, 128, 1024, 8
    rng = np.random.default_rng(5)
    x = _dev(S.activation(rng, T, H, 0, 1.0, bf16=True))
    logits = torch.from_numpy(S.gaussian_logits(rng, T, E)).cuda()
    masters = [S.trainer_layer_weights_device(5, l, E, H, I) for l in range(layers)]
    rc = Q.RouteCall(logits, top)
    ids, w, offs, rt, inv = rc()
    R = T * top
    stages = [("route", rc)]
    if qdq == "codes":
        qgu = Q.empty_nvfp4(2 * E, I, H, "cuda")
        qdn = Q.empty_nvfp4(E, H, I, "cuda")
        h = torch.empty(R, I, dtype=torch.bfloat16, device="cuda")
        y = torch.empty(R, H, dtype=torch.float32, device="cuda")
        gu = Q.GemmCall(N=2 * I, K=H, expert_offsets=offs, num_rows=R, row_token=rt, x_bf16=x,
                        w_codes=qgu.codes.view(E, 2 * I, H // 2), w_scales=qgu.scales.view(E, 2 * I, H // 16),
                        w_gscale=qgu.gscale, n_seg=2, epilogue=Q.EPI_SWIGLU, y=h)
        dn = Q.GemmCall(N=H, K=I, expert_offsets=offs, num_rows=R, x_bf16=h, w_codes=qdn.codes,
                        w_scales=qdn.scales, w_gscale=qdn.gscale, y=y)
        cc = Q.CombineCall(y, inv, w)
        for l in range(layers):
            stages += [(f"L{l}.quantize_gate_up", Q.QuantizeCall(masters[l][0], out=qgu)),
                       (f"L{l}.quantize_down", Q.QuantizeCall(masters[l][1], out=qdn)),
                       (f"L{l}.gate_up_prepare", gu.prepare), (f"L{l}.gate_up", gu.run),
                       (f"L{l}.down_prepare", dn.prepare), (f"L{l}.down", dn.run), (f"L{l}.combine", cc)]
        kern = "k_gemm_pp<bf16 x NVFP4 weights decoded to QDQ values, SWIGLU> (gate_up)"
    elif qdq == "in_gemm":
        g_gu = torch.empty(2 * E, dtype=torch.float32, device="cuda")
        g_dn = torch.empty(E, dtype=torch.float32, device="cuda")
        h = torch.empty(R, I, dtype=torch.bfloat16, device="cuda")
        y = torch.empty(R, H, dtype=torch.float32, device="cuda")
        for l in range(layers):
            gu = Q.GemmCall(N=2 * I, K=H, expert_offsets=offs, num_rows=R, row_token=rt, x_bf16=x,
                            w_bf16=masters[l][0].view(E, 2 * I, H), w_gscale=g_gu, n_seg=2, qdq=True,
                            epilogue=Q.EPI_SWIGLU, y=h)
            dn = Q.GemmCall(N=H, K=I, expert_offsets=offs, num_rows=R, x_bf16=h, w_bf16=masters[l][1],
                            w_gscale=g_dn, qdq=True, y=y)
            cc = Q.CombineCall(y, inv, w)
            stages += [(f"L{l}.scales_gate_up", Q.ScalesCall(masters[l][0], g_gu)),
                       (f"L{l}.scales_down", Q.ScalesCall(masters[l][1], g_dn)),
                       (f"L{l}.gate_up_prepare", gu.prepare), (f"L{l}.gate_up", gu.run),
                       (f"L{l}.down_prepare", dn.prepare), (f"L{l}.down", dn.run), (f"L{l}.combine", cc)]
        kern = "k_gemm_pp<QDQ-fused bf16 masters, SWIGLU> (gate_up)"
    else:
        wq_gu = torch.empty_like(masters[0][0])  # [2E, I, H]: matrix 2e = gate of expert e, 2e+1 = up
        wq_dn = torch.empty_like(masters[0][1])  # [E, H, I]
        gu = Q.GemmCall(N=2 * I, K=H, expert_offsets=offs, num_rows=R, row_token=rt, x_bf16=x,
                        w_bf16=wq_gu.view(E, 2 * I, H), epilogue=Q.EPI_SWIGLU)
        dn = Q.GemmCall(N=H, K=I, expert_offsets=offs, num_rows=R, x_bf16=gu.y, w_bf16=wq_dn)
        cc = Q.CombineCall(dn.y, inv, w)
        for l in range(layers):
            stages += [(f"L{l}.qdq_gate_up", Q.QdqCall(masters[l][0], out=wq_gu)),
                       (f"L{l}.qdq_down", Q.QdqCall(masters[l][1], out=wq_dn)),
                       (f"L{l}.gate_up_prepare", gu.prepare), (f"L{l}.gate_up", gu.run),
                       (f"L{l}.down_prepare", dn.prepare), (f"L{l}.down", dn.run), (f"L{l}.combine", cc)]
        kern = "k_gemm_pp<bf16 operands, SWIGLU> (gate_up)"
    flops_layer = 2.0 * R * (2 * I) * H + 2.0 * R * H * I
    qdq_bytes_layer = 4.0 * (masters[0][0].numel() + masters[0][1].numel())  # bf16 in + bf16 out
    cfg = {"workload": "trainer_qdq", "tokens": T, "hidden": H, "experts": E, "top": top, "intermediate": I,
           "layers": layers, "master_weights_bytes": 2 * layers * (masters[0][0].numel() + masters[0][1].numel()),
           "qdq": {"in_gemm": "fused into the GEMMs (scales-only pass + QUADS_OPERANDS_BF16_QDQ)",
                   "codes": "masters quantized to NVFP4, decoded to QDQ values in the GEMMs (QUADS_OPERANDS_BF16_W4)",
                   "separate": "separate quads_weight_qdq into a bf16 buffer"}[qdq],
           "note": "QDQ of every layer's masters + bf16 grouped forward; same synthetic input for every layer"}
    return dict(stages=stages, plain=None, tokens=T, flops=flops_layer * layers, dominant=None,
                dominant_stage_for_roofline="L0.gate_up", bound="mfma", dominant_work=2.0 * R * (2 * I) * H,
                dominant_exec=2.0 * R * (2 * I) * H, dominant_kernel=kern, config=cfg, cpu_baseline=None,
                qdq_bytes_layer=qdq_bytes_layer if qdq == "separate" else None,
                layer0_stages=[st for st in stages if st[0].startswith(("route", "L0."))])


def setup_trainer_bwd(Q, S):
    """Backward of one trainer layer's two grouped projections (W4A16 QAT,
    straight-through QDQ), with seeded synthetic upstream gradients."""
    import torch
    T, H, E, I, top = 8192, 2048, 128, 1024, 8
    rng = np.random.default_rng(6)
    x = _dev(S.activation(rng, T, H, 0, 1.0, bf16=True))
    logits = torch.from_numpy(S.gaussian_logits(rng, T, E)).cuda()
    gu_m, dn_m = S.trainer_layer_weights_device(6, 0, E, H, I)
    wq_gu, _ = Q.QdqCall(gu_m)()
    wq_dn, _ = Q.QdqCall(dn_m)()
    _, _, offs, rt, inv = Q.moe_route(logits, top)
    R = T * top
    gen = torch.Generator(device="cuda")
    gen.manual_seed(6)
    dy_gu = torch.randn((R, 2 * I), generator=gen, device="cuda").to(torch.bfloat16)
    dy_dn = torch.randn((R, H), generator=gen, device="cuda").to(torch.bfloat16)
    h = torch.randn((R, I), generator=gen, device="cuda").to(torch.bfloat16)
    bgu = Q.QatBackward(wq_gu.view(E, 2 * I, H), dy_gu, x, offs, rt, inv)
    bdn = Q.QatBackward(wq_dn, dy_dn, h, offs)
    stages = [(f"gate_up.{n}", f) for n, f in bgu.stages()] + [(f"down.{n}", f) for n, f in bdn.stages()]
    flops = 2.0 * 2.0 * R * (2 * I) * H + 2.0 * 2.0 * R * H * I  # dX and dW of both projections
    cfg = {"workload": "trainer_bwd", "tokens": T, "hidden": H, "experts": E, "top": top, "intermediate": I,
           "note": "W4A16 QAT backward of gate_up and down (straight-through QDQ): dX and FP32 dW; synthetic dY"}

    def cpu_baseline():
        """The oracle's backward (QDQ of the expert's masters, dX, dW in
        float64) of gate_up for whole experts, repeated until
        CPU_BASELINE_MIN_S; converted to tokens/s of the full step by flops."""
        from oracle import quads_oracle as O
        ho, hrt = offs.cpu().numpy(), rt.cpu().numpy()
        xs = x.float().cpu().numpy()
        reps, fl, t0 = 0, 0.0, time.perf_counter()
        while True:
            e = reps % E
            a, b = int(ho[e]), int(ho[e + 1])
            w = gu_m[2 * e:2 * e + 2].float().cpu().numpy().reshape(1, 2 * I, H)
            O.qat_linear_backward(xs, w, dy_gu[a:b].float().cpu().numpy(), hrt[a:b], np.array([0, b - a]))
            fl += 2.0 * 2.0 * (b - a) * (2 * I) * H
            reps += 1
            secs = time.perf_counter() - t0
            if secs >= CPU_BASELINE_MIN_S:
                break
        return T * (fl / flops) / secs, secs, (f"oracle gate_up backward of {reps} whole experts (weight QDQ, dX, dW "
                                               "in float64), scaled to the full step by flops")

    return dict(stages=stages, plain=None, tokens=T, flops=flops, dominant="gate_up.wgrad",
                bound="mfma", dominant_work=2.0 * R * (2 * I) * H, dominant_exec=2.0 * R * (2 * I) * H,
                dominant_kernel="gate_up dW: k_pad_map + 2 gather-transposes + k_wgrad (bf16 MFMA, FP32 dW)",
                config=cfg, cpu_baseline=cpu_baseline,
                cpu_cores_note="float64 products on the BLAS threads; the weight QDQ single-threaded NumPy")


def run_ablation(Q, S):
    """The ablation report (one JSON line): errors vs float64 and
    trainer/rollout mismatches for two seeded layers."""
    import torch
    from fp4_quantized_moe_amd import ablation as A
    rng = np.random.default_rng(7)
    layers = {}
    wl = S.expert_gemm()
    dense = (_dev(wl.x), _dev(wl.w)[None], [0, wl.x.f32.shape[0]], S.drifted(rng, wl.x))
    dec = S.moe_decode()
    _, _, offs, _, _ = Q.moe_route(torch.from_numpy(dec.logits).cuda(), dec.top)
    offs = [int(v) for v in offs.cpu().numpy()]
    R, I = offs[-1], dec.w_down.f32.shape[2]
    h = S.activation(rng, R, I, I // 100, 30.0, bf16=True)
    down = (_dev(h), _dev(dec.w_down), offs, S.drifted(rng, h))
    pairs = [("w4a4", "w4a16"), ("rac25", "w4a16"), ("rac50", "w4a16"), ("rac100", "w4a16"),
             ("rac50_pe", "w4a16"), ("w4a4", "w4a4_sym"), ("rac50", "w4a4_sym")]
    for name, (x, w, o, xd) in (("expert_gemm", dense), ("decode_down", down)):
        out = A.grouped_linear_variants(x, w, o)
        err = A.errors(out, A.reference_fp64(x, w, o))
        drift = A.grouped_linear_variants(x, w, o, x_rollout=_dev(xd))
        layers[name] = {"rows": o[-1], "experts": len(o) - 1, "N": w.shape[1], "K": w.shape[2],
                        "error_vs_fp64": err, "mismatch": A.mismatch(out, pairs),
                        "mismatch_with_drift": A.mismatch(drift, pairs)}
    print(json.dumps({
        "metric": "QUADS ablation: relative output error vs the float64 master product (RAC k=50%, decode-shaped down projection)",
        "value": layers["decode_down"]["error_vs_fp64"]["rac50"]["rel_fro"], "unit": "relative Frobenius error",
        "higher_is_better": False, "n_gpus": 1, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "ablation", "drift": "rollout activation = bf16(x * (1 + e)), e ~ N(0, 2^-9)",
                   "down_input": "bf16 N(0,1) rows with 1% outlier channels x30 over the decode routing"},
        "layers": layers}), flush=True)


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def capture(fns, reps=1):
    """One HIP graph holding `reps` passes over fns (every library call enqueues
    on torch's current stream, which is the capture stream here)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            for fn in fns:
                fn()
    return g


EVENT_EVERY = 10  # timed steps per step whose dominant stage is bracketed by HIP events


def run_steps(stages, steps, warmup, dominant=None, graph=False):
    """Run `warmup` untimed steps, then `steps` timed steps bracketed by device
    synchronisation.  Every library call only enqueues work, so the host runs
    ahead of the device and the kernels of consecutive steps execute back to
    back.  HIP events recorded on the stream every call uses, around the
    dominant stage of every EVENT_EVERY-th timed step (at least one), give
    that kernel's duration inside the timed region: each timing event is a
    barrier packet that stops the kernels around it from overlapping their
    launch, about 13 us per event pair on the expert-GEMM step, so recording
    them in every step would time the instrumentation too.  With graph=True
    the stages before and after the dominant one are replayed as HIP graphs
    instead (on this stack no faster than direct launches).
    Returns (wall seconds, event ms over all steps, dominant-stage ms per step)."""
    import torch
    for _, fn in stages:  # eager pass: lazy allocations happen outside any capture
        fn()
    torch.cuda.synchronize()
    names = [n for n, _ in stages]
    i = names.index(dominant) if dominant in names else len(names)
    pre, dom, post = stages[:i], stages[i:i + 1], stages[i + 1:]
    if graph:
        g_pre = capture([fn for _, fn in pre]) if pre else None
        g_post = capture([fn for _, fn in post]) if post else None
        run_pre = [g_pre.replay] if g_pre else []
        run_post = [g_post.replay] if g_post else []
    else:
        run_pre = [fn for _, fn in pre]
        run_post = [fn for _, fn in post]

    def step(ev=None):
        for fn in run_pre:
            fn()
        if ev:
            ev[0].record()
        for _, fn in dom:
            fn()
        if ev:
            ev[1].record()
        for fn in run_post:
            fn()

    for _ in range(warmup):
        step()
    every = max(1, min(EVENT_EVERY, steps))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if s % every == 0 else None
           for s in range(steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for s in range(steps):
        step(evs[s])
    e1.record()
    torch.cuda.synchronize()
    secs = time.perf_counter() - t0
    dom_ms = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in evs if ev is not None])) if dom else None
    return secs, e0.elapsed_time(e1), dom_ms


def stage_times(stages, reps=20, iters=3):
    """Mean device time of each stage per call: a graph of `reps` back-to-back
    calls of that stage alone, replayed `iters` times between HIP events on the
    stream the graph runs on.  Stages are pure functions of buffers set up
    beforehand, so repeating one in isolation recomputes the same outputs."""
    import torch
    out = {}
    for name, fn in stages:
        g = capture([fn], reps)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) / (reps * iters)
    return out


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def cold_stage_times(stages, names, reps=10):
    """Device time of one call of each named stage with the Infinity Cache
    flushed first: a 1 GiB buffer is overwritten, then HIP events on the
    stream the call uses bracket that one call (the events include the
    launch gap of about 1-2 us).  Returns {name: mean ms}."""
    import torch
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    fns = dict(stages)
    out = {}
    for name in names:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            flush.zero_()
            a.record()
            fns[name]()
            b.record()
        torch.cuda.synchronize()
        out[name] = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    del flush
    return out


def _bw(stage_bytes, warm, cold):
    """{stage: {bytes, GB/s warm and cold, fraction of HBM peak (cold)}}."""
    out = {}
    for name, nb in stage_bytes.items():
        gw = nb / (warm[name] * 1e-3) / 1e9
        gc = nb / (cold[name] * 1e-3) / 1e9
        out[name] = {"algorithmic_bytes": nb, "ms_warm": warm[name], "ms_cold": cold[name], "GBps_warm": gw,
                     "GBps_cold": gc, "frac_hbm_cold": gc / PEAK_HBM_GBS}
    return out


def _roofline(wl, dom_ms, traffic=None, tinfo=None):
    work, ex = wl["dominant_work"], wl["dominant_exec"]
    if wl["bound"] == "hbm":
        ach = work / (dom_ms * 1e-3) / 1e9
        r = {"bound": "hbm", "kernel": wl["dominant_kernel"], "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": ach / PEAK_HBM_GBS, "traffic": traffic, "bytes_per_launch": work, "avg_launch_ms": dom_ms}
    else:
        ach = work / (dom_ms * 1e-3) / 1e12
        exe = ex / (dom_ms * 1e-3) / 1e12
        r = {"bound": "mfma", "kernel": wl["dominant_kernel"], "achieved": ach, "peak": PEAK_F16_TFLOPS,
             "unit": "TFLOP/s", "frac": ach / PEAK_F16_TFLOPS, "traffic": traffic,
             "flops_per_launch": work, "avg_launch_ms": dom_ms,
             "work_note": "achieved counts the algorithmic RAC GEMM work 2*rows*N*(K+nsel); executed counts the MFMA "
                          "work the kernel issues",
             "executed": {"flops_per_launch": ex, "achieved": exe, "frac": exe / PEAK_F16_TFLOPS}}
    if tinfo is not None:
        r["traffic_note"] = tinfo
    return r


def _traffic(wl):
    """(HBM bytes per launch of the dominant kernel, note) from its committed
    rocprofv3 traffic summary, or (None, reason)."""
    from fp4_quantized_moe_amd.profiling import read_traffic
    if not wl.get("traffic_summary"):
        return None, "no traffic summary for this workload"
    traffic, tinfo = read_traffic(wl["traffic_summary"])
    if traffic is not None:
        tinfo = (f"HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE scaled by a plain copy), "
                 f"{os.path.relpath(wl['traffic_summary'], ROOT)}")
    return traffic, tinfo


def _cpu(wl, note_default):
    rate, cpu_s, sample = wl["cpu_baseline"]()
    return {"value": rate, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle", "sample": sample,
            "seconds": cpu_s, "host_cpus": os.cpu_count(), "cores_note": wl.get("cpu_cores_note", note_default)}


CPU_NOTE = "fp64 GEMM on the BLAS threads; quantize and RAC single-threaded NumPy"


def measure_layer(wl, args):
    """One MoE layer block: step time, tokens/s, plain W4A4 step and RAC
    overhead, roofline of gate_up, per-stage times and bandwidths, oracle."""
    import torch
    secs, _, dom_ms = run_steps(wl["stages"], args.steps, args.warmup, wl["dominant"], args.graph)
    ms = secs * 1e3 / args.steps
    warm = stage_times(wl["stages"])
    cold = cold_stage_times(wl["stages"], list(wl["stage_bytes"]))
    traffic, tinfo = _traffic(wl)
    blk = {"config": wl["config"], "ms_per_step": ms, "tokens_per_s": wl["tokens"] * args.steps / secs,
           "tflops_step_algorithmic": wl["flops"] / (ms * 1e-3) / 1e12, "stages_ms": warm,
           "stage_bandwidth": _bw(wl["stage_bytes"], warm, cold), "roofline": _roofline(wl, dom_ms, traffic, tinfo)}
    if wl.get("layer_floor_bytes"):
        fl = wl["layer_floor_bytes"] / (PEAK_HBM_GBS * 1e9) * 1e3
        blk["hbm_floor"] = {"weight_bytes": wl["layer_floor_bytes"], "floor_ms": fl, "frac_of_step": fl / ms}
    if not args.no_plain and wl.get("plain"):
        psecs, _, _ = run_steps(wl["plain"], args.steps, args.warmup, None, args.graph)
        blk["plain_w4a4_ms_per_step"] = psecs * 1e3 / args.steps
        blk["plain_stages_ms"] = stage_times(wl["plain"])
        blk["rac_overhead_pct"] = 100.0 * (secs / psecs - 1.0)
    torch.cuda.synchronize()
    if not args.no_cpu_baseline and wl.get("cpu_baseline") is not None:
        blk["cpu_baseline"] = _cpu(wl, CPU_NOTE)
    return blk


def measure_trainer_layer(Q, S, args):
    """One trainer layer's W4A16 forward (8192 tokens, 128 experts, top-8),
    with the weight QDQ as a separate pass and in both fused forms."""
    out = {}
    for name, mode in (("separate_qdq", "separate"), ("qdq_in_gemm", "in_gemm"), ("nvfp4_decode_in_gemm", "codes")):
        wl = setup_trainer(Q, S, 1, mode)
        secs, _, _ = run_steps(wl["stages"], args.steps, args.warmup)
        per = stage_times(wl["stages"])
        out[name] = {"ms_per_layer": secs * 1e3 / args.steps, "stages_ms": per,
                     "tflops_layer": wl["flops"] / (secs / args.steps) / 1e12}
        del wl
    for name in ("qdq_in_gemm", "nvfp4_decode_in_gemm"):
        out[name]["speedup_vs_separate"] = out["separate_qdq"]["ms_per_layer"] / out[name]["ms_per_layer"]
    return out


def measure_qdq(Q, S, args):
    ql = setup_qdq_layer(Q, S)
    warm = stage_times(ql["stages"])
    cold = cold_stage_times(ql["stages"], [n for n, _ in ql["stages"]])
    ms_w, ms_c = sum(warm.values()), sum(cold.values())
    traffic, tinfo = _traffic({"traffic_summary": os.path.join(ROOT, "profiles", "k_quantize_qdq_trainer_traffic.txt")})
    blk = {"config": {"workload": "trainer_qdq_layer", "matrices": "128 experts x (gate, up, down) of 2048x1024 bf16",
                      "elements": ql["elems"]},
           "algorithmic_bytes": ql["bytes"], "ms_warm": ms_w, "ms_cold": ms_c,
           "roofline": {"bound": "hbm", "kernel": "k_quantize<bf16, QDQ> (quads_weight_qdq)",
                        "achieved": ql["bytes"] / (ms_c * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": ql["bytes"] / (ms_c * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": traffic,
                        "traffic_note": (tinfo if traffic is None else
                                         tinfo + "; the launch time here also holds the amax pass over the masters"),
                        "bytes_per_launch": ql["bytes"] / 2, "avg_launch_ms": ms_c / 2},
           "GBps_warm": ql["bytes"] / (ms_w * 1e-3) / 1e9}
    if not args.no_cpu_baseline:
        rate, cpu_s, sample = ql["cpu_baseline"]()
        blk["cpu_baseline"] = {"value": rate, "unit": "GB/s", "cores": 1, "kind": "oracle", "sample": sample,
                               "seconds": cpu_s, "host_cpus": os.cpu_count()}
    return blk


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        sys.stderr.write("bench.py measures one GPU only: this build runs the hot path on a single MI355X "
                         "(no multi-GPU path); run it with --gpus 1.\n")
        sys.exit(2)
    import torch
    from fp4_quantized_moe_amd import _lib as Q
    from fp4_quantized_moe_amd import synthetic as S

    global MERGED_RAC
    MERGED_RAC = args.rac_form == "merged"
    torch.cuda.set_device(0)
    Q.load()
    if args.workload == "ablation":
        run_ablation(Q, S)
        return
    if args.workload == "expert_gemm":
        wl = setup_expert_gemm(Q, S, args.k)
    elif args.workload == "trainer_bwd":
        wl = setup_trainer_bwd(Q, S)
    elif args.workload in ("moe_prefill", "moe_decode"):
        wl = setup_moe(Q, S, args.k, args.workload == "moe_decode")
    else:
        wl = setup_trainer(Q, S, args.layers, args.qdq)
    torch.cuda.synchronize()

    secs, ev_ms, dom_ms = run_steps(wl["stages"], args.steps, args.warmup, wl["dominant"], args.graph)
    per = stage_times(wl.get("layer0_stages", wl["stages"]))
    if dom_ms is None:  # no directly launched dominant stage: its graph-of-20 time
        dom_ms = per[wl["dominant_stage_for_roofline"]]
    ms = secs * 1e3 / args.steps
    tokens_per_s = wl["tokens"] * args.steps / secs
    traffic, tinfo = _traffic(wl)
    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_events": ev_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": wl["config"],
        "tflops_step_algorithmic": wl["flops"] / (ms * 1e-3) / 1e12,
        "stages_ms": per,
        "timing": ("stages launched directly (host runs ahead of the device)" if not args.graph else
                   "stages before/after the dominant one replayed as HIP graphs") +
                  f"; roofline.avg_launch_ms from HIP events around the dominant kernel in every {EVENT_EVERY}th "
                  "timed step (each event pair is a barrier packet that costs the step about 13 us); "
                  "stages_ms from graphs of 20 back-to-back calls of one stage; stage_bandwidth cold from one call "
                  "after a 1 GiB write that evicts the Infinity Cache",
        "roofline": _roofline(wl, dom_ms, traffic, tinfo),
    }
    if wl.get("stage_bytes"):
        cold = cold_stage_times(wl["stages"], list(wl["stage_bytes"]))
        out["stage_bandwidth"] = _bw(wl["stage_bytes"], per, cold)
    if wl.get("qdq_bytes_layer"):
        qdq_ms = per["L0.qdq_gate_up"] + per["L0.qdq_down"]
        out["qdq"] = {"bytes_per_layer": wl["qdq_bytes_layer"], "ms_per_layer": qdq_ms,
                      "achieved_GBps": wl["qdq_bytes_layer"] / (qdq_ms * 1e-3) / 1e9, "peak_GBps": PEAK_HBM_GBS}
    if not args.no_plain and wl.get("plain"):
        psecs, _, _ = run_steps(wl["plain"], args.steps, args.warmup, None, args.graph)
        out["plain_w4a4_ms_per_step"] = psecs * 1e3 / args.steps
        out["plain_stages_ms"] = stage_times(wl["plain"])
        out["rac_overhead_pct"] = 100.0 * (secs / psecs - 1.0)
    if not args.no_cpu_baseline and wl.get("cpu_baseline") is not None:
        out["cpu_baseline"] = _cpu(wl, CPU_NOTE)
    if args.workload == "expert_gemm" and not args.no_moe:
        del wl
        torch.cuda.empty_cache()
        out["workloads"] = {}
        for name, decode in (("moe_prefill", False), ("moe_decode", True)):
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            lw = setup_moe(Q, S, args.k, decode)
            torch.cuda.synchronize()
            out["workloads"][name] = measure_layer(lw, args)
            del lw
            torch.cuda.empty_cache()
        print("[bench] trainer_qdq_layer", file=sys.stderr, flush=True)
        out["workloads"]["trainer_qdq_layer"] = measure_qdq(Q, S, args)
        torch.cuda.empty_cache()
        print("[bench] trainer_forward_layer", file=sys.stderr, flush=True)
        out["workloads"]["trainer_forward_layer"] = measure_trainer_layer(Q, S, args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
