"""Ablation variants of one grouped linear layer, computed with the library's
kernels through the C ABI.

The QUADS technical summary's ablations (section 4) set the asymmetric W4A16
trainer (section 2.2-A) against symmetric W4A4 QAT, which fake-quantizes the
trainer's activations too (section 2.1). They also run the rollout without
the residual compensation of section 2.2-B. One RAC mask per expert is added
here as the alternative to one mask per input tensor. For
Y[i] = W[e(i)] . x[i] over rows grouped by expert, the variants are:

  bf16       trainer without QAT: bf16 masters and activations (bf16 MFMA)
  w4a16      asymmetric QAT trainer: NVFP4 QDQ of each weight matrix,
             activations kept in bf16
  w4a4_sym   symmetric QAT trainer: QDQ of the weights and of the activation
             tensor (one tensor scale)
  w4a4       rollout: NVFP4 W4A4 without compensation
  rac{k}     rollout: W4A4 + RAC at k% with one channel mask for the tensor
  rac{k}_pe  rollout: W4A4 + RAC at k% with one mask per expert, scored over
             that expert's rows

The rollout variants use the codes, scales and tensor scales that the
trainer's weight QDQ exports, which is the shared weight path of section 2.1.
A rollout activation different from the trainer's models engine drift between
the two sides. `errors()` measures each variant against the float64 product
of the bf16 masters and activations.

The per-expert variant runs one quantize, select and GEMM call per expert.
It is an ablation path, not a fused kernel.
"""
from __future__ import annotations

import torch

from . import _lib as Q


def _gemm_bf16(x, w, offs, R):
    E, N, K = w.shape
    return Q.moe_w4a4_gemm(N=N, K=K, expert_offsets=offs, num_rows=R, x_bf16=x, w_bf16=w)


def per_expert_rac(x, q, wq, offsets, k_percent, y=None):
    """W4A4 + RAC with one channel mask per expert.

    x: bf16 [R, K] rows grouped by expert; q: its NVFP4 quantization (the
    tensor scale is reused for every expert); wq: exported NVFP4 weights
    [E, N, K]; offsets: host list of E+1 row offsets.  Returns
    (y fp32 [R, N], [(sel_idx, residual, nsel) or None per expert])."""
    E = len(offsets) - 1
    N, K = wq.rows, wq.cols
    R = x.shape[0]
    if y is None:
        y = torch.empty(R, N, dtype=torch.float32, device=x.device)
    parts = []
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            parts.append(None)
            continue
        xe = x[a:b]
        qe, se = Q.quantize_nvfp4(xe, want_scores=True, gscale=q.gscale)
        sel, res, nsel = Q.rac_select(xe, qe, se, k_percent)
        offs_e = torch.tensor([0, b - a], dtype=torch.int32, device=x.device)
        Q.moe_w4a4_gemm(w_codes=wq.codes[e:e + 1], w_scales=wq.scales[e:e + 1], w_gscale=wq.gscale[e:e + 1],
                        N=N, K=K, expert_offsets=offs_e, num_rows=b - a, x=qe, res=res if nsel else None,
                        sel_idx=sel, y=y[a:b])
        parts.append((sel, res, nsel))
    return y, parts


def grouped_linear_variants(x, w, offsets, k_list=(25, 50, 100), per_expert_k=(50,), x_rollout=None):
    """Every variant of the module docstring for one grouped linear layer.

    x: bf16 [R, K] trainer activation, rows grouped by expert; w: bf16
    [E, N, K] master weights; offsets: host list of E+1 row offsets;
    x_rollout: the rollout side's activation (default x).  Returns a dict
    name -> fp32 [R, N] device tensor."""
    E, N, K = w.shape
    R = x.shape[0]
    if len(offsets) != E + 1 or int(offsets[-1]) != R:
        raise Q.QuadsError("offsets must hold E+1 row offsets ending at the row count")
    offs = torch.tensor([int(v) for v in offsets], dtype=torch.int32, device=x.device)
    out = {}
    out["bf16"] = _gemm_bf16(x, w, offs, R)
    w_qdq, wq = Q.weight_qdq(w, export=True)
    out["w4a16"] = _gemm_bf16(x, w_qdq, offs, R)
    x_qdq, _ = Q.weight_qdq(x)
    out["w4a4_sym"] = _gemm_bf16(x_qdq, w_qdq, offs, R)

    xr = x if x_rollout is None else x_rollout
    q, scores = Q.quantize_nvfp4(xr, want_scores=True)

    def w4a4(res=None, sel=None):
        return Q.moe_w4a4_gemm(w_codes=wq.codes, w_scales=wq.scales, w_gscale=wq.gscale, N=N, K=K,
                               expert_offsets=offs, num_rows=R, x=q, res=res, sel_idx=sel)

    out["w4a4"] = w4a4()
    for k in k_list:
        sel, res, nsel = Q.rac_select(xr, q, scores, k)
        out[f"rac{k}"] = w4a4(res if nsel else None, sel)
    for k in per_expert_k:
        out[f"rac{k}_pe"] = per_expert_rac(xr, q, wq, offsets, k)[0]
    return out


def reference_fp64(x, w, offsets):
    """Float64 product of the bf16 masters and the trainer's activation, per
    expert: the unquantized layer that every variant approximates."""
    E, N, _ = w.shape
    y = torch.zeros(x.shape[0], N, dtype=torch.float64, device=x.device)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a < b:
            y[a:b] = x[a:b].double() @ w[e].double().T
    return y


def errors(out, y_ref):
    """name -> {"rel_fro": |Y - Y_ref|_F / |Y_ref|_F, "rel_max": max|Y - Y_ref| / max|Y_ref|}."""
    nf = float(torch.linalg.norm(y_ref))
    nm = float(y_ref.abs().max())
    res = {}
    for name, y in out.items():
        d = y.double() - y_ref
        res[name] = {"rel_fro": float(torch.linalg.norm(d)) / nf, "rel_max": float(d.abs().max()) / nm}
    return res


def mismatch(out, pairs):
    """Trainer/rollout output distance: (rollout, trainer) -> |Y_r - Y_t|_F / |Y_t|_F."""
    res = {}
    for r, t in pairs:
        yt = out[t].double()
        res[f"{r}|{t}"] = float(torch.linalg.norm(out[r].double() - yt)) / float(torch.linalg.norm(yt))
    return res
