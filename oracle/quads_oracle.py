"""Plain CPU oracle for the QUADS rollout/trainer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no common helpers, tables or constants) and imports nothing from the
``fp4_quantized_moe_amd`` package.

Sources (the method is described on three web pages about one paper, "QUADS:
Stabilizing NVFP4 Reinforcement Learning for MoE via QUantization-error
Alignment across Dual Sides"):

* [Gist]   gist.science technical summary "Technische Samenvatting: QUADS",
           sections 1 (Probleemstelling), 2.1 (Foutanalyse en Diagnose),
           2.2-A (Asymmetrische QAT) and 2.2-B (Residual Activation
           Compensatie).
* [Wiki]   AI-Wiki summary of the paper, sections "Key Contributions" and
           "Methodology".
* [Explained] ArxivLens "Paper Explained" page, "Detailed Explanation".

The pages fix the method (NVFP4 activations recomputed online; E2M1's coarse
grid of 8 magnitudes per sign; residual ΔX of the activation quantization; a
binary top-k% channel mask on the residual magnitude; a second-pass
quantization of the masked residual channels added to the quantized path; a
shared weight quantize-dequantize path for the trainer).  They do not fix
the NVFP4 encoding details.  This library specifies them as follows, and the
oracle implements exactly that specification:

* blocks of 16 consecutive elements along the contraction (column) axis, one
  OCP FP8 E4M3 ("fn" variant: no infinities, max 448) scale per block, one
  FP32 scale per tensor;
* element format OCP E2M1 (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6);
* round-to-nearest, ties-to-even everywhere, with saturation at the format
  maximum;
* two E2M1 codes per byte, element 2j in the low nibble.

Where the specification leaves a step open the oracle takes the readings
listed in the repository's design notes (per-tensor scale
g = fl32(amax/2688), g = 1 for an all-zero tensor; block scale
s = E4M3(fl32(fl32(amax_b/6)/g)); v = fl32(|x|/fl32(dec(s)·g)); the sign bit is
always kept; channel score = max over rows of |ΔX|, ties to the lower channel
index; nsel = floor(K·k/100) selected channels, padded to a multiple of 16
with zero residual entries; selected channels gathered in ascending order).

Floating point: every step the method performs in FP32 is done here with
NumPy float32 element-wise operations (IEEE round-to-nearest-even, no FMA
contraction); the GEMM reference accumulates the exactly dequantized operands
in float64.

All functions are pinned by ``tests/test_oracle_*.py`` against format
definitions, closed forms, invariants and brute force; nothing in this file
is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Element and scale formats
# ---------------------------------------------------------------------------

#: E2M1 magnitudes indexed by the 3 low bits of a code (sign is bit 3).
#: [Gist §1] gives the count: eight levels per sign.  Values: OCP MX E2M1.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0
E4M3_MAX_CODE = 0x7E


def e2m1_decode(code):
    """Value of E2M1 code(s) (4-bit, sign in bit 3) as float64."""
    code = np.asarray(code, dtype=np.int64)
    mag = E2M1_MAGNITUDES[code & 7]
    return np.where((code & 8) != 0, -mag, mag)


def e2m1_round_magnitude(v):
    """Index (0..7) of the E2M1 magnitude nearest to v >= 0.

    Ties go to the even index (round-half-to-even on the E2M1 mantissa);
    values beyond 6 saturate to index 7 (the nearest level is 6).
    Implemented literally as "nearest level, even index on a tie".
    """
    v = np.asarray(v, dtype=np.float64)
    flat = v.reshape(-1)
    out = np.empty(flat.shape, dtype=np.int64)
    step = 1 << 20
    for lo in range(0, flat.size, step):
        vv = np.minimum(flat[lo:lo + step], 8.0)  # anything above 6 is nearest to 6
        dist = np.abs(vv[:, None] - E2M1_MAGNITUDES[None, :])  # exact in f64
        best = np.argmin(dist, axis=1)  # first (lowest) index of the minimum
        nxt = np.minimum(best + 1, 7)
        tie = (nxt != best) & (dist[np.arange(vv.size), nxt] == dist[np.arange(vv.size), best])
        # on a tie the candidates are best (lower) and best+1: take the even one
        best = np.where(tie & (best % 2 == 1), nxt, best)
        out[lo:lo + step] = best
    return out.reshape(v.shape)


def _e4m3_table():
    """Values of the 127 non-negative finite E4M3 codes 0x00..0x7E (float64)."""
    vals = np.empty(127, dtype=np.float64)
    for c in range(127):
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 0:
            vals[c] = (m / 8.0) * 2.0 ** (-6)  # subnormal
        else:
            vals[c] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()


def e4m3_decode(byte):
    """Value of E4M3 byte(s) as float64.  Only non-negative finite codes
    (0x00..0x7E) are produced by the encoder; others raise."""
    byte = np.asarray(byte, dtype=np.int64)
    if np.any((byte < 0) | (byte > E4M3_MAX_CODE)):
        raise ValueError("e4m3_decode: only non-negative finite codes are used")
    return E4M3_VALUES[byte]


def e4m3_encode(v):
    """E4M3 code nearest to v >= 0, ties to the even code, saturating at 448."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(v < 0):
        raise ValueError("e4m3_encode: expects finite non-negative values")
    t = E4M3_VALUES
    hi = np.searchsorted(t, v, side="left")  # t[hi-1] < v <= t[hi]
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo = np.abs(v - t[lo])
    dhi = np.abs(t[hi] - v)
    pick = np.where(dlo < dhi, lo, hi)
    tie = dlo == dhi
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(v >= E4M3_MAX, E4M3_MAX_CODE, pick)
    return pick.astype(np.uint8)


# ---------------------------------------------------------------------------
# bf16 helpers (round-to-nearest-even from fp32 bit patterns)
# ---------------------------------------------------------------------------

def bf16_bits_from_f32(x):
    """Round float32 array to bfloat16 (nearest, ties to even); returns uint16 bits.
    Inputs are finite."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def f32_from_bf16_bits(b):
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


# ---------------------------------------------------------------------------
# NVFP4 quantization of one tensor (activation rows or one weight matrix)
# ---------------------------------------------------------------------------

TENSOR_SCALE_DIVISOR = np.float32(E2M1_MAX * E4M3_MAX)  # 2688


def tensor_scale(x):
    """Per-tensor FP32 scale g = fl32(max|x| / 2688); g = 1 for an all-zero tensor."""
    a = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float32)))) if np.size(x) else np.float32(0)
    if a == 0:
        return np.float32(1.0)
    return np.float32(a / TENSOR_SCALE_DIVISOR)


class NVFP4:
    """An NVFP4 tensor: packed codes [rows, cols/2] u8, E4M3 scales [rows, cols/16] u8,
    FP32 tensor scale g.  ``mag`` / ``sign`` / ``dq`` are kept for the RAC steps."""

    def __init__(self, codes, scales, g, mag, sign, dq):
        self.codes, self.scales, self.g = codes, scales, np.float32(g)
        self.mag, self.sign, self.dq = mag, sign, dq


def pack_nibbles(code):
    """[rows, cols] 4-bit codes -> [rows, cols/2] bytes, element 2j in the low nibble."""
    code = np.asarray(code, dtype=np.uint8)
    return (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def quantize_nvfp4(x, g=None):
    """NVFP4-quantize a 2-D float32 tensor [rows, cols] (cols % 16 == 0).

    Steps (the activation quantization that [Gist §2.1] says is recomputed
    online on every rollout forward, and the weight path of [Gist §2.2-A]):
      1. g = tensor_scale(x) unless given;
      2. per 16-block: amax_b, s_real = fl32(fl32(amax_b/6)/g), s = E4M3(s_real);
      3. d = fl32(dec(s)·g);
      4. per element: v = fl32(|x|/d), magnitude index = nearest E2M1 level
         (0 if d == 0); code = sign bit << 3 | index;
      5. dq = ±fl32(level·d), the FP32 dequantized value.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % 16:
        raise ValueError("quantize_nvfp4 expects [rows, cols] with cols % 16 == 0")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    rows, cols = x.shape
    g = tensor_scale(x) if g is None else np.float32(g)
    ax = np.abs(x)
    blk_amax = ax.reshape(rows, cols // 16, 16).max(axis=2)
    s_real = (blk_amax / np.float32(6.0)).astype(np.float32)
    s_real = (s_real / g).astype(np.float32)
    s = e4m3_encode(s_real)
    d_blk = (e4m3_decode(s).astype(np.float32) * g).astype(np.float32)
    d = np.repeat(d_blk, 16, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(d > 0, ax / np.where(d > 0, d, np.float32(1)), np.float32(0)).astype(np.float32)
    mag = e2m1_round_magnitude(v)
    mag = np.where(d > 0, mag, 0)
    sign = np.signbit(x)
    code = ((sign.astype(np.uint8) << 3) | mag.astype(np.uint8)).astype(np.uint8)
    lvl = E2M1_MAGNITUDES[mag].astype(np.float32)
    dqm = (lvl * d).astype(np.float32)
    dq = np.where(sign, -dqm, dqm).astype(np.float32)
    return NVFP4(pack_nibbles(code), s, g, mag, sign, dq)


def dequant_exact(codes, scales, g):
    """Exact value of every element, sign·level·dec(s)·g, in float64
    (at most 2+4+24 significant bits, so exact)."""
    code = unpack_nibbles(codes)
    rows, cols = code.shape
    val = e2m1_decode(code)
    sc = np.repeat(e4m3_decode(scales), 16, axis=1)
    return val * sc * np.float64(np.float32(g))


def dequant_f32(codes, scales, g):
    """FP32 dequantized value ±fl32(level·fl32(dec(s)·g))."""
    code = unpack_nibbles(codes)
    d = np.repeat((e4m3_decode(scales).astype(np.float32) * np.float32(g)).astype(np.float32), 16, axis=1)
    lvl = E2M1_MAGNITUDES[code & 7].astype(np.float32)
    m = (lvl * d).astype(np.float32)
    return np.where((code & 8) != 0, -m, m).astype(np.float32)


# ---------------------------------------------------------------------------
# Residual Activation Compensation ([Gist §2.2-B], [Wiki Methodology])
# ---------------------------------------------------------------------------

def rac_nsel(cols, k_percent):
    """Number of selected channels: floor(cols·k/100) in integer arithmetic."""
    if not (0 <= k_percent <= 100):
        raise ValueError("k_percent must be in [0, 100]")
    return (int(cols) * int(k_percent)) // 100


def rac_kpad(nsel):
    return ((int(nsel) + 15) // 16) * 16


def rac_residual(x, q):
    """ΔX = fl32(x − dq): the first-pass quantization error of the activation."""
    return (np.asarray(x, dtype=np.float32) - q.dq).astype(np.float32)


def rac_scores(x, q):
    """Channel score: max over all rows of |ΔX[:, c]| (the residual magnitude
    the channel mask ranks by).  Over zero rows every score is 0: the largest
    of no magnitudes is taken as 0, as tensor_scale takes the amax of an empty
    tensor (the pages do not speak of an empty batch)."""
    r = np.abs(rac_residual(x, q))
    if r.shape[0] == 0:
        return np.zeros(r.shape[1], dtype=np.float32)
    return r.max(axis=0).astype(np.float32)


def rac_select(scores, k_percent):
    """Binary top-k% channel mask as an ascending index list.

    Channels are ranked by (score descending, index ascending) and the first
    nsel are taken; the result is returned sorted ascending, padded to a
    multiple of 16 with index 0 (pad entries carry a zero residual).
    Returns (sel_idx int32 [kpad], nsel).
    """
    scores = np.asarray(scores, dtype=np.float32)
    K = scores.shape[0]
    nsel = rac_nsel(K, k_percent)
    order = np.lexsort((np.arange(K), -scores.astype(np.float64)))
    chosen = np.sort(order[:nsel])
    sel = np.zeros(rac_kpad(nsel), dtype=np.int32)
    sel[:nsel] = chosen
    return sel, nsel


def rac_quantize_residual(x, q, sel_idx, nsel):
    """Second-pass NVFP4 quantization of the masked residual channels.

    G[r, j] = ΔX[r, sel_j] for j < nsel, 0 for pad columns; G is quantized with
    its own tensor scale (whose amax is the largest selected channel score).
    """
    dx = rac_residual(x, q)
    rows = dx.shape[0]
    kpad = sel_idx.shape[0]
    G = np.zeros((rows, kpad), dtype=np.float32)
    if nsel:
        G[:, :nsel] = dx[:, sel_idx[:nsel]]
    if kpad == 0:
        return NVFP4(np.zeros((rows, 0), np.uint8), np.zeros((rows, 0), np.uint8),
                     tensor_scale(G), np.zeros((rows, 0), np.int64),
                     np.zeros((rows, 0), bool), G)
    return quantize_nvfp4(G)


def rac_compensated_activation(x, q, r, sel_idx, nsel):
    """FP32 view of the compensated activation dq + (scatter of the residual dq)."""
    out = q.dq.copy()
    if nsel:
        out[:, sel_idx[:nsel]] = (out[:, sel_idx[:nsel]] + r.dq[:, :nsel]).astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# GEMM reference (extended-K W4A4 + RAC), float64 accumulation
# ---------------------------------------------------------------------------

def gemm_ref(xq_exact, w_exact, rq_exact=None, sel_idx=None):
    """Y = Xq·Wqᵀ + Rq·Wq[:, sel]ᵀ in float64 for one expert.

    xq_exact [M, K], w_exact [N, K], rq_exact [M, kpad], sel_idx [kpad]
    (pad entries multiply zero residual columns).  This is the quantized path
    plus the correction term, which [Wiki Methodology] adds before the GEMM
    and [Gist §2.2-B] adds to the quantized output — the same sum by linearity.
    """
    y = xq_exact @ w_exact.T
    if rq_exact is not None and sel_idx is not None and sel_idx.size:
        y = y + rq_exact @ w_exact[:, sel_idx].T
    return y


# ---------------------------------------------------------------------------
# Trainer-side weight quantize-dequantize ([Gist §2.1], [Gist §2.2-A])
# ---------------------------------------------------------------------------

def weight_qdq(w, g=None):
    """Fake-quantize one weight matrix: NVFP4 quantize, then dequantize to bf16
    (round-to-nearest-even of the FP32 dequantized value).  Returns
    (bf16 bits uint16 [rows, cols], NVFP4)."""
    q = quantize_nvfp4(w, g)
    return bf16_bits_from_f32(q.dq), q


# ---------------------------------------------------------------------------
# MoE routing, SwiGLU and combine (support steps around the expert GEMM)
# ---------------------------------------------------------------------------

def softmax(logits):
    z = np.asarray(logits, dtype=np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def route(logits, top):
    """Top-`top` experts per token by logit (ties to the lower expert index);
    combine weights are the softmax probabilities of the chosen experts (no
    renormalization).  Routed rows are ordered by (expert, token, slot).

    Returns ids [T, top] int32, weights [T, top] float64, expert_offsets [E+1]
    int32, row_token [T·top] int32, inverse [T, top] int32 (row of (t, slot)).
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    ids = order[:, :top].astype(np.int32)
    p = softmax(logits)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    counts = np.zeros(E, dtype=np.int64)
    for e in ids.reshape(-1):
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    row_token = np.empty(T * top, dtype=np.int32)
    inverse = np.empty((T, top), dtype=np.int32)
    fill = offsets[:-1].astype(np.int64).copy()
    for t in range(T):  # tokens in order, so each expert's rows are token-ordered
        for j in range(top):
            e = ids[t, j]
            inverse[t, j] = fill[e]
            row_token[fill[e]] = t
            fill[e] += 1
    return ids, w, offsets, row_token, inverse


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(y_gate, y_up):
    return silu(y_gate) * np.asarray(y_up, dtype=np.float64)


def combine(y, inverse, weights):
    """out[t] = Σ_slot w[t, slot] · y[inverse[t, slot]] (float64)."""
    y = np.asarray(y, dtype=np.float64)
    inverse = np.asarray(inverse)
    w = np.asarray(weights, dtype=np.float64)
    out = np.zeros((inverse.shape[0], y.shape[1]), dtype=np.float64)
    for j in range(inverse.shape[1]):
        out += w[:, j:j + 1] * y[inverse[:, j]]
    return out


# ---------------------------------------------------------------------------
# Composite paths used by tests and the CPU baseline
# ---------------------------------------------------------------------------

def quantize_weights(w, n_seg=1):
    """Quantize expert weights [E, N, K] with one tensor scale per (expert,
    segment of N/n_seg rows).  Returns codes [E,N,K/2], scales [E,N,K/16],
    gscale [E, n_seg] and the exact dequantized weights [E,N,K] (float64)."""
    w = np.asarray(w, dtype=np.float32)
    E, N, K = w.shape
    seg = N // n_seg
    codes = np.empty((E, N, K // 2), np.uint8)
    scales = np.empty((E, N, K // 16), np.uint8)
    gs = np.empty((E, n_seg), np.float32)
    exact = np.empty((E, N, K), np.float64)
    for e in range(E):
        for s in range(n_seg):
            q = quantize_nvfp4(w[e, s * seg:(s + 1) * seg])
            codes[e, s * seg:(s + 1) * seg] = q.codes
            scales[e, s * seg:(s + 1) * seg] = q.scales
            gs[e, s] = q.g
            exact[e, s * seg:(s + 1) * seg] = dequant_exact(q.codes, q.scales, q.g)
    return codes, scales, gs, exact


def rac_linear(x, w_exact, k_percent, row_token=None, expert_offsets=None):
    """Quantize activation x [A, K] (+ RAC at k%), then the grouped expert GEMM
    reference for rows i with activation row row_token[i] (identity if None)
    and expert e for offsets[e] <= i < offsets[e+1].  Returns a dict with every
    intermediate the GPU path exposes."""
    x = np.asarray(x, dtype=np.float32)
    q = quantize_nvfp4(x)
    scores = rac_scores(x, q)
    sel, nsel = rac_select(scores, k_percent)
    r = rac_quantize_residual(x, q, sel, nsel)
    xe = dequant_exact(q.codes, q.scales, q.g)
    re = dequant_exact(r.codes, r.scales, r.g) if sel.size else None
    E = w_exact.shape[0]
    R = x.shape[0] if row_token is None else len(row_token)
    rt = np.arange(R) if row_token is None else np.asarray(row_token)
    offs = np.array([0, R]) if expert_offsets is None else np.asarray(expert_offsets)
    y = np.zeros((R, w_exact.shape[1]), np.float64)
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if a == b:
            continue
        rows = rt[a:b]
        y[a:b] = gemm_ref(xe[rows], w_exact[e], None if re is None else re[rows], sel if nsel else None)
    return dict(q=q, scores=scores, sel=sel, nsel=nsel, r=r, y=y)


def moe_layer(x, logits, w_gu_exact, w_down_exact, k_percent, top=8):
    """Oracle MoE FFN layer: route -> W4A4+RAC gate_up -> SwiGLU (rounded to
    bf16) -> W4A4+RAC down -> combine.  Returns a dict of stages."""
    ids, wts, offs, rt, inv = route(logits, top)
    gu = rac_linear(x, w_gu_exact, k_percent, rt, offs)
    I = w_gu_exact.shape[1] // 2
    h = swiglu(gu["y"][:, :I], gu["y"][:, I:])
    h_bf16 = f32_from_bf16_bits(bf16_bits_from_f32(h.astype(np.float32)))
    dn = rac_linear(h_bf16, w_down_exact, k_percent, None, offs)
    out = combine(dn["y"], inv, wts)
    return dict(ids=ids, weights=wts, offsets=offs, row_token=rt, inverse=inv,
                gate_up=gu, h=h, h_bf16=h_bf16, down=dn, out=out)


# ---------------------------------------------------------------------------
# Ablation variants ([Gist §2.1], [Gist §4] "Ablatie studies")
# ---------------------------------------------------------------------------

def fake_quant_activation(x):
    """Symmetric W4A4 QAT's trainer-side activation: the same NVFP4
    quantize-dequantize as the weights, applied to the activation tensor (one
    tensor scale for the whole tensor), rounded to bf16.  [Gist §2.1] names
    this scheme (weights and activations fake-quantized on the trainer) and
    [Gist §4] compares it with the asymmetric W4A16 scheme.  Returns bf16 bits
    [rows, cols]."""
    return weight_qdq(x)[0]


def rac_linear_per_expert(x, w_exact, k_percent, expert_offsets):
    """RAC with one channel mask per expert instead of one per input tensor.

    Rows of x are grouped by expert (row i belongs to expert e for
    offsets[e] <= i < offsets[e+1]).  The activation is quantized once with
    its tensor scale g; each expert then scores the channels over its own rows
    only, selects its top k% and quantizes its own residual with its own
    residual tensor scale.  Y rows are the expert's W4A4 + RAC product.
    Returns dict(q=global NVFP4, experts=[per-expert dict or None], y)."""
    x = np.asarray(x, dtype=np.float32)
    offs = np.asarray(expert_offsets)
    q = quantize_nvfp4(x)
    E = w_exact.shape[0]
    y = np.zeros((x.shape[0], w_exact.shape[1]), np.float64)
    experts = []
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if a == b:
            experts.append(None)
            continue
        xe = x[a:b]
        qe = quantize_nvfp4(xe, q.g)  # row blocks: the same codes as q's rows a..b
        scores = rac_scores(xe, qe)
        sel, nsel = rac_select(scores, k_percent)
        r = rac_quantize_residual(xe, qe, sel, nsel)
        xq = dequant_exact(qe.codes, qe.scales, qe.g)
        rq = dequant_exact(r.codes, r.scales, r.g) if sel.size else None
        y[a:b] = gemm_ref(xq, w_exact[e], rq, sel if nsel else None)
        experts.append(dict(q=qe, scores=scores, sel=sel, nsel=nsel, r=r))
    return dict(q=q, experts=experts, y=y)


# ---------------------------------------------------------------------------
# W4A16 QAT backward of a grouped linear ([Gist §2.2-A])
# ---------------------------------------------------------------------------

def qat_linear_backward(x, w_master, dy, row_token=None, expert_offsets=None):
    """Backward of y[i] = W_qdq[e(i)] · x[t(i)] with the straight-through
    estimator through the weight QDQ.

    [Gist §2.2-A]: every forward sees the discretized weights while the
    optimizer updates the bf16 masters; the gradient reaches the masters
    unchanged through the QDQ (the straight-through reading).
    - dX: per routed row i, dxr[i] = dy[i] · W_qdq[e(i)]; each token sums
      the rows that read it: dx[t] = sum over {i : t(i) = t} of dxr[i].
    - dW: dW_master[e] = dW_qdq[e] = sum over the expert's rows i of
      dy[i]^T x[t(i)].
    x [A, K], w_master [E, N, K] float32 (bf16 values), dy [R, N]; float64
    products.  Returns dict(w_qdq float64 [E,N,K], dxr [R,K], dx [A,K],
    dw [E,N,K])."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    w_master = np.asarray(w_master, dtype=np.float32)
    E, N, K = w_master.shape
    R = dy.shape[0]
    rt = np.arange(R) if row_token is None else np.asarray(row_token)
    offs = np.array([0, R]) if expert_offsets is None else np.asarray(expert_offsets)
    w_qdq = np.stack([f32_from_bf16_bits(weight_qdq(w_master[e])[0]) for e in range(E)]).astype(np.float64)
    dxr = np.zeros((R, K), np.float64)
    dw = np.zeros((E, N, K), np.float64)
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if a == b:
            continue
        dxr[a:b] = dy[a:b] @ w_qdq[e]
        dw[e] = dy[a:b].T @ x[rt[a:b]]
    dx = np.zeros_like(x)
    np.add.at(dx, rt, dxr)
    return dict(w_qdq=w_qdq, dxr=dxr, dx=dx, dw=dw)


def rac_merged_operand(q, r, sel_idx, nsel):
    """The RAC-corrected activation as one fp16 operand, in units of the
    activation's tensor scale: for a selected channel c = sel_j,
    A[t, c] = fp16(X'[t, c] + fl32(R'[t, j] * fl32(g_r / g_x))), and X'[t, c]
    elsewhere.  X' and R' are the exact e2m1 * e4m3 values (no tensor scale);
    the sum is one fp32 addition, then one rounding to fp16 ([Gist §2.2-B]:
    the correction is added to the quantized activation before the GEMM).
    Returns float16 [rows, cols]."""
    xs = dequant_exact(q.codes, q.scales, np.float32(1.0)).astype(np.float32)
    out = xs.copy()
    if nsel:
        rs = dequant_exact(r.codes, r.scales, np.float32(1.0)).astype(np.float32)
        ratio = np.float32(np.float32(r.g) / np.float32(q.g))
        cols = sel_idx[:nsel]
        out[:, cols] = (xs[:, cols] + (rs[:, :nsel] * ratio).astype(np.float32)).astype(np.float32)
    return out.astype(np.float16)
