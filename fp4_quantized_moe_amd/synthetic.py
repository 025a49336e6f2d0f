"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle runs.

This module only draws random numbers and casts them to the storage dtype
(float32 -> bfloat16 round-to-nearest-even via torch's CPU cast).  It holds
none of the quantization, selection or GEMM arithmetic, and imports neither
the HIP binding nor the oracle.

Workloads (all from numpy PCG64 streams, fp32 first, then cast where bf16 is
named; "N(0, s)" means standard deviation s):

* ``dense_small``   X fp32 64x256 ~N(0,1) with 4 outlier channels x20,
                    W fp32 512x256 ~N(0,0.02)                  (seed 1)
* ``expert_gemm``   X bf16 4096x2048 ~N(0,1) with 1% outlier channels x30,
                    W bf16 1536x2048 ~N(0,0.02)                (seed 2)
* ``moe_prefill``   16384 tokens, hidden 2048, 64 experts, top-8 routing
                    with Zipf(1.1)-skewed expert load (Gumbel-perturbed
                    log-Zipf logits), SwiGLU intermediate 768   (seed 3)
* ``moe_decode``    256 tokens, hidden 2048, 128 experts, top-8 from
                    N(0,1) logits, intermediate 1024           (seed 4)
* ``trainer_qdq``   48 layers x 128 experts x 3 matrices of 2048x1024 bf16
                    ~N(0,0.02) masters and a bf16 grouped forward on 8192
                    tokens with N(0,1) logits, top-8           (seed 5)
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


def to_bf16(x_f32: np.ndarray):
    """Round float32 values to bfloat16 with torch's CPU cast.  Returns
    (uint16 bit patterns, float32 values of those bf16 numbers)."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16).copy()
    vals = t.to(torch.float32).numpy().copy()
    return bits, vals


@dataclass
class Activation:
    """An activation or weight tensor: float32 values and, if stored as bf16,
    the bf16 bit patterns (``bits``) the device receives."""
    f32: np.ndarray
    bits: np.ndarray | None  # uint16 when the storage dtype is bf16

    @property
    def is_bf16(self) -> bool:
        return self.bits is not None


def _normal(rng, shape, std=1.0):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def activation(rng, rows, cols, n_outliers, outlier_scale, bf16=True):
    """N(0,1) activations with `n_outliers` channels (chosen without
    replacement) multiplied by `outlier_scale`."""
    x = _normal(rng, (rows, cols))
    if n_outliers:
        ch = rng.choice(cols, n_outliers, replace=False)
        x[:, ch] *= np.float32(outlier_scale)
    if bf16:
        bits, vals = to_bf16(x)
        return Activation(vals, bits)
    return Activation(x, None)


def weights(rng, shape, std=0.02, bf16=True):
    w = _normal(rng, shape, std)
    if bf16:
        bits, vals = to_bf16(w)
        return Activation(vals, bits)
    return Activation(w, None)


def drifted(rng, act, rel_std=2.0 ** -9):
    """A second copy of a bf16 activation that differs from it by engine
    drift: each element is multiplied by (1 + e) with e ~ N(0, rel_std) and
    rounded to bf16 again (about one bf16 rounding step of noise at the
    default)."""
    e = _normal(rng, act.f32.shape, rel_std)
    bits, vals = to_bf16(act.f32 * (np.float32(1.0) + e))
    return Activation(vals, bits)


def zipf_logits(rng, tokens, experts, s=1.1):
    """Logits log p_Zipf(s)[rank(e)] + Gumbel(0,1) noise; ranks are a seeded
    permutation of the experts.  Top-k of these is sampling without
    replacement proportional to the Zipf weights (Gumbel-top-k)."""
    ranks = rng.permutation(experts) + 1
    base = -s * np.log(ranks.astype(np.float64))
    gumbel = rng.gumbel(0.0, 1.0, size=(tokens, experts))
    return (base[None, :] + gumbel).astype(np.float32)


def gaussian_logits(rng, tokens, experts):
    return rng.standard_normal((tokens, experts), dtype=np.float32)


@dataclass
class DenseWorkload:
    name: str
    x: Activation
    w: Activation  # [N, K]
    k_values: tuple


def dense_small(seed=1):
    rng = np.random.default_rng(seed)
    x = activation(rng, 64, 256, 4, 20.0, bf16=False)
    w = weights(rng, (512, 256), 0.02, bf16=False)
    return DenseWorkload("dense_small", x, w, (50,))


def expert_gemm(seed=2, M=4096, K=2048, N=1536):
    rng = np.random.default_rng(seed)
    x = activation(rng, M, K, (K * 1) // 100, 30.0, bf16=True)
    w = weights(rng, (N, K), 0.02, bf16=True)
    return DenseWorkload("expert_gemm", x, w, (0, 25, 50, 100))


@dataclass
class MoEWorkload:
    name: str
    x: Activation          # [T, H] bf16
    logits: np.ndarray     # [T, E] fp32
    w_gate_up: Activation  # [E, 2I, H]: gate rows then up rows
    w_down: Activation     # [E, H, I]
    top: int
    k_percent: int


def moe_prefill(seed=3, T=16384, H=2048, E=64, I=768, top=8, k=50):
    rng = np.random.default_rng(seed)
    x = activation(rng, T, H, H // 100, 30.0, bf16=True)
    logits = zipf_logits(rng, T, E)
    wgu = weights(rng, (E, 2 * I, H))
    wd = weights(rng, (E, H, I))
    return MoEWorkload("moe_prefill", x, logits, wgu, wd, top, k)


def moe_decode(seed=4, T=256, H=2048, E=128, I=1024, top=8, k=50):
    rng = np.random.default_rng(seed)
    x = activation(rng, T, H, H // 100, 30.0, bf16=True)
    logits = gaussian_logits(rng, T, E)
    wgu = weights(rng, (E, 2 * I, H))
    wd = weights(rng, (E, H, I))
    return MoEWorkload("moe_decode", x, logits, wgu, wd, top, k)


def trainer_layer_weights_device(seed, layer, experts=128, hidden=2048, inter=1024, device="cuda"):
    """Bf16 master weights of one trainer layer, drawn on the device with a
    seeded torch generator (38.65 G elements over 48 layers do not fit a host
    array).  Returns (gate_up [experts*2, inter, hidden], down [experts,
    hidden, inter]); matrix 2e is expert e's gate, 2e+1 its up projection.
    Blocks run along each matrix's input dimension (the last axis)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1000003 + layer)
    gu = torch.randn((experts * 2, inter, hidden), generator=gen, device=device, dtype=torch.float32)
    gu = (gu * 0.02).to(torch.bfloat16)
    dn = torch.randn((experts, hidden, inter), generator=gen, device=device, dtype=torch.float32)
    dn = (dn * 0.02).to(torch.bfloat16)
    return gu, dn
