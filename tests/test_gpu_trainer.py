"""GPU parity of the trainer side at full size: NVFP4 QDQ of one layer's bf16
master weights (128 experts x gate, up, down), bit-exact against the oracle on
sampled matrices, and the bf16-operand grouped forward (8192 tokens, top-8)
on sampled experts against a float64 product of the oracle's own QDQ weights.
The masters come from the seeded device generator, as in the benchmark."""
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


def _f32(t):
    return host(t.float())


def test_trainer_layer_full_size_sampled():
    T, H, E, I, top = 8192, 2048, 128, 1024, 8
    rng = np.random.default_rng(5)
    xa = S.activation(rng, T, H, 0, 1.0, bf16=True)
    logits = S.gaussian_logits(rng, T, E)
    gu_m, dn_m = S.trainer_layer_weights_device(5, 0, E, H, I)
    log(f"[trainer] layer 0 QDQ: gate_up {tuple(gu_m.shape)} down {tuple(dn_m.shape)}")
    wq_gu, _ = Q.QdqCall(gu_m)()
    wq_dn, _ = Q.QdqCall(dn_m)()
    pick = np.random.default_rng(96)
    oracle_w = {}
    for b in sorted(set(int(v) for v in pick.choice(2 * E, 6, replace=False)) | {0, 2 * E - 1}):
        bits, _ = O.weight_qdq(_f32(gu_m[b]))
        assert np.array_equal(_bits(wq_gu[b]), bits), ("gate_up", b)
        oracle_w[b] = bits
    for b in sorted(set(int(v) for v in pick.choice(E, 3, replace=False)) | {E - 1}):
        bits, _ = O.weight_qdq(_f32(dn_m[b]))
        assert np.array_equal(_bits(wq_dn[b]), bits), ("down", b)

    log("[trainer] bf16 grouped gate_up forward, sampled experts")
    ids, w, offs, rt, inv = Q.moe_route(torch.from_numpy(logits).cuda(), top)
    _, _, roffs, rrt, _ = O.route(logits, top)
    assert np.array_equal(host(offs), roffs) and np.array_equal(host(rt), rrt)
    R = T * top
    y = Q.moe_w4a4_gemm(N=2 * I, K=H, expert_offsets=offs, num_rows=R, row_token=rt, x_bf16=dev_act(xa),
                        w_bf16=wq_gu.view(E, 2 * I, H))
    xs = xa.f32.astype(np.float64)
    cnt = np.diff(roffs)
    experts = sorted({int(np.argmax(cnt)), int(np.argmin(cnt)), int(pick.integers(0, E))})
    for e in experts:
        a, b = int(roffs[e]), int(roffs[e + 1])
        if a == b:
            continue
        # the oracle's own QDQ of this expert's gate and up masters
        wg = O.f32_from_bf16_bits(O.weight_qdq(_f32(gu_m[2 * e]))[0]).astype(np.float64)
        wu = O.f32_from_bf16_bits(O.weight_qdq(_f32(gu_m[2 * e + 1]))[0]).astype(np.float64)
        ref = xs[rrt[a:b]] @ np.concatenate([wg, wu]).T
        err = rel_err(host(y[a:b]), ref)
        log(f"  expert {e} rows {b - a}: rel err {err:.2e}")
        assert err <= 1e-3, e
