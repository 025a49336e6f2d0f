"""GPU parity of the W4A16 QAT backward (straight-through weight QDQ) through
the C ABI, against the oracle's float64 gradients:
- quads_transpose_bf16 is bit-exact;
- dX (routed rows and per-token sums) and dW are within 1e-3;
- an expert with no rows gets an exactly zero dW.
The shapes are a small routed layer with an empty expert and ragged experts,
identity rows, and the full-size trainer layer (8192 tokens, 128 experts,
2048 -> 2048) on sampled experts and rows."""
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


def _bf16_dev(a):
    return dev_act(a)


@pytest.mark.parametrize("shape", [(3, 40, 72), (1, 256, 128), (2, 8, 1032)])
def test_transpose_bit_exact(shape):
    log(f"[backward] transpose {shape}")
    rng = np.random.default_rng(501)
    a = S.weights(rng, shape, 1.0)
    out = Q.transpose_bf16(_bf16_dev(a))
    assert np.array_equal(_bits(out), np.swapaxes(a.bits, -1, -2))


def _routed_case(seed, T, E, top, N, K, empty=None):
    rng = np.random.default_rng(seed)
    logits = S.gaussian_logits(rng, T, E)
    if empty is not None:
        logits[:, empty] = -1e4  # no token picks this expert
    x = S.activation(rng, T, K, 2, 30.0, bf16=True)
    w = S.weights(rng, (E, N, K))
    ids, tw, offs, rt, inv = Q.moe_route(torch.from_numpy(logits).cuda(), top)
    R = T * top
    dy = S.activation(rng, R, N, 0, 1.0, bf16=True)
    return x, w, dy, offs, rt, inv


def test_backward_routed_small():
    T, E, top, N, K = 50, 5, 2, 256, 128
    log(f"[backward] routed T={T} E={E} top={top} N={N} K={K}, expert 3 empty")
    x, w, dy, offs, rt, inv = _routed_case(502, T, E, top, N, K, empty=3)
    w_qdq, _ = Q.weight_qdq(_bf16_dev(w))
    bw = Q.QatBackward(w_qdq, _bf16_dev(dy), _bf16_dev(x), offs, rt, inv)
    dx, dxr, dw = bw()
    ref = O.qat_linear_backward(x.f32, w.f32, dy.f32, host(rt), host(offs))
    assert np.array_equal(_bits(w_qdq).reshape(E, N, K),
                          np.stack([O.weight_qdq(w.f32[e])[0] for e in range(E)]))
    ho = host(offs)
    assert ho[3] == ho[4]
    assert (host(dw)[3] == 0).all()
    for name, got, want in (("dxr", dxr, ref["dxr"]), ("dx", dx, ref["dx"]), ("dw", dw, ref["dw"])):
        err = rel_err(host(got), want)
        log(f"  {name}: rel err {err:.2e}")
        assert err <= 1e-3, name


def test_backward_identity_rows_ragged():
    """Rows not gathered (the down projection's layout): dx is dxr. Expert row
    counts are not multiples of the 64-row padding."""
    counts = [33, 1, 0, 70, 31]
    E, N, K = len(counts), 128, 384
    R = sum(counts)
    log(f"[backward] identity rows {counts} N={N} K={K}")
    rng = np.random.default_rng(503)
    h = S.activation(rng, R, K, 3, 30.0, bf16=True)
    w = S.weights(rng, (E, N, K))
    dy = S.activation(rng, R, N, 0, 1.0, bf16=True)
    offs_h = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    offs = torch.from_numpy(offs_h).cuda()
    w_qdq, _ = Q.weight_qdq(_bf16_dev(w))
    dx, dxr, dw = Q.QatBackward(w_qdq, _bf16_dev(dy), _bf16_dev(h), offs)()
    ref = O.qat_linear_backward(h.f32, w.f32, dy.f32, None, offs_h)
    assert dx.data_ptr() == dxr.data_ptr()
    assert (host(dw)[2] == 0).all()
    for name, got, want in (("dx", dx, ref["dx"]), ("dw", dw, ref["dw"])):
        err = rel_err(host(got), want)
        log(f"  {name}: rel err {err:.2e}")
        assert err <= 1e-3, name


def test_backward_full_size_sampled():
    """The trainer layer's gate_up at full size: 8192 tokens, 128 experts,
    top-8, K=2048 inputs, N=2048 outputs (gate and up of 1024 each). dW of
    sampled experts and dX of sampled routed rows against the oracle."""
    T, H, E, I, top = 8192, 2048, 128, 1024, 8
    log("[backward] full-size gate_up backward (sampled)")
    rng = np.random.default_rng(504)
    x = S.activation(rng, T, H, 0, 1.0, bf16=True)
    logits = S.gaussian_logits(rng, T, E)
    gu_m, _ = S.trainer_layer_weights_device(5, 0, E, H, I)
    w_qdq, _ = Q.weight_qdq(gu_m)
    w_qdq = w_qdq.view(E, 2 * I, H)
    _, _, offs, rt, inv = Q.moe_route(torch.from_numpy(logits).cuda(), top)
    R = T * top
    gen = torch.Generator(device="cuda")
    gen.manual_seed(504)
    dy = torch.randn((R, 2 * I), generator=gen, device="cuda").to(torch.bfloat16)
    dx, dxr, dw = Q.QatBackward(w_qdq, dy, _bf16_dev(x), offs, rt, inv)()
    ho, hrt = host(offs), host(rt)
    xs = x.f32.astype(np.float64)
    pick = np.random.default_rng(97)
    cnt = np.diff(ho)
    for e in sorted({int(np.argmax(cnt)), int(np.argmin(cnt)), int(pick.integers(0, E))}):
        a, b = int(ho[e]), int(ho[e + 1])
        dye = host(dy[a:b].float()).astype(np.float64)
        ref = dye.T @ xs[hrt[a:b]]
        err = rel_err(host(dw[e]), ref)
        log(f"  dW expert {e} rows {b - a}: rel err {err:.2e}")
        assert err <= 1e-3, e
        # the oracle's own QDQ of this expert's gate and up masters
        wq = np.concatenate([O.f32_from_bf16_bits(O.weight_qdq(host(gu_m[2 * e + s].float()))[0])
                             for s in (0, 1)]).astype(np.float64)
        rows = np.unique(pick.integers(a, b, 8)) if b > a else []
        for i in rows:
            err = rel_err(host(dxr[i]), dye[i - a] @ wq)
            assert err <= 1e-3, (e, i)
        log(f"  dX rows of expert {e}: {len(rows)} checked")
