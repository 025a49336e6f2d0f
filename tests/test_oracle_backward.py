"""Pins for the oracle's W4A16 QAT backward (CPU only).

The technical summary's section 2.2-A: the trainer's forward sees NVFP4
fake-quantized weights while the bf16 masters are updated; the gradient
passes the QDQ unchanged (straight-through). The loss L = sum(dy * y) is
linear in x and in W_qdq, so central finite differences of the oracle's own
forward are exact up to rounding and pin both gradients with no shared
formula. Pins:
- central finite differences in x and in W_qdq;
- an element-by-element triple loop;
- token summation through the routing;
- a grid weight for which the QDQ is the identity.
"""
import numpy as np

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import synthetic as S


def _layer(seed, A=5, K=32, N=16, counts=(3, 0, 4), top=None):
    rng = np.random.default_rng(seed)
    x = S.activation(rng, A, K, 0, 1.0, bf16=True).f32
    w = S.weights(rng, (len(counts), N, K)).f32
    R = int(sum(counts))
    rt = rng.integers(0, A, R).astype(np.int32)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    dy = rng.standard_normal((R, N))
    return x, w, dy, rt, offs


def _forward(x, w_qdq, rt, offs):
    y = np.zeros((len(rt), w_qdq.shape[1]))
    for e in range(w_qdq.shape[0]):
        a, b = offs[e], offs[e + 1]
        for i in range(a, b):
            y[i] = w_qdq[e] @ x[rt[i]]
    return y


def test_finite_differences_in_x_and_w():
    x, w, dy, rt, offs = _layer(401)
    g = O.qat_linear_backward(x, w, dy, rt, offs)
    wq = g["w_qdq"]
    h = 2.0 ** -10

    def loss(xx, ww):
        return float((dy * _forward(xx, ww, rt, offs)).sum())

    x64 = x.astype(np.float64)
    for (t, k) in [(0, 0), (2, 7), (4, 31), (1, 16)]:
        xp, xm = x64.copy(), x64.copy()
        xp[t, k] += h
        xm[t, k] -= h
        fd = (loss(xp, wq) - loss(xm, wq)) / (2 * h)
        assert abs(fd - g["dx"][t, k]) <= 1e-9 * max(1.0, abs(fd))
    for (e, n, k) in [(0, 0, 0), (2, 15, 31), (0, 3, 9), (1, 5, 5)]:
        wp, wm = wq.copy(), wq.copy()
        wp[e, n, k] += h
        wm[e, n, k] -= h
        fd = (loss(x64, wp) - loss(x64, wm)) / (2 * h)
        assert abs(fd - g["dw"][e, n, k]) <= 1e-9 * max(1.0, abs(fd))
    assert (g["dw"][1] == 0).all()  # expert 1 has no rows


def test_triple_loop():
    x, w, dy, rt, offs = _layer(402, A=4, K=16, N=8, counts=(2, 3))
    g = O.qat_linear_backward(x, w, dy, rt, offs)
    wq = g["w_qdq"]
    dx = np.zeros(x.shape)
    dw = np.zeros(wq.shape)
    for e in range(2):
        for i in range(offs[e], offs[e + 1]):
            for n in range(8):
                for k in range(16):
                    dx[rt[i], k] += dy[i, n] * wq[e, n, k]
                    dw[e, n, k] += dy[i, n] * float(x[rt[i], k])
    assert np.allclose(g["dx"], dx, rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dw"], dw, rtol=1e-12, atol=1e-12)


def test_token_sum_and_identity_rows():
    """With the identity row map each token has one row, so dx == dxr; with
    every row reading token 0, dx[0] is the column sum of dxr."""
    x, w, dy, _, offs = _layer(403, A=7, counts=(3, 4))
    g = O.qat_linear_backward(x, w, dy, None, offs)
    assert np.array_equal(g["dx"], g["dxr"])
    g0 = O.qat_linear_backward(x, w, dy, np.zeros(7, np.int32), offs)
    assert np.allclose(g0["dx"][0], g0["dxr"].sum(axis=0), rtol=1e-12)
    assert (g0["dx"][1:] == 0).all()


def test_grid_weights_pass_qdq_unchanged():
    """Weights on the NVFP4 grid: W_qdq == W, so the backward is the plain
    linear backward of the masters."""
    rng = np.random.default_rng(404)
    lv = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    sc = O.E4M3_VALUES[rng.integers(48, 120, (16, 2))]
    sc[0, 0] = 448.0
    m = lv[rng.integers(0, 8, (16, 32))] * np.where(rng.random((16, 32)) < 0.5, -1, 1)
    m[:, ::16] = 6.0
    w = (m * np.repeat(sc, 16, axis=1) * 2.0 ** -12).astype(np.float32)[None]
    x = rng.standard_normal((6, 32)).astype(np.float32)
    dy = rng.standard_normal((6, 16))
    g = O.qat_linear_backward(x, w, dy)
    assert np.array_equal(g["w_qdq"][0], w[0].astype(np.float64))
    assert np.allclose(g["dw"][0], dy.T @ x.astype(np.float64), rtol=1e-12)
    assert np.allclose(g["dx"], dy @ w[0].astype(np.float64), rtol=1e-12)
