"""Pins for the oracle's MoE support steps: routing, SwiGLU and combine (CPU only).

Pins: softmax closed-form properties, top-k against brute-force sorting,
permutation invariants (offsets sum to R, every (token, slot) appears once,
rows ordered by expert then token), the identity-expert combine, and SiLU's
closed-form identities.
"""
import numpy as np

from oracle import quads_oracle as O
from fp4_quantized_moe_amd import synthetic as S


def test_softmax_properties():
    rng = np.random.default_rng(61)
    z = rng.standard_normal((10, 64)).astype(np.float32)
    p = O.softmax(z)
    assert np.allclose(p.sum(1), 1.0, rtol=0, atol=1e-12)
    assert np.allclose(O.softmax(z.astype(np.float64) + 7.5), p, rtol=1e-12, atol=0)
    two = O.softmax(np.array([[0.0, np.log(3.0)]]))
    assert np.allclose(two, [[0.25, 0.75]], rtol=1e-15)


def test_route_topk_brute_force_and_ties():
    rng = np.random.default_rng(62)
    logits = np.round(rng.standard_normal((50, 16)) * 2).astype(np.float32)  # many ties
    ids, w, offs, rt, inv = O.route(logits, 4)
    for t in range(50):
        ranked = sorted(range(16), key=lambda e: (-float(logits[t, e]), e))
        assert list(ids[t]) == ranked[:4]
    p = O.softmax(logits)
    assert np.array_equal(w, np.take_along_axis(p, ids.astype(np.int64), 1))


def test_route_nan_order():
    """Non-finite logits (outside the method's domain, but the library must
    stay memory-safe and agree with the oracle): experts are chosen by value
    descending, -inf after every real value, NaN after -inf, ties to the
    lower index; -0 ties +0.  Brute force with an explicit class rank."""
    rng = np.random.default_rng(64)
    lg = rng.standard_normal((40, 12)).astype(np.float32)
    lg[::2, ::3] = np.nan
    lg[1::3, 1::2] = -np.inf
    lg[::5, 4] = 0.0
    lg[::5, 5] = -0.0
    lg[7] = np.nan
    ids, *_ = O.route(lg, 10)

    def rank(t, e):
        v = float(lg[t, e])
        if np.isnan(v):
            return (2, 0.0, e)
        if v == -np.inf:
            return (1, 0.0, e)
        return (0, -v, e)

    for t in range(40):
        assert list(ids[t]) == sorted(range(12), key=lambda e: rank(t, e))[:10]


def test_route_permutation_invariants():
    wl = S.moe_decode()
    ids, w, offs, rt, inv = O.route(wl.logits, 8)
    T, E = wl.logits.shape
    assert offs[0] == 0 and offs[-1] == T * 8 and np.all(np.diff(offs) >= 0)
    seen = np.zeros((T, 8), bool)
    for t in range(T):
        for j in range(8):
            row = inv[t, j]
            assert rt[row] == t
            e = ids[t, j]
            assert offs[e] <= row < offs[e + 1]
            seen[t, j] = True
    assert seen.all()
    for e in range(E):
        toks = rt[offs[e]:offs[e + 1]]
        assert np.all(np.diff(toks) > 0)  # token order within an expert


def test_combine_identity_experts():
    """P12: if every expert is the identity, combine returns Σ_j w_tj · x_t."""
    rng = np.random.default_rng(63)
    x = rng.standard_normal((20, 8))
    logits = rng.standard_normal((20, 6)).astype(np.float32)
    ids, w, offs, rt, inv = O.route(logits, 3)
    y = x[rt]  # identity expert output per routed row
    out = O.combine(y, inv, w)
    assert np.allclose(out, x * w.sum(1, keepdims=True), rtol=1e-14, atol=0)


def test_silu_identities():
    z = np.linspace(-30, 30, 1001)
    s = O.silu(z)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(s - O.silu(-z), z, rtol=0, atol=1e-12)   # silu(z) - silu(-z) = z
    assert np.allclose(O.silu(np.array([40.0])), 40.0, rtol=1e-15)
    assert np.allclose(O.swiglu(z, 2.0 * np.ones_like(z)), 2 * s)


def test_zipf_load_is_skewed():
    """The prefill routing generator yields the intended skew (hottest expert
    carries several times the mean load; no expert is empty)."""
    wl = S.moe_prefill(T=4096, H=32, E=64, I=16)
    ids, _, offs, _, _ = O.route(wl.logits, 8)
    cnt = np.diff(offs)
    assert cnt.max() > 3 * cnt.mean() and cnt.min() > 0
