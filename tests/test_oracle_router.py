"""Pins of the oracle's router product (CPU only).

The pages print no router values, so the product is pinned by closed forms,
exact special cases and a brute-force sum on tiny shapes, each of which a
dropped term, a transposed operand or a wrong bias index would fail.
"""
import math

import numpy as np

import oracle
from synth import CONFIGS, f32_to_bf16_bits, make_router, make_x


def bf16(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_one_hot_rows_select_columns():
    """w[e] = unit vector at column c(e): logits[:, e] = x[:, c(e)] exactly."""
    rng = np.random.default_rng(1)
    T, H, E = 5, 48, 7
    cols = rng.permutation(H)[:E]
    w = np.zeros((E, H), dtype=np.float32)
    w[np.arange(E), cols] = 1.0
    x = rng.standard_normal((T, H)).astype(np.float32)
    out = oracle.router_logits(x, bf16(w))
    assert np.array_equal(out, x[:, cols].astype(np.float64))


def test_constant_router_is_scaled_row_sum():
    """w = 0.5 everywhere: logits[t, e] = 0.5 * sum_h x[t, h] for every e."""
    rng = np.random.default_rng(2)
    T, H, E = 4, 64, 3
    x = bf16(rng.standard_normal((T, H)))
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out = oracle.router_logits(x, bf16(np.full((E, H), 0.5)))
    want = np.array([0.5 * math.fsum(r) for r in xf])
    assert np.allclose(out, want[:, None], rtol=0, atol=1e-12)


def test_brute_force_tiny():
    """A plain triple loop with exact summation on a tiny shape, with a bias."""
    rng = np.random.default_rng(3)
    T, H, E = 3, 8, 5
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = bf16(rng.standard_normal((E, H)))
    wf = (w.astype(np.uint32) << 16).view(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    out = oracle.router_logits(x, w, bias)
    for t in range(T):
        for e in range(E):
            want = math.fsum([float(x[t, h]) * float(wf[e, h]) for h in range(H)] + [float(bias[e])])
            assert abs(out[t, e] - want) <= 1e-12 * (1 + abs(want))
            # operand order matters: the transpose (w[h, e] reading) must not match
    assert not np.allclose(out, oracle.router_logits(x, w[:, ::-1].copy(), bias))


def test_linear_in_x_and_bias_adds():
    """Doubling x doubles the product exactly; the bias shifts expert e only."""
    cfg = CONFIGS[0]
    w, bias = make_router(cfg, seed=4)
    x = make_x(cfg, seed=4)
    a = oracle.router_logits(x, w)
    assert np.array_equal(oracle.router_logits(2 * x, w), 2 * a)
    b = np.zeros(cfg.E, dtype=np.float32)
    b[3] = 0.75
    d = oracle.router_logits(x, w, b) - a
    assert np.allclose(d[:, 3], 0.75, atol=1e-12) and np.allclose(np.delete(d, 3, axis=1), 0, atol=0)


def test_generated_router_scale():
    """The generated router gives scores of about unit spread for N(0,1) inputs
    (the recipe's 1/sqrt(H) row scale), plus the layer's Zipf bias."""
    cfg = CONFIGS[1]
    w, bias = make_router(cfg, seed=0)
    x = make_x(cfg.with_(T=64), seed=0)
    s = oracle.router_logits(x, w)
    assert 0.8 < s.std() < 1.2
    assert np.array_equal(bias, np.asarray(__import__("synth").zipf_bias(cfg, 0), dtype=np.float32))
