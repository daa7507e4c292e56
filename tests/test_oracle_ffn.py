"""Pins of the oracle's dequantisation and expert FFN / combine.

The dequant pins plant single codes and check that exactly the intended weight
moves, so a wrong bit order, block index or affine term fails. The FFN pins
compare the C oracle with an independent NumPy float64 dense brute force, a
closed form for constant weights, a textbook SwiGLU MLP in torch, linearity in
the gates and token-permutation equivariance.
"""
import numpy as np
import pytest

import oracle
from oracle.dense import dense_layer, dequant_expert, x_float64
from synth import CONFIGS, make_layer

F16 = lambda v: np.float16(v).view(np.uint16)  # noqa: E731


def test_half_conversion_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits[::7]])
    r = ref[::7]
    nan = np.isnan(r)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], r[~nan])


def one_block(d, m, codes=None, hi=None):
    codes = np.zeros(8, np.uint8) if codes is None else np.asarray(codes, np.uint8)
    dm = np.array([F16(d), F16(m)], dtype=np.uint16)
    return codes, hi, dm


@pytest.mark.parametrize("prec", ["f32", "f64"])
def test_dequant_constant_cases(prec):
    d, m = 0.0625, -0.09375
    c, _, dm = one_block(d, m)
    assert np.all(oracle.dequant_row(2, c, None, dm, 32, prec) == m)              # q = 0
    assert np.all(oracle.dequant_row(2, np.full(8, 0xFF, np.uint8), None, dm, 32, prec)
                  == 3 * d + m)                                                    # q = 3
    assert np.all(oracle.dequant_row(3, np.full(8, 0xFF, np.uint8), np.full(4, 0xFF, np.uint8),
                                     dm, 32, prec) == 7 * d + m)                   # q = 7
    c0, _, dm0 = one_block(0.0, m, np.full(8, 0xAA, np.uint8))
    assert np.all(oracle.dequant_row(2, c0, None, dm0, 32, prec) == m)            # d = 0


@pytest.mark.parametrize("j", range(32))
def test_dequant_planted_code(j):
    d, m = 0.5, 0.25
    for q in (1, 2, 3):
        codes = np.zeros(8, np.uint8)
        codes[j // 4] = q << (2 * (j % 4))
        w = oracle.dequant_row(2, codes, None, np.array([F16(d), F16(m)], np.uint16), 32)
        expect = np.full(32, m)
        expect[j] = q * d + m
        assert np.array_equal(w, expect), (j, q)
    # Q3: bit j of the high plane adds 4 to code j only
    hi = np.zeros(4, np.uint8)
    hi[j // 8] = 1 << (j % 8)
    w = oracle.dequant_row(3, np.zeros(8, np.uint8), hi, np.array([F16(d), F16(m)], np.uint16), 32)
    expect = np.full(32, m)
    expect[j] = 4 * d + m
    assert np.array_equal(w, expect)


def test_dequant_blocks_use_their_own_scale():
    K = 96
    codes = np.full(24, 0x55, np.uint8)           # q = 1 everywhere
    ds = [0.5, 0.25, 2.0]
    ms = [0.0, -1.0, 0.125]
    dm = np.array([v for p in zip(ds, ms) for v in (F16(p[0]), F16(p[1]))], np.uint16)
    w = oracle.dequant_row(2, codes, None, dm, K)
    assert np.array_equal(w, np.repeat(np.array(ds) + np.array(ms), 32))


def test_dequant_subnormal_scale_exact():
    d_bits = np.uint16(0x0003)                   # 3 * 2^-24, fp16 subnormal
    m_bits = np.uint16(0x8001)                   # -2^-24
    codes = np.full(8, 0xFF, np.uint8)
    w = oracle.dequant_row(2, codes, None, np.array([d_bits, m_bits], np.uint16), 32, "f64")
    assert np.all(w == 9 * 2.0 ** -24 - 2.0 ** -24)


def small_cfg(qtype=2, shared=1, xdtype="bf16", T=6, H=256, E=32, k=4, I=64):
    base = CONFIGS[1] if qtype == 2 else CONFIGS[4]
    return base.with_(T=T, H=H, E=E, k=k, I=I, shared=shared, xdtype=xdtype, cid=base.cid)


def rel_l2_rows(a, b):
    return np.linalg.norm(a - b, axis=1) / np.linalg.norm(b, axis=1)


@pytest.mark.parametrize("cfg", [CONFIGS[0], small_cfg(2), small_cfg(3), small_cfg(2, shared=0),
                                 small_cfg(3, xdtype="f32", k=1)],
                         ids=["tiny", "q2_shared", "q3_shared", "q2_noshared", "q3_k1"])
def test_layer_matches_dense_f64(cfg):
    lay = make_layer(cfg, seed=11)
    idx, gates = oracle.route(lay["logits"], cfg.k)
    y64 = oracle.layer_rows(lay, idx, gates, prec="f64")
    y32 = oracle.layer_rows(lay, idx, gates, prec="f32")
    yd = dense_layer(lay)
    assert np.max(rel_l2_rows(y64, yd)) < 1e-6      # gates rounded to f32 are the only gap
    assert np.max(rel_l2_rows(y32.astype(np.float64), y64)) < 1e-5


def test_expert_forward_matches_matrices():
    cfg = small_cfg(3, H=128, I=96)
    lay = make_layer(cfg, seed=5)
    e = 3
    x = x_float64(lay["x"][0])
    o, g, u, h = oracle.expert_forward(3, cfg.H, cfg.I, lay["codes"][e], lay["hi"][e],
                                       lay["dm"][e], x)
    wg, wu, wd = dequant_expert(3, cfg.H, cfg.I, lay["codes"][e], lay["hi"][e], lay["dm"][e])
    assert np.allclose(g, wg @ x, rtol=1e-12, atol=1e-12)
    assert np.allclose(u, wu @ x, rtol=1e-12, atol=1e-12)
    assert np.allclose(h, g / (1 + np.exp(-g)) * u, rtol=1e-12, atol=1e-14)
    assert np.allclose(o, wd @ h, rtol=1e-12, atol=1e-12)


def test_constant_weights_closed_form():
    # every gate weight a, up weight b, down weight c (codes q = 1 everywhere)
    H, I, E, k, T = 64, 32, 4, 2, 3
    cfg = small_cfg(2, T=T, H=H, E=E, k=k, I=I, xdtype="f32")
    nb_gu, nb = I * H // 32, 3 * H * I // 32
    dm = np.empty((E + 1, nb, 2), np.uint16)
    (da, ma), (db, mb), (dc, mc) = (0.5, 0.25), (0.25, -0.125), (0.125, -0.0625)
    dm[:, :nb_gu] = [F16(da), F16(ma)]
    dm[:, nb_gu:2 * nb_gu] = [F16(db), F16(mb)]
    dm[:, 2 * nb_gu:] = [F16(dc), F16(mc)]
    a, b, c = da + ma, db + mb, dc + mc
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((T, H)) * 0.1).astype(np.float32)
    lay = {"cfg": cfg, "x": x, "codes": np.full((E + 1, nb * 8), 0x55, np.uint8), "hi": None,
           "dm": dm.reshape(E + 1, -1)}
    idx = np.array([[0, 3], [2, 1], [3, 0]], np.int32)
    gates = np.array([[0.75, 0.25], [0.5, 0.5], [0.125, 0.875]], np.float32)
    y = oracle.layer_rows(lay, idx, gates)
    S = x.astype(np.float64).sum(axis=1)
    h = (a * S) / (1 + np.exp(-a * S)) * (b * S)
    o = c * I * h                                     # same for every output element
    expect = (gates.astype(np.float64).sum(axis=1) + 1.0) * o   # routed + shared
    assert np.allclose(y, expect[:, None], rtol=1e-12)


def test_single_expert_is_textbook_swiglu_mlp():
    torch = pytest.importorskip("torch")
    cfg = small_cfg(2, T=5, H=96, E=1, k=1, I=64, shared=0, xdtype="f32")
    lay = make_layer(cfg, seed=9)
    idx, gates = oracle.route(lay["logits"], 1)
    assert np.all(idx == 0) and np.all(gates == 1.0)
    y = oracle.layer_rows(lay, idx, gates)
    wg, wu, wd = (torch.from_numpy(w) for w in dequant_expert(2, cfg.H, cfg.I, lay["codes"][0],
                                                               None, lay["dm"][0]))
    xt = torch.from_numpy(lay["x"].astype(np.float64))
    mlp = (torch.nn.functional.silu(xt @ wg.T) * (xt @ wu.T)) @ wd.T
    assert np.allclose(y, mlp.numpy(), rtol=1e-10, atol=1e-12)


def test_routed_part_linear_in_gates():
    cfg = small_cfg(2)
    lay = make_layer(cfg, seed=12)
    idx, gates = oracle.route(lay["logits"], cfg.k)
    y1 = oracle.layer_rows(lay, idx, gates)
    y2 = oracle.layer_rows(lay, idx, 2 * gates)
    y0 = oracle.layer_rows(lay, idx, 0 * gates)       # shared expert only
    assert np.allclose(y2 - y1, y1 - y0, rtol=1e-9, atol=1e-12)
    assert not np.allclose(y1, y0)


def test_token_permutation_equivariance():
    cfg = small_cfg(3)
    lay = make_layer(cfg, seed=13)
    idx, gates = oracle.route(lay["logits"], cfg.k)
    y = oracle.layer_rows(lay, idx, gates)
    p = np.random.default_rng(0).permutation(cfg.T)
    lay2 = dict(lay, x=lay["x"][p])
    y2 = oracle.layer_rows(lay2, idx[p], gates[p])
    assert np.array_equal(y2, y[p])
    # and a subset of rows equals the same rows of the full evaluation
    rows = np.array([4, 0, 2], np.int32)
    assert np.array_equal(oracle.layer_rows(lay, idx, gates, rows=rows), y[rows])
