"""GPU edge cases of the expert FFN against the oracle, through the C ABI.

fp16-subnormal block scales: the dequantisation w = d*q + m must keep fp16
subnormal d and m exactly (the oracle converts them exactly and is pinned on
all 65,536 fp16 patterns). Every down block gets a subnormal d (the down
output stays in fp32, so its size does not matter), and one block column in
eight of gate and up gets a subnormal d, with the activations on those
columns made 1,000 times larger so that these blocks carry a sizeable part
of every gate/up product: flushing them to zero would move the outputs far
past the fast-mode tolerance.
"""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, make_layer
from synth.gen import bf16_bits_to_f32, f32_to_bf16_bits
from gpu_util import experts_of, log, oracle_rows, rel_l2_rows, torch_cuda, upload, y_to_f64

pytestmark = pytest.mark.gpu

TOL = {"fast": 1e-2, "check": 1e-4}


def subnormal_layer(T, seed=51):
    cfg = CONFIGS[1].with_(T=T)
    lay = make_layer(cfg, seed=seed)
    H, I = cfg.H, cfg.I
    nb_mat = I * H // 32
    rng = np.random.default_rng(seed)
    dm = lay["dm"].reshape(cfg.E_tot, -1, 2).copy()
    blk = np.arange(3 * nb_mat)
    sub = np.zeros(3 * nb_mat, bool)
    sub[:2 * nb_mat] = (blk[:2 * nb_mat] % (H // 32)) % 8 == 3   # gate/up block columns
    sub[2 * nb_mat:] = True                                       # every down block
    n_sub = int(sub.sum())
    for e in range(cfg.E_tot):
        d = rng.integers(1, 1024, size=n_sub).astype(np.uint16)  # fp16 subnormal bit patterns
        m = (-1.5 * d.view(np.float16).astype(np.float32)).astype(np.float16).view(np.uint16)
        dm[e, sub, 0] = d
        dm[e, sub, 1] = m
    x = bf16_bits_to_f32(lay["x"]).reshape(T, H // 32, 32)
    x[:, 3::8, :] *= 1000.0
    lay = dict(lay, dm=dm.reshape(lay["dm"].shape), x=f32_to_bf16_bits(x.reshape(T, H)))
    return lay


@pytest.mark.parametrize("T,mode", [(4, "fast"), (64, "fast"), (300, "fast"), (64, "check")])
def test_subnormal_block_scales(T, mode):
    """Decode window (4 tokens), small-batch kernels (64), prefill tiles (300)
    and the fp32 check mode, all with fp16-subnormal d and m."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    lay = subnormal_layer(T)
    dev = upload(lay)
    cfg = lay["cfg"]
    ex = experts_of(lay, dev)
    log(f"[subnormal d] T={T} mode={mode}")
    idx, gates, y = moe.layer(dev["logits"], dev["x"], ex, cfg.k, mode=mode)
    torch.cuda.synchronize()
    idx_o, g_o = oracle.route(lay["logits"], cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    ref = oracle_rows(lay, idx_o, g_o)
    err = rel_l2_rows(y_to_f64(y), ref)
    # the same layer with its gate/up subnormal blocks flushed to zero is far off
    nb = cfg.I * cfg.H // 32
    dm = lay["dm"].reshape(cfg.E_tot, -1, 2).copy()
    gu = dm[:, :2 * nb]
    gu[(gu & 0x7C00) == 0] = 0
    dm[:, :2 * nb] = gu
    flushed = dict(lay, dm=dm.reshape(lay["dm"].shape))
    far = rel_l2_rows(oracle_rows(flushed, idx_o, g_o), ref)
    log(f"[subnormal d] T={T} {mode}: max rel-L2 {err.max():.3e}; flushed gate/up scales "
        f"would give >= {far.min():.2e}")
    assert far.min() > 10 * TOL[mode]
    assert err.max() <= TOL[mode]
    ex.close()


# Row scales of the activation-range cases: rows past fp16's range (65,504),
# rows of tiny values (fp16 would flush them), and ordinary rows, mixed in one
# batch so that every row's scaling is its own.
ROW_SCALES = (1e5, 3e-9, 1.0, 2.5e4, 1e-6, 7e5, 1e-10, 0.5)


def scaled_rows_layer(cfg, seed):
    lay = make_layer(cfg, seed=seed)
    sc = np.array([ROW_SCALES[t % len(ROW_SCALES)] for t in range(cfg.T)], np.float64)
    if cfg.xdtype == "f32":
        x = (lay["x"].astype(np.float64) * sc[:, None]).astype(np.float32)
    else:
        x = f32_to_bf16_bits((bf16_bits_to_f32(lay["x"]).astype(np.float64) * sc[:, None]).astype(np.float32))
    return dict(lay, x=x)


@pytest.mark.parametrize("name,kw,mode", [
    ("window T=4", dict(T=4), "fast"),
    ("window T=3 f32", dict(T=3, xdtype="f32"), "fast"),
    ("two-kernel window k=20", dict(T=4, k=20), "fast"),
    ("small batch T=64 Q3", dict(T=64, qtype=3), "fast"),
    ("small batch T=37", dict(T=37), "fast"),
    ("tiles T=300", dict(T=300), "fast"),
    ("GEMV + tiles H=4096 I=256", dict(T=24, H=4096, I=256, E=64, k=4), "fast"),
    ("check T=64", dict(T=64), "check"),
])
def test_activation_range(name, kw, mode):
    """bf16 activations are honoured over their whole range: each token row
    enters the fp16 matrix cores scaled by its own power of two and h stays in
    bf16, so rows of 1e5 (past fp16's largest value) and of 1e-10 (below its
    smallest) agree with the oracle like ordinary rows."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = CONFIGS[1].with_(**kw)
    lay = scaled_rows_layer(cfg, seed=61)
    dev = upload(lay)
    ex = experts_of(lay, dev)
    log(f"[activation range] {name} mode={mode}")
    idx, gates, y = moe.layer(dev["logits"], dev["x"], ex, cfg.k, mode=mode)
    torch.cuda.synchronize()
    idx_o, g_o = oracle.route(lay["logits"], cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    ref = oracle_rows(lay, idx_o, g_o)
    got = y_to_f64(y)
    assert np.isfinite(got).all(), f"{name}: non-finite outputs"
    err = rel_l2_rows(got, ref)
    log(f"[activation range] {name}: max rel-L2 {err.max():.3e} (row norms "
        f"{np.linalg.norm(ref, axis=1).min():.1e} .. {np.linalg.norm(ref, axis=1).max():.1e})")
    assert err.max() <= TOL[mode], name
    ex.close()


def test_activation_range_prefill_1k_tiled():
    """The same at the 1,024-token chunk through the benchmark's call form
    (grouping launch writes the scaled copy; tiled weights)."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = CONFIGS[2]
    lay = scaled_rows_layer(cfg, seed=62)
    dev = upload(lay)
    ex = experts_of(lay, dev)
    ex.attach_tiled()
    log("[activation range] prefill 1K tiled")
    idx, gates, y = moe.layer(dev["logits"], dev["x"], ex, cfg.k)
    torch.cuda.synchronize()
    idx_o, g_o = oracle.route(lay["logits"], cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    rows = np.concatenate([np.arange(16), np.random.default_rng(62).choice(cfg.T, 240, replace=False)])
    rows = np.unique(rows).astype(np.int32)
    got = y_to_f64(y)
    assert np.isfinite(got).all()
    err = rel_l2_rows(got[rows], oracle_rows(lay, idx_o, g_o, rows=rows))
    log(f"[activation range] prefill 1K tiled: max rel-L2 {err.max():.3e}")
    assert err.max() <= TOL["fast"]
    ex.close()
