"""Seeded input generator: determinism, shapes, value recipe."""
import numpy as np

from synth import (CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_layer, make_logits,
                   make_x, plane_sizes, zipf_bias)


def test_same_seed_same_bytes():
    cfg = CONFIGS[0]
    a = make_layer(cfg, seed=3)
    b = make_layer(cfg, seed=3)
    for key in ("logits", "x", "codes", "dm"):
        assert np.array_equal(a[key], b[key])
    c = make_layer(cfg, seed=4)
    assert not np.array_equal(a["codes"], c["codes"])
    assert not np.array_equal(a["logits"], c["logits"])


def test_shapes_and_sizes():
    for cid, cfg in CONFIGS.items():
        ps = plane_sizes(cfg)
        assert ps["blocks"] == 3 * cfg.H * cfg.I // 32
        assert cfg.expert_bytes() == ps["codes"] + 2 * ps["dm"] + ps["hi"]
    # 2-bit codes + fp16 d + fp16 m per 32 weights = 3 bits per weight
    assert CONFIGS[1].expert_bytes() == 1_179_648
    assert CONFIGS[4].expert_bytes() == 1_572_864
    # the 48-layer stack: 24,576 routed experts, about 29 GB of Q2 planes
    c3 = CONFIGS[3]
    routed = c3.layers * c3.E * c3.expert_bytes()
    assert c3.layers * c3.E == 24_576
    assert abs(routed / 1e9 - 28.99) < 0.01


def test_value_recipe_tiny():
    cfg = CONFIGS[0]
    lay = make_layer(cfg, seed=0)
    assert lay["logits"].shape == (cfg.T, cfg.E) and lay["logits"].dtype == np.float32
    assert lay["x"].dtype == np.float32
    dm = lay["dm"].reshape(cfg.E_tot, -1, 2)
    d = dm[..., 0].view(np.float16).astype(np.float64)
    m = dm[..., 1].view(np.float16).astype(np.float64)
    assert (d >= 0).all()
    assert abs(np.sqrt(np.mean(d ** 2)) - 0.02) < 0.002      # |N(0, 0.02)|
    assert np.array_equal(m, (-1.5 * d).astype(np.float16).astype(np.float64))
    # codes are uniform bytes -> each 2-bit code uniform over 0..3
    c = lay["codes"].reshape(-1)
    q = np.concatenate([(c >> s) & 3 for s in (0, 2, 4, 6)])
    frac = np.bincount(q, minlength=4) / q.size
    assert np.all(np.abs(frac - 0.25) < 0.01)


def test_bf16_rounding():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 2 ** -7, 1.0 + 3 * 2 ** -8, -2.5, 0.0],
                 dtype=np.float32)
    b = f32_to_bf16_bits(v)
    back = bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    assert list(back) == [1.0, 1.0, 1.0 + 2 ** -7, 1.0 + 2 ** -6, -2.5, 0.0]


def test_zipf_skew():
    cfg = CONFIGS[2]
    bias = zipf_bias(cfg, seed=0)
    ranks = np.round(np.exp(-bias / 1.1)).astype(int)
    assert sorted(ranks) == list(range(1, cfg.E + 1))
    lg = make_logits(cfg, seed=0)
    top1 = np.argmax(lg, axis=1)
    # the rank-1 expert wins far more often than uniform routing would allow
    assert np.bincount(top1, minlength=cfg.E).max() > 20 * cfg.T / cfg.E


def test_bf16_activations():
    cfg = CONFIGS[1]
    x = make_x(cfg, seed=0)
    assert x.dtype == np.uint16 and x.shape == (cfg.T, cfg.H)
    xf = bf16_bits_to_f32(x)
    assert abs(xf.std() - 1.0) < 0.05


def test_stream_ranking_reading_of_batched_decode():
    """Two readings of the 16-stream batched decode: one Zipf ranking shared by
    every stream (60-75 distinct experts per layer) or a ranking of its own per
    stream (240-270). The second reading changes only the logits' bias rows."""
    import oracle
    shared = CONFIGS[4]
    own = shared.with_(stream_ranking=True)
    d_shared, d_own = [], []
    for layer in range(6):
        a = make_logits(shared, 0, layer)
        b = make_logits(own, 0, layer)
        assert a.shape == b.shape == (64, 512)
        d_shared.append(len(np.unique(oracle.route(a, shared.k)[0])))
        d_own.append(len(np.unique(oracle.route(b, own.k)[0])))
        # rows of one stream share a bias: their differences are bias-free
        assert not np.allclose(b[0] - b[4], a[0] - a[4], atol=1e-3)
        assert np.allclose(b[0] - b[1], a[0] - a[1], atol=1e-4)
    assert 55 <= min(d_shared) and max(d_shared) <= 80, d_shared
    assert 230 <= min(d_own) and max(d_own) <= 280, d_own
