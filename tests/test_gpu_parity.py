"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Bars: top-k indices and every grouping array bit-exact; gates within 1e-6
absolute; FFN output rows within relative L2 1e-4 (fp32 check mode) and 1e-2
(fast mode) of the float64 oracle. Inputs are the seeded synthetic layers.
"""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, make_layer, make_logits
from gpu_util import (experts_of, log, oracle_rows, rel_l2_rows, torch_cuda, upload, y_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    torch_cuda()

TOL_CHECK = 1e-4
TOL_FAST = 1e-2

_cache = {}


def layer_for(cid, seed=0, layer=0):
    key = (cid, seed, layer)
    if key not in _cache:
        lay = make_layer(CONFIGS[cid], seed=seed, layer=layer)
        _cache[key] = (lay, upload(lay))
    return _cache[key]


def gpu_route(logits_np, k):
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    idx, gates = moe.route_topk(torch.from_numpy(np.ascontiguousarray(logits_np)).cuda(), k)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), gates.cpu().numpy()


def check_route(logits_np, k, what):
    log(f"[route] {what} T={logits_np.shape[0]} E={logits_np.shape[1]} k={k}")
    idx_o, g_o = oracle.route(logits_np, k)
    idx_g, g_g = gpu_route(logits_np, k)
    assert np.array_equal(idx_g, idx_o), what
    assert np.max(np.abs(g_g - g_o), initial=0.0) <= 1e-6, what


@pytest.mark.parametrize("cid", [0, 1, 2, 4])
def test_route_bit_exact(cid):
    cfg = CONFIGS[cid]
    check_route(make_logits(cfg, seed=0), cfg.k, f"cfg{cid}")


def test_route_prefill_8k_all_layers():
    cfg = CONFIGS[3]
    for layer in range(cfg.layers):
        check_route(make_logits(cfg, seed=0, layer=layer), cfg.k, f"cfg3 layer {layer}")


def test_route_adversarial():
    rng = np.random.default_rng(7)
    check_route(rng.integers(0, 4, size=(300, 64)).astype(np.float32), 10, "ties")
    check_route(np.full((17, 16), 0.5, np.float32), 16, "all equal, k=E")
    check_route(np.full((3, 16), -2.0, np.float32), 1, "all equal, k=1")
    lg = np.array([[-0.0, 0.0, np.nan, -1.0, np.nan, 0.5, -np.inf, 3e38]], np.float32)
    idx_o, _ = oracle.route(lg, 8)
    idx_g, _ = gpu_route(lg, 8)
    assert np.array_equal(idx_g, idx_o)
    check_route(rng.standard_normal((9, 2048)).astype(np.float32), 64, "E=2048 k=64")
    check_route(rng.standard_normal((5, 1)).astype(np.float32), 1, "E=1")
    check_route(rng.standard_normal((1, 700)).astype(np.float32), 700, "k=E=700")


def gpu_group(idx_np, E, shared):
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    g = moe.group(torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).cuda(), E, shared)
    torch.cuda.synchronize()
    return (g.counts.cpu().numpy(), g.offsets.cpu().numpy(), g.perm.cpu().numpy(),
            g.slot_of.cpu().numpy())


def check_group(idx_np, E, shared, what):
    log(f"[group] {what} T={idx_np.shape[0]} k={idx_np.shape[1]} E={E} shared={shared}")
    ref = oracle.group(idx_np, E, shared)
    got = gpu_group(idx_np, E, shared)
    for name, a, b in zip(("counts", "offsets", "perm", "slot_of"), got, ref):
        assert np.array_equal(a, b), f"{what}: {name} differs"


@pytest.mark.parametrize("cid", [0, 1, 2, 3, 4])
def test_group_bit_exact(cid):
    cfg = CONFIGS[cid]
    idx, _ = oracle.route(make_logits(cfg, seed=0), cfg.k)
    check_group(idx, cfg.E, bool(cfg.shared), f"cfg{cid}")


def test_group_edges():
    rng = np.random.default_rng(3)
    check_group(np.tile(np.array([5, 0, 2], np.int32), (5000, 1)), 8, True, "one expert per slot")
    check_group(rng.integers(0, 64, size=(20000, 10)).astype(np.int32), 64, False, "T=20000 E=64")
    check_group(rng.integers(0, 2048, size=(3000, 7)).astype(np.int32), 2048, True, "E=2048")
    check_group(np.zeros((1, 1), np.int32), 1, False, "T=1 E=1")
    check_group(rng.integers(0, 3, size=(1700, 2)).astype(np.int32), 3, True, "E=3 ragged")


@pytest.mark.parametrize("cid,T", [(0, 8), (1, 4), (4, 64), (1, 1), (2, 1024), (0, 3)])
def test_route_group_fused_bit_exact(cid, T):
    """The one-call route + group (single workgroup for small batches) equals
    the oracle's top-k followed by its grouping."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = CONFIGS[cid].with_(T=T)
    lg = make_logits(CONFIGS[cid], seed=3)[:T].copy()
    log(f"[route_group] cfg{cid} T={T}")
    idx, gates, g = moe.route_group(torch.from_numpy(lg).cuda(), cfg.k, bool(cfg.shared))
    torch.cuda.synchronize()
    idx_o, g_o = oracle.route(lg, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    assert np.max(np.abs(gates.cpu().numpy() - g_o)) <= 1e-6
    ref = oracle.group(idx_o, cfg.E, bool(cfg.shared))
    got = (g.counts.cpu().numpy(), g.offsets.cpu().numpy(), g.perm.cpu().numpy(),
           g.slot_of.cpu().numpy())
    for name, a, b in zip(("counts", "offsets", "perm", "slot_of"), got, ref):
        assert np.array_equal(a, b), name


@pytest.mark.parametrize("cid,T,mode", [(1, 4, "fast"), (1, 1, "fast"), (1, 3, "fast"),
                                         (4, 4, "fast"), (4, 2, "fast"), (0, 4, "fast"),
                                         (0, 8, "fast"), (4, 64, "fast"), (1, 4, "check")])
def test_layer_call(cid, T, mode):
    """moe_layer (whole layer in one call; the one-kernel window path for T <= 4
    in fast mode at the decode shapes, the two-kernel one at the tiny shape)
    against the oracle's route, grouping and layer."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    base = CONFIGS[cid]
    lay = make_layer(base, seed=21)
    cfg = base.with_(T=T)
    lay = dict(lay, cfg=cfg, x=lay["x"][:T].copy(), logits=lay["logits"][:T].copy())
    dev = upload(lay)
    ex = experts_of(lay, dev)
    log(f"[layer call] cfg{cid} T={T} mode={mode}")
    idx, gates, y = moe.layer(dev["logits"], dev["x"], ex, cfg.k, mode=mode)
    torch.cuda.synchronize()
    idx_o, g_o = oracle.route(lay["logits"], cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    assert np.max(np.abs(gates.cpu().numpy() - g_o)) <= 1e-6
    ref = oracle_rows(lay, idx_o, g_o)
    err = rel_l2_rows(y_to_f64(y), ref)
    log(f"[layer call] cfg{cid} T={T} {mode}: max rel-L2 {err.max():.3e}")
    assert err.max() <= (TOL_CHECK if mode == "check" else TOL_FAST)
    y2 = moe.layer(dev["logits"], dev["x"], ex, cfg.k, mode=mode)[2]
    torch.cuda.synchronize()
    if mode == "fast" and T <= 4:
        assert torch.equal(y, y2), "window path must be reproducible run to run"
    ex.close()


@pytest.mark.parametrize("name,kw", [("f32 activations", dict(xdtype="f32")),
                                     ("k=14: 60 rows of h", dict(k=14)),
                                     ("k=16: 64 assignments, two-kernel window", dict(k=16)),
                                     ("k=20: two-kernel window", dict(k=20)),
                                     ("H=4096, I=256", dict(H=4096, I=256, E=16, k=2)),
                                     ("Q3, H=1024", dict(qtype=3, H=1024, E=64, k=4))])
def test_layer_window_variants(name, kw):
    """The decode window at the config-1 shapes with float32 activations, near
    the one-kernel form's limit (its down roles hold every routed (expert,
    token) row of h in 64 KB of LDS: 63 rows at I = 512, so T k + T <= 63 with
    the shared expert) and past it (the two-kernel form at H = 2048), and at
    the one-kernel form's other shapes (H = 4096 with I = 256; Q3 at
    H = 1024), against the oracle."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = CONFIGS[1].with_(**kw)
    lay = make_layer(cfg, seed=23)
    dev = upload(lay)
    ex = experts_of(lay, dev)
    log(f"[window variant] {name}")
    idx, gates, y = moe.layer(dev["logits"], dev["x"], ex, cfg.k)
    torch.cuda.synchronize()
    idx_o, g_o = oracle.route(lay["logits"], cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    err = rel_l2_rows(y_to_f64(y), oracle_rows(lay, idx_o, g_o))
    log(f"[window variant] {name}: max rel-L2 {err.max():.3e}")
    assert err.max() <= TOL_FAST
    ex.close()


def test_layer_window_65_active_experts():
    """A one-kernel window at I = 256 whose four tokens pick 16 distinct
    experts each (64 routed + the shared expert = 65 active): the down roles
    hold 64 experts' weights in registers at a time, so the 65th comes from a
    second chunk of weight requests after the first chunk's products; against
    the oracle."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = CONFIGS[1].with_(I=256, k=16)
    lay = make_layer(cfg, seed=27)
    lg = lay["logits"].copy()
    for t in range(cfg.T):  # token t's top 16: experts 16 t + 100 .. 16 t + 115
        lg[t, 100 + 16 * t:116 + 16 * t] = 40.0 + np.arange(16, dtype=np.float32) * 0.25
    lay = dict(lay, logits=lg)
    dev = upload(lay)
    ex = experts_of(lay, dev)
    log("[window 65 experts] I=256 k=16")
    idx, gates, y = moe.layer(dev["logits"], dev["x"], ex, cfg.k)
    torch.cuda.synchronize()
    idx_o, g_o = oracle.route(lg, cfg.k)
    assert len(set(idx_o.ravel().tolist())) == 64
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    err = rel_l2_rows(y_to_f64(y), oracle_rows(lay, idx_o, g_o))
    log(f"[window 65 experts] max rel-L2 {err.max():.3e}")
    assert err.max() <= TOL_FAST
    ex.close()


def test_layer_window_shared_workspace():
    """One zero-filled workspace serves window calls of two layer instances,
    repeated, with a 64-token call of the same experts in between: the
    one-kernel window's counters at the head of the workspace carry over from
    call to call (they count over all calls; every result stays exact), the
    guard word stays zero, and the other call form leaves the head alone."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    base = CONFIGS[1].with_(T=64)
    lays = [make_layer(base, seed=s) for s in (41, 42)]
    devs = [upload(l) for l in lays]
    exs = [experts_of(l, d) for l, d in zip(lays, devs)]
    k = base.k
    nbytes = max(int(moe.lib().moe_layer_workspace_size(exs[0].handle, T, k, 0)) for T in (4, 64))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    refs = []
    for lay in lays:
        idx_o, g_o = oracle.route(lay["logits"][:4], k)
        win = dict(lay, cfg=base.with_(T=4), x=lay["x"][:4].copy(), logits=lay["logits"][:4].copy())
        refs.append((idx_o, g_o, oracle_rows(win, idx_o, g_o)))
    for rep in range(3):
        for i, (dev, ex) in enumerate(zip(devs, exs)):
            log(f"[shared ws] rep {rep} instance {i}: window")
            idx, gates, y = moe.layer(dev["logits"][:4], dev["x"][:4], ex, k, workspace=ws)
            torch.cuda.synchronize()
            idx_o, g_o, ref = refs[i]
            assert np.array_equal(idx.cpu().numpy(), idx_o)
            assert rel_l2_rows(y_to_f64(y), ref).max() <= TOL_FAST
            assert int(ws[:128].count_nonzero()) == 0
        log(f"[shared ws] rep {rep}: 64-token call")
        head = ws[:8192].clone()
        moe.layer(devs[rep % 2]["logits"], devs[rep % 2]["x"], exs[rep % 2], k, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ws[:8192], head)
    for ex in exs:
        ex.close()


def test_layer_window_unzeroed_head_gives_nan():
    """A workspace whose head was not zeroed (the never-written guard word is
    set from the host) makes the one-kernel window write NaN rows at once,
    without waiting on any counter; zeroing the head restores exact results."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = CONFIGS[1]
    lay = make_layer(cfg, seed=43)
    dev = upload(lay)
    ex = experts_of(lay, dev)
    nbytes = int(moe.lib().moe_layer_workspace_size(ex.handle, cfg.T, cfg.k, 0))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    y_ok = moe.layer(dev["logits"], dev["x"], ex, cfg.k, workspace=ws)[2]
    ws[:4] = 7  # the guard word
    log("[window guard] head not zero")
    y_bad = moe.layer(dev["logits"], dev["x"], ex, cfg.k, workspace=ws)[2]
    torch.cuda.synchronize()
    assert bool(torch.isnan(y_bad.float()).all())
    ws.zero_()
    y_again = moe.layer(dev["logits"], dev["x"], ex, cfg.k, workspace=ws)[2]
    torch.cuda.synchronize()
    assert torch.equal(y_ok, y_again)
    ex.close()


def test_layer_window_workspace_across_shapes():
    """One zero-filled workspace through one-kernel windows of different layer
    shapes (config 1: I = 512, 16 gate/up groups, 8 down groups; H = 4096,
    I = 256: 8 gate/up groups, 16 down groups; Q3 at H = 1024) and back, each
    result against the oracle: the head's counters do not depend on the
    shape."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    shapes = [CONFIGS[1], CONFIGS[1].with_(H=4096, I=256, E=16, k=2), CONFIGS[1].with_(qtype=3, H=1024, E=64, k=4)]
    lays = [make_layer(c, seed=45 + i) for i, c in enumerate(shapes)]
    devs = [upload(l) for l in lays]
    exs = [experts_of(l, d) for l, d in zip(lays, devs)]
    nbytes = max(int(moe.lib().moe_layer_workspace_size(e.handle, c.T, c.k, 0)) for e, c in zip(exs, shapes))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for i in (0, 1, 2, 0, 2, 1, 0):
        cfg, lay, dev, ex = shapes[i], lays[i], devs[i], exs[i]
        log(f"[ws across shapes] H={cfg.H} I={cfg.I} Q{cfg.qtype}")
        idx, gates, y = moe.layer(dev["logits"], dev["x"], ex, cfg.k, workspace=ws)
        torch.cuda.synchronize()
        idx_o, g_o = oracle.route(lay["logits"], cfg.k)
        assert np.array_equal(idx.cpu().numpy(), idx_o)
        assert rel_l2_rows(y_to_f64(y), oracle_rows(lay, idx_o, g_o)).max() <= TOL_FAST
    for ex in exs:
        ex.close()


def test_layer_window_timeouts_leave_consistent_head():
    """Waits that time out leave the head consistent for the next call. A
    bound of one wall-clock tick on the down roles' wait, written from the host
    into the head's spin word, makes them give up (their rows become NaN)
    while the gate/up roles still finish; with the bound cleared, the next
    calls on the same workspace are exact and equal to the result on a fresh
    workspace. Every kernel ends normally on either path."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = CONFIGS[1]
    lay = make_layer(cfg, seed=44)
    dev = upload(lay)
    ex = experts_of(lay, dev)
    nbytes = int(moe.lib().moe_layer_workspace_size(ex.handle, cfg.T, cfg.k, 0))
    fresh = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    y_ref = moe.layer(dev["logits"], dev["x"], ex, cfg.k, workspace=fresh)[2]
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ws[128:132] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8)  # spin bound: 1 tick
    for rep in range(2):
        log(f"[window timeouts] forced timeouts, call {rep}")
        y_to = moe.layer(dev["logits"], dev["x"], ex, cfg.k, workspace=ws)[2]
        torch.cuda.synchronize()
        log(f"[window timeouts] NaN rows: {int(torch.isnan(y_to.float()).any(dim=1).sum())} of {cfg.T}")
    ws[128:132] = 0
    idx_o, g_o = oracle.route(lay["logits"], cfg.k)
    ref = oracle_rows(lay, idx_o, g_o)
    for rep in range(3):
        log(f"[window timeouts] bound cleared, call {rep}")
        y = moe.layer(dev["logits"], dev["x"], ex, cfg.k, workspace=ws)[2]
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
        assert rel_l2_rows(y_to_f64(y), ref).max() <= TOL_FAST
    ex.close()


def run_ffn(lay, dev, idx_np, gates_np, mode, use_gpu_grouping=False, tiled=False):
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = lay["cfg"]
    ex = experts_of(lay, dev)
    if tiled:
        ex.attach_tiled()
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).cuda()
    gates = torch.from_numpy(np.ascontiguousarray(gates_np, dtype=np.float32)).cuda()
    grp = moe.group(idx, cfg.E, bool(cfg.shared)) if use_gpu_grouping else None
    y = moe.ffn_q(dev["x"], ex, idx, gates, grouping=grp, mode=mode)
    torch.cuda.synchronize()
    out = y_to_f64(y)
    ex.close()
    return out


@pytest.mark.parametrize("mode,tol", [("check", TOL_CHECK), ("fast", TOL_FAST)])
@pytest.mark.parametrize("cid", [0, 1, 4, 2])
def test_ffn_parity(cid, mode, tol):
    lay, dev = layer_for(cid)
    cfg = lay["cfg"]
    idx, gates = oracle.route(lay["logits"], cfg.k)
    log(f"[ffn] cfg{cid} mode={mode} T={cfg.T}")
    y = run_ffn(lay, dev, idx, gates, mode, use_gpu_grouping=(cid % 2 == 0))
    ref = oracle_rows(lay, idx, gates)
    err = rel_l2_rows(y, ref)
    log(f"[ffn] cfg{cid} {mode}: max rel-L2 {err.max():.3e}  p99 {np.percentile(err, 99):.3e}  "
        f"mean {err.mean():.3e}")
    assert err.max() <= tol


@pytest.mark.parametrize("cid", [2, 4])
def test_ffn_parity_tiled_weights(cid):
    """Matrix-core tiles reading the tiled weight copy: oracle tolerance, and
    agreement with the canonical-plane path up to fp32 summation order."""
    lay, dev = layer_for(cid)
    cfg = lay["cfg"]
    idx, gates = oracle.route(lay["logits"], cfg.k)
    log(f"[ffn] cfg{cid} tiled weights T={cfg.T}")
    y_t = run_ffn(lay, dev, idx, gates, "fast", use_gpu_grouping=True, tiled=True)
    y_c = run_ffn(lay, dev, idx, gates, "fast", use_gpu_grouping=True, tiled=False)
    ref = oracle_rows(lay, idx, gates)
    err = rel_l2_rows(y_t, ref)
    log(f"[ffn] cfg{cid} tiled: max rel-L2 {err.max():.3e}; vs canonical "
        f"{rel_l2_rows(y_t, y_c).max():.3e}")
    assert err.max() <= TOL_FAST
    assert rel_l2_rows(y_t, y_c).max() <= 5e-3


@pytest.mark.parametrize("cid", [0, 1, 4])
def test_layer_end_to_end(cid):
    """route -> group -> ffn all on the GPU, against the oracle's own route."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    lay, dev = layer_for(cid)
    cfg = lay["cfg"]
    log(f"[layer] cfg{cid}")
    idx, gates = moe.route_topk(dev["logits"], cfg.k)
    grp = moe.group(idx, cfg.E, bool(cfg.shared))
    ex = experts_of(lay, dev)
    y = moe.ffn_q(dev["x"], ex, idx, gates, grouping=grp, mode="fast")
    torch.cuda.synchronize()
    idx_o, g_o = oracle.route(lay["logits"], cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    ref = oracle_rows(lay, idx_o, g_o)
    assert rel_l2_rows(y_to_f64(y), ref).max() <= TOL_FAST
    ex.close()


@pytest.mark.parametrize("layer", [0, 47])
def test_prefill_8k_sampled_rows(layer):
    """Full-size 8,192-token layer of the 48-layer stack; 256 sampled rows checked."""
    lay, dev = make_layer(CONFIGS[3], seed=0, layer=layer), None
    dev = upload(lay)
    cfg = lay["cfg"]
    idx, gates = oracle.route(lay["logits"], cfg.k)
    rows = np.random.default_rng(layer).choice(cfg.T, 256, replace=False).astype(np.int32)
    ref = oracle_rows(lay, idx, gates, rows=rows)
    for mode, tol, tiled in (("fast", TOL_FAST, False), ("fast", TOL_FAST, True),
                             ("check", TOL_CHECK, False)):
        log(f"[ffn] cfg3 layer {layer} mode={mode} tiled={tiled}")
        y = run_ffn(lay, dev, idx, gates, mode, use_gpu_grouping=True, tiled=tiled)
        err = rel_l2_rows(y[rows], ref)
        log(f"[ffn] cfg3 layer {layer} {mode} tiled={tiled}: max rel-L2 {err.max():.3e}")
        assert err.max() <= tol


@pytest.mark.parametrize("T,E,k", [(16, 512, 64), (12, 2048, 40), (9, 64, 7)])
def test_route_group_segments_bit_exact(T, E, k):
    """The one-workgroup route + group with several grouping segments (up to
    one per wave, fewer where the per-segment bases would overflow LDS), and
    the two-launch form past 16 tokens, equal the oracle."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    rng = np.random.default_rng(T * 1000 + k)
    for TT in (T, 4 * T):
        lg = rng.standard_normal((TT, E)).astype(np.float32)
        lg[:, :3] += 2.0  # a few hot experts: long runs inside segments
        log(f"[route_group segments] T={TT} E={E} k={k}")
        idx, gates, g = moe.route_group(torch.from_numpy(lg).cuda(), k, True)
        torch.cuda.synchronize()
        idx_o, _ = oracle.route(lg, k)
        assert np.array_equal(idx.cpu().numpy(), idx_o)
        ref = oracle.group(idx_o, E, True)
        got = (g.counts.cpu().numpy(), g.offsets.cpu().numpy(), g.perm.cpu().numpy(),
               g.slot_of.cpu().numpy())
        for name, a, b in zip(("counts", "offsets", "perm", "slot_of"), got, ref):
            assert np.array_equal(a, b), name


def test_group_size_invariance():
    """A token evaluated alone and inside its verify window agree within tolerance."""
    lay, dev = layer_for(1)
    cfg = lay["cfg"]
    idx, gates = oracle.route(lay["logits"], cfg.k)
    full = run_ffn(lay, dev, idx, gates, "fast")
    for t in range(cfg.T):
        one = dict(lay, cfg=cfg.with_(T=1), x=lay["x"][t:t + 1], logits=lay["logits"][t:t + 1])
        d1 = upload(one)
        y1 = run_ffn(one, d1, idx[t:t + 1], gates[t:t + 1], "fast")
        err = rel_l2_rows(y1, full[t:t + 1])[0]
        log(f"[invariance] token {t}: rel-L2 alone vs batch {err:.2e} "
            f"bitwise={'yes' if np.array_equal(y1, full[t:t + 1]) else 'no'}")
        assert err <= TOL_FAST


def test_edge_all_tokens_one_expert_and_k_equals_E():
    cfg = CONFIGS[0].with_(T=200)
    lay = make_layer(cfg, seed=4)
    dev = upload(lay)
    # every token picks expert 3 first (MFMA tiles, ragged tail of 200 = 3*64 + 8)
    lg = lay["logits"].copy()
    lg[:, 3] += 100.0
    idx, gates = oracle.route(lg, cfg.k)
    assert np.all(idx[:, 0] == 3)
    for mode, tol in (("fast", TOL_FAST), ("check", TOL_CHECK)):
        y = run_ffn(lay, dev, idx, gates, mode, use_gpu_grouping=True)
        assert rel_l2_rows(y, oracle_rows(lay, idx, gates)).max() <= tol
    # k = E: every expert holds every token
    cfg16 = CONFIGS[0].with_(k=16)
    lay16 = dict(make_layer(CONFIGS[0], seed=5), cfg=cfg16)
    dev16 = upload(lay16)
    idx, gates = oracle.route(lay16["logits"], 16)
    for mode, tol in (("fast", TOL_FAST), ("check", TOL_CHECK)):
        y = run_ffn(lay16, dev16, idx, gates, mode)
        assert rel_l2_rows(y, oracle_rows(lay16, idx, gates)).max() <= tol


def test_edge_zero_and_max_scales():
    """d = 0 blocks (w = m), and all-3 codes with the largest generated scales."""
    lay = make_layer(CONFIGS[0], seed=6)
    dm = lay["dm"].reshape(lay["dm"].shape[0], -1, 2).copy()
    dm[:, ::3, 0] = 0                        # every third block has d = 0
    codes = lay["codes"].copy()
    codes[:, 1::5] = 0xFF                    # some bytes hold the largest code
    lay = dict(lay, dm=dm.reshape(lay["dm"].shape), codes=codes)
    dev = upload(lay)
    idx, gates = oracle.route(lay["logits"], CONFIGS[0].k)
    for mode, tol in (("fast", TOL_FAST), ("check", TOL_CHECK)):
        y = run_ffn(lay, dev, idx, gates, mode)
        assert rel_l2_rows(y, oracle_rows(lay, idx, gates)).max() <= tol


def test_edge_empty_batch():
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    lay, dev = layer_for(0)
    cfg = lay["cfg"]
    idx, gates = moe.route_topk(dev["logits"][:0], cfg.k)
    assert idx.shape == (0, cfg.k)
    ex = experts_of(lay, dev)
    y = moe.ffn_q(dev["x"][:0], ex, idx, gates)
    torch.cuda.synchronize()
    assert y.shape == (0, cfg.H)
    ex.close()
