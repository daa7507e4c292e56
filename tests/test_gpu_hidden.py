"""GPU parity of the layer from hidden states (moe_layer_hidden) against the oracle.

The router product and its top-k feed the layer ("Strata - the details", How
it works: each layer's router runs on the GPU in front of its experts):
  * the logits written lie within the rigorous float32 bound of the oracle's
    float64 product, (H + 2) 2^-24 sum_h |x w| (+ 2^-24 |bias|);
  * idx and gates are the top-k of those logits (bit for bit against the
    oracle's top-k of the same logits: an integer decision in the kernel's
    precision);
  * on every token whose k-th and (k+1)-th oracle scores are further apart
    than twice the largest logit error seen, idx equals the oracle's own
    routing of its own logits (the other tokens are near-ties that either
    routing may break either way);
  * y matches the oracle's layer on the oracle's routing.
The one-kernel decode window computes the logits inside the layer's launch;
other shapes launch the router product first.
"""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, make_layer, make_router
from gpu_util import experts_of, log, oracle_rows, rel_l2_rows, torch_cuda, upload, y_to_f64

pytestmark = pytest.mark.gpu

TOL = {"fast": 1e-2, "check": 1e-4}


def _bits_to_f64(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def router_bound(x, w, bias):
    absx = np.abs(_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64))
    absw = np.abs(_bits_to_f64(w))
    H = w.shape[1]
    return (H + 2) * 2.0 ** -24 * (absx @ absw.T) + 2.0 ** -24 * np.abs(bias)[None, :] + 1e-30


def hidden_case(cfg, seed):
    torch = torch_cuda()
    lay = make_layer(cfg, seed=seed)
    w, bias = make_router(cfg, seed)
    dev = upload(lay)
    wt = torch.from_numpy(w.view(np.int16)).cuda()
    bt = torch.from_numpy(bias).cuda()
    return lay, w, bias, dev, wt, bt


def check_hidden(lay, w, bias, idx, gates, y, lg, mode, rows=None, name=""):
    cfg = lay["cfg"]
    k = cfg.k
    lg_np = lg.cpu().numpy()
    ref = oracle.router_logits(lay["x"], w, bias)
    err = np.abs(lg_np.astype(np.float64) - ref)
    bound = router_bound(lay["x"], w, bias)
    log(f"[hidden] {name}: logit error / bound max {np.max(err / bound):.3e}, max abs {err.max():.3e}")
    assert np.all(err <= bound), f"{name}: router error beyond the float32 bound"
    idx_np, g_np = idx.cpu().numpy(), gates.cpu().numpy()
    idx_k, g_k = oracle.route(lg_np, k)
    assert np.array_equal(idx_np, idx_k), f"{name}: idx is not the top-k of the logits written"
    assert np.abs(g_np - g_k).max() <= 1e-6, f"{name}: gates"
    idx_o, g_o = oracle.route(ref.astype(np.float32), k)
    srt = -np.sort(-ref, axis=1)
    margin = srt[:, k - 1] - (srt[:, k] if k < cfg.E else -np.inf)
    clear = margin > 2 * err.max() + 1e-30
    assert clear.mean() > 0.9, f"{name}: too many near-ties to judge ({clear.mean():.2f})"
    assert np.array_equal(idx_np[clear], idx_o[clear]), f"{name}: routing differs from the oracle's"
    if rows is None:
        rows = np.arange(cfg.T, dtype=np.int32)
    rows = rows[clear[rows]]
    got = y_to_f64(y)
    assert np.isfinite(got).all(), f"{name}: non-finite outputs"
    e = rel_l2_rows(got[rows], oracle_rows(lay, idx_o, g_o, rows=rows))
    log(f"[hidden] {name}: {int(clear.sum())} of {cfg.T} tokens clear of near-ties; "
        f"max rel-L2 {e.max():.3e} over {len(rows)} rows")
    assert e.max() <= TOL[mode], name


@pytest.mark.parametrize("name,cid,kw,mode", [
    ("window T=4", 1, {}, "fast"),
    ("window T=1", 1, dict(T=1), "fast"),
    ("window T=3 f32", 1, dict(T=3, xdtype="f32"), "fast"),
    ("window Q3", 1, dict(qtype=3), "fast"),
    ("window H=1024 I=256 E=64 k=4", 1, dict(H=1024, I=256, E=64, k=4), "fast"),
    ("window E=200", 1, dict(E=200), "fast"),
    ("two-kernel window k=20", 1, dict(k=20), "fast"),
    ("check T=4", 1, {}, "check"),
    ("batched Q3 T=64", 4, {}, "fast"),
    ("prefill 1K", 2, {}, "fast"),
    ("prefill T=300 (ragged)", 2, dict(T=300), "fast"),
    ("check T=300", 2, dict(T=300), "check"),
])
def test_layer_hidden(name, cid, kw, mode):
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = CONFIGS[cid].with_(**kw)
    lay, w, bias, dev, wt, bt = hidden_case(cfg, seed=81)
    ex = experts_of(lay, dev)
    if cfg.T >= 1024:
        ex.attach_tiled()
    log(f"[hidden] {name} mode={mode}")
    idx, gates, y, lg = moe.layer_hidden(dev["x"], wt, bt, ex, cfg.k, mode=mode)
    idx2, gates2, y2, lg2 = moe.layer_hidden(dev["x"], wt, bt, ex, cfg.k, mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(lg, lg2) and torch.equal(idx, idx2), f"{name}: not reproducible"
    assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y,
                       y2.view(torch.int16) if y2.dtype == torch.bfloat16 else y2), name
    rows = None
    if cfg.T > 256:
        rng = np.random.default_rng(81)
        rows = np.unique(np.concatenate([np.arange(16), rng.choice(cfg.T, 240, replace=False)]))
        rows = rows.astype(np.int32)
    check_hidden(lay, w, bias, idx, gates, y, lg, mode, rows=rows, name=name)
    ex.close()


def test_layer_hidden_shares_workspace_with_layer():
    """Window calls from hidden states and from logits alternate on one
    workspace: every call equals the same call on a fresh workspace (the
    router counters and the window's other counters stay in step)."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = CONFIGS[1]
    lay, w, bias, dev, wt, bt = hidden_case(cfg, seed=82)
    ex = experts_of(lay, dev)
    L = moe.lib()
    n = max(int(L.moe_layer_hidden_workspace_size(ex.handle, cfg.T, cfg.k, 0)),
            int(L.moe_layer_workspace_size(ex.handle, cfg.T, cfg.k, 0)))
    y_h = moe.layer_hidden(dev["x"], wt, bt, ex, cfg.k,
                           workspace=torch.zeros(n, dtype=torch.uint8, device="cuda"))[2]
    lg_ref = moe.router_logits(dev["x"], wt, bt)
    y_l = moe.layer(lg_ref, dev["x"], ex, cfg.k,
                    workspace=torch.zeros(n, dtype=torch.uint8, device="cuda"))[2]
    torch.cuda.synchronize()
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for i, form in enumerate(["hidden", "logits", "hidden", "hidden", "logits", "hidden"]):
        log(f"[hidden] shared workspace call {i}: from {form}")
        if form == "hidden":
            y = moe.layer_hidden(dev["x"], wt, bt, ex, cfg.k, workspace=ws)[2]
            ref = y_h
        else:
            y = moe.layer(lg_ref, dev["x"], ex, cfg.k, workspace=ws)[2]
            ref = y_l
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"call {i} ({form})"
        assert int(ws[:128].count_nonzero()) == 0
    ex.close()


def test_layer_hidden_timeouts_leave_consistent_head():
    """A one-tick bound on the waits (written from the host into the head's
    spin word) makes the workgroups give up on the router roles and on the
    gate/up roles; rows that did are NaN, idx stays in range. With the bound
    cleared, the next calls on the same workspace equal a fresh workspace's."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = CONFIGS[1]
    lay, w, bias, dev, wt, bt = hidden_case(cfg, seed=83)
    ex = experts_of(lay, dev)
    n = int(moe.lib().moe_layer_hidden_workspace_size(ex.handle, cfg.T, cfg.k, 0))
    y_ref = moe.layer_hidden(dev["x"], wt, bt, ex, cfg.k,
                             workspace=torch.zeros(n, dtype=torch.uint8, device="cuda"))[2]
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    ws[128:132] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8)
    for rep in range(2):
        log(f"[hidden timeouts] forced timeouts, call {rep}")
        idx_to, _, y_to, _ = moe.layer_hidden(dev["x"], wt, bt, ex, cfg.k, workspace=ws)
        torch.cuda.synchronize()
        assert int(idx_to.min()) >= 0 and int(idx_to.max()) < cfg.E
        log(f"[hidden timeouts] NaN rows: {int(torch.isnan(y_to.float()).any(dim=1).sum())} of {cfg.T}")
    ws[128:132] = 0
    for rep in range(3):
        log(f"[hidden timeouts] bound cleared, call {rep}")
        idx, gates, y, lg = moe.layer_hidden(dev["x"], wt, bt, ex, cfg.k, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    check_hidden(lay, w, bias, idx, gates, y, lg, "fast", name="after timeouts")
    ex.close()
