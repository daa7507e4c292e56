"""GPU parity of the router product (moe_router_logits) against the oracle.

Logits are floating point: each entry is checked against the float64 oracle
within the rigorous bound of a float32 sum of H exact products (plus one
rounding per product for float32 activations), (H + 2) * 2^-24 * sum_h |x w|.
Selection is an integer decision taken on the kernel's own logits, so the
top-k of the GPU logits must equal the oracle's top-k of the same logits
bit for bit.
"""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, make_router, make_x
from gpu_util import log, torch_cuda

pytestmark = pytest.mark.gpu


def run_router(cfg, seed, T=None, E=None):
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    if T is not None:
        cfg = cfg.with_(T=T)
    if E is not None:
        cfg = cfg.with_(E=E)
    w, bias = make_router(cfg, seed)
    x = make_x(cfg, seed)
    xt = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()
    if x.dtype == np.uint16:
        xt = xt.view(torch.bfloat16)
    wt = torch.from_numpy(w.view(np.int16)).cuda()
    bt = torch.from_numpy(bias).cuda()
    log(f"[router] cfg{cfg.cid} T={cfg.T} H={cfg.H} E={cfg.E} x={x.dtype}")
    got = moe.router_logits(xt, wt, bt)
    again = moe.router_logits(xt, wt, bt)
    torch.cuda.synchronize()
    got_np = got.cpu().numpy()
    assert np.array_equal(got_np, again.cpu().numpy()), "router logits must be reproducible"
    ref = oracle.router_logits(x, w, bias)
    absx = np.abs((x.astype(np.uint32) << 16).view(np.float32) if x.dtype == np.uint16 else x).astype(np.float64)
    absw = np.abs((w.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    bound = (cfg.H + 2) * 2.0 ** -24 * (absx @ absw.T) + 2.0 ** -24 * np.abs(bias)[None, :] + 1e-30
    err = np.abs(got_np.astype(np.float64) - ref)
    log(f"[router] max err / bound {np.max(err / bound):.3e}, max abs err {err.max():.3e}")
    assert np.all(err <= bound), f"router error beyond the float32 bound: {np.max(err / bound):.3f}"
    return cfg, got, got_np


@pytest.mark.parametrize("cid,T,E", [(0, None, None), (1, None, None), (4, None, None),
                                     (2, None, None), (2, 1000, None), (2, 300, 100),
                                     (3, None, None)])
def test_router_parity(cid, T, E):
    cfg, got, got_np = run_router(CONFIGS[cid], seed=31, T=T, E=E)
    import bit_quantized_moe_topk_amd as moe
    idx, gates = moe.route_topk(got, cfg.k)
    idx_o, gates_o = oracle.route(got_np, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    assert np.max(np.abs(gates.cpu().numpy() - gates_o)) <= 1e-6


@pytest.mark.parametrize("cid,T,E,k", [(3, None, None, None), (2, 300, None, None), (2, 512, 256, 8),
                                       (2, 33, None, 64)])
def test_router_topk_fused(cid, T, E, k):
    """moe_router_topk: the logits within the float32 bound of the oracle's
    product, idx and gates exactly the top-k of the logits written, and equal
    to the separate router + top-k calls' logits within the same bound."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = CONFIGS[cid]
    if T is not None:
        cfg = cfg.with_(T=T)
    if E is not None:
        cfg = cfg.with_(E=E)
    if k is not None:
        cfg = cfg.with_(k=k)
    w, bias = make_router(cfg, 32)
    x = make_x(cfg, 32)
    xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    wt = torch.from_numpy(w.view(np.int16)).cuda()
    bt = torch.from_numpy(bias).cuda()
    log(f"[router_topk] cfg{cfg.cid} T={cfg.T} E={cfg.E} k={cfg.k}")
    idx, gates, lg = moe.router_topk(xt, wt, bt, cfg.k)
    idx2, gates2, lg2 = moe.router_topk(xt, wt, bt, cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(lg, lg2) and torch.equal(idx, idx2), "not reproducible"
    got = lg.cpu().numpy()
    ref = oracle.router_logits(x, w, bias)
    absx = np.abs((x.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    absw = np.abs((w.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    bound = (cfg.H + 2) * 2.0 ** -24 * (absx @ absw.T) + 2.0 ** -24 * np.abs(bias)[None, :] + 1e-30
    err = np.abs(got.astype(np.float64) - ref)
    log(f"[router_topk] max err / bound {np.max(err / bound):.3e}")
    assert np.all(err <= bound)
    idx_o, gates_o = oracle.route(got, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    assert np.max(np.abs(gates.cpu().numpy() - gates_o)) <= 1e-6
