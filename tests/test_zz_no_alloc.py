"""The allocation-free layer entry point (moe_layer_static) against moe_layer.

moe_layer_static runs the layer on the library's own per-GPU scratch array
instead of a caller's workspace. Called through the C ABI twice in a row, the
second call with a smaller input (a 64-token batch, then a 4-token decode
window, which uses the counters at the head of the array), each result must
equal moe_layer's on the same inputs: top-k indices and gates identically,
outputs within the fast-mode tolerance (both calls run the same kernels, so
they are in fact expected to be bit-identical), and the oracle's bar too.
"""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, make_layer
from gpu_util import experts_of, log, oracle_rows, rel_l2_rows, torch_cuda, upload, y_to_f64

pytestmark = pytest.mark.gpu

TOL_FAST = 1e-2


def test_layer_static_matches_layer():
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    base = CONFIGS[1].with_(T=64)
    lay = make_layer(base, seed=71)
    for T in (64, 4):  # the second call has the smaller input
        cfg = base.with_(T=T)
        sub = dict(lay, cfg=cfg, x=lay["x"][:T].copy(), logits=lay["logits"][:T].copy())
        dev = upload(sub)
        ex = experts_of(sub, dev)
        log(f"[layer_static] T={T}")
        idx_s, g_s, y_s = moe.layer_static(dev["logits"], dev["x"], ex, cfg.k)
        torch.cuda.synchronize()
        idx_l, g_l, y_l = moe.layer(dev["logits"], dev["x"], ex, cfg.k)
        torch.cuda.synchronize()
        assert torch.equal(idx_s, idx_l) and torch.equal(g_s, g_l), f"T={T}: routing differs"
        err = rel_l2_rows(y_to_f64(y_s), y_to_f64(y_l))
        same = torch.equal(y_s, y_l)
        log(f"[layer_static] T={T}: rel-L2 to moe_layer {err.max():.2e}, bit-identical={same}")
        assert err.max() <= TOL_FAST
        idx_o, g_o = oracle.route(sub["logits"], cfg.k)
        assert np.array_equal(idx_s.cpu().numpy(), idx_o)
        assert rel_l2_rows(y_to_f64(y_s), oracle_rows(sub, idx_o, g_o)).max() <= TOL_FAST
        ex.close()


def test_layer_static_rejects_large_inputs():
    """Past its scratch size the entry point returns MOE_ERR_WORKSPACE and
    launches nothing."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    import ctypes as C
    cfg = CONFIGS[2]
    lay = make_layer(cfg, seed=72)
    dev = upload(lay)
    ex = experts_of(lay, dev)
    need = int(moe.lib().moe_layer_workspace_size(ex.handle, cfg.T, cfg.k, moe.FAST))
    assert need > (16 << 20)
    y = torch.full((cfg.T, cfg.H), 7.0, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    gates = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    P = lambda t: C.c_void_p(t.data_ptr())  # noqa: E731
    st = moe.lib().moe_layer_static(P(dev["logits"]), P(dev["x"]), moe.BF16, cfg.T, ex.handle,
                                    cfg.k, P(idx), P(gates), P(y), moe.FAST,
                                    C.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == moe.ERR_WORKSPACE
    assert bool((y.float() == 7.0).all())
    ex.close()
