"""GPU parity of the prefill call forms the benchmark times, through the C ABI.

moe_layer in fast mode with the tiled weight copy attached, exactly as the
benchmark calls it: the layer routes, groups (the grouping launch's spare
workgroups write the fp16 activation copy, so the matrix-core tiles skip their
own copy kernel) and runs the FFN. Checked at the 1,024-token chunk and on
every one of the 48 layers of the 8,192-token stack: top-k indices bit-exact,
gates within 1e-6, the grouping arrays bit-exact, and 256 sampled output rows
within relative L2 1e-2 of the float64 oracle (rows are independent per token,
so sampling is exact).
"""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, make_layer
from gpu_util import experts_of, log, oracle_rows, rel_l2_rows, torch_cuda, upload, y_to_f64

pytestmark = pytest.mark.gpu

TOL_FAST = 1e-2
N_ROWS = 256


def layer_bench_form(lay, dev, tiled=True):
    """moe.layer in fast mode with the tiled copy attached (the benchmark's call)."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = lay["cfg"]
    ex = experts_of(lay, dev)
    if tiled:
        ex.attach_tiled()
    idx, gates, y = moe.layer(dev["logits"], dev["x"], ex, cfg.k, mode="fast")
    torch.cuda.synchronize()
    out = (idx.cpu().numpy(), gates.cpu().numpy(), y_to_f64(y))
    ex.close()
    return out


def check_layer(lay, dev, seed, what, tiled=True):
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = lay["cfg"]
    log(f"[prefill layer] {what}: moe_layer fast tiled={tiled} T={cfg.T}")
    idx_g, gates_g, y = layer_bench_form(lay, dev, tiled)
    idx_o, g_o = oracle.route(lay["logits"], cfg.k)
    assert np.array_equal(idx_g, idx_o), f"{what}: top-k differs"
    assert np.max(np.abs(gates_g - g_o)) <= 1e-6, f"{what}: gates differ"
    assert np.isfinite(y).all(), f"{what}: non-finite outputs"
    # the grouping from the same routing kernels the layer runs
    _, _, grp = moe.route_group(dev["logits"], cfg.k, bool(cfg.shared))
    torch.cuda.synchronize()
    ref_g = oracle.group(idx_o, cfg.E, bool(cfg.shared))
    got_g = (grp.counts.cpu().numpy(), grp.offsets.cpu().numpy(), grp.perm.cpu().numpy(),
             grp.slot_of.cpu().numpy())
    for name, a, b in zip(("counts", "offsets", "perm", "slot_of"), got_g, ref_g):
        assert np.array_equal(a, b), f"{what}: grouping {name} differs"
    rows = np.random.default_rng(seed).choice(cfg.T, N_ROWS, replace=False).astype(np.int32)
    err = rel_l2_rows(y[rows], oracle_rows(lay, idx_o, g_o, rows=rows))
    log(f"[prefill layer] {what}: max rel-L2 {err.max():.3e} over {N_ROWS} rows")
    assert err.max() <= TOL_FAST, what


@pytest.mark.parametrize("tiled", [True, False])
def test_layer_call_prefill_1k(tiled):
    """The 1,024-token chunk through moe_layer (the one-workgroup grouping
    launch writes the tiles' activation copy)."""
    lay = make_layer(CONFIGS[2], seed=0)
    check_layer(lay, upload(lay), 1024 + tiled, f"cfg2 tiled={tiled}", tiled)


@pytest.mark.parametrize("layer", range(CONFIGS[3].layers))
def test_layer_call_prefill_8k_every_layer(layer):
    """Every layer of the 48-layer 8,192-token stack through moe_layer with the
    tiled copy (the count launch of the grouping writes the activation copy)."""
    lay = make_layer(CONFIGS[3], seed=0, layer=layer, threads=16)
    check_layer(lay, upload(lay), 8192 + layer, f"cfg3 layer {layer}")
