"""GPU parity of the small-batch expert FFN (fewer than 256 tokens, fast mode)
against the float64 oracle (relative L2 per token row within 1e-2), through
the C ABI; two runs must agree bit for bit.

Cases on the small-batch matrix-core kernels cover several 16-token groups
per expert and more than 64 tokens of one expert (h staged in chunks), both
quantisations, H = 1024 / I = 256, float32 activations, no shared expert, a
single token, a ragged batch and more slots than the LDS tables hold; two
shapes outside those kernels run the GEMV kernels (experts with 1..4
assignments) beside the matrix-core tiles. The activation layout of the
small-batch kernels is written in three ways, each checked: by the FFN
call's own grouping launch, by the whole-layer call's routing launch, and by
a separate kernel when the caller brings the grouping.
"""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, make_layer
from gpu_util import experts_of, log, oracle_rows, rel_l2_rows, torch_cuda, upload, y_to_f64

pytestmark = pytest.mark.gpu

TOL_FAST = 1e-2

CASES = [
    ("Q3 T=64 (16 streams x 4)", dict(), None),
    ("Q3 T=200 E=64: many tokens per expert", dict(T=200, E=64), None),
    ("Q2 T=255, every token on expert 5", dict(T=255, E=64, qtype=2), 5),
    ("Q2 H=1024 I=256 T=37 f32", dict(T=37, H=1024, I=256, E=32, k=4, qtype=2, xdtype="f32"), None),
    ("Q3 H=1024 I=512 T=9 no shared", dict(T=9, H=1024, E=48, k=6, shared=0), None),
    ("Q2 T=1", dict(T=1, qtype=2), None),
    ("Q2 E=2048 k=8 T=48: the largest expert map", dict(T=48, E=2048, k=8, qtype=2), None),
    # more than 4,096 assignment slots: token ids and gates read without the LDS tables
    ("Q3 T=100 k=48 E=64: 4,900 slots", dict(T=100, E=64, k=48), None),
    # outside the small-batch kernels' shapes: GEMV for 1..4 assignments, tiles for the rest
    ("Q2 H=4096 I=256 T=20: GEMV + tiles", dict(T=20, H=4096, I=256, E=32, k=4, qtype=2), 3),
    ("Q3 H=512 I=128 T=40: GEMV + tiles", dict(T=40, H=512, I=128, E=24, k=3), None),
]


@pytest.mark.parametrize("name,kw,hot", CASES, ids=[c[0] for c in CASES])
def test_batch_ffn_parity(name, kw, hot):
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = CONFIGS[4].with_(**kw)
    lay = make_layer(cfg, seed=31)
    if hot is not None:
        lg = lay["logits"].copy()
        lg[:, hot] += 100.0
        lay = dict(lay, logits=lg)
    dev = upload(lay)
    ex = experts_of(lay, dev)
    idx_np, gates_np = oracle.route(lay["logits"], cfg.k)
    if hot is not None:
        assert np.all(idx_np[:, 0] == hot)
    log(f"[batch] {name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} Q{cfg.qtype}")
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).cuda()
    gates = torch.from_numpy(np.ascontiguousarray(gates_np, dtype=np.float32)).cuda()
    y1 = moe.ffn_q(dev["x"], ex, idx, gates)
    y2 = moe.ffn_q(dev["x"], ex, idx, gates)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), "two runs differ"
    err = rel_l2_rows(y_to_f64(y1), oracle_rows(lay, idx_np, gates_np))
    log(f"[batch] {name}: max rel-L2 {err.max():.3e}  mean {err.mean():.3e}")
    assert err.max() <= TOL_FAST
    ex.close()


LAYOUT_CASES = [
    ("Q3 T=64 layer", dict(), "layer"),
    ("Q2 T=37 f32 layer", dict(T=37, qtype=2, xdtype="f32"), "layer"),
    ("Q3 T=9 layer (one-workgroup routing: separate layout kernel)", dict(T=9), "layer"),
    ("Q3 T=64 caller grouping", dict(), "grouping"),
    ("Q2 H=1024 I=256 T=20 f32 caller grouping", dict(T=20, H=1024, I=256, E=32, k=4, qtype=2, xdtype="f32"),
     "grouping"),
]


@pytest.mark.parametrize("name,kw,how", LAYOUT_CASES, ids=[c[0] for c in LAYOUT_CASES])
def test_batch_activation_layout_paths(name, kw, how):
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfg = CONFIGS[4].with_(**kw)
    lay = make_layer(cfg, seed=37)
    dev = upload(lay)
    ex = experts_of(lay, dev)
    idx_np, gates_np = oracle.route(lay["logits"], cfg.k)
    log(f"[batch-layout] {name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} Q{cfg.qtype}")
    if how == "layer":
        idx, gates, y = moe.layer(dev["logits"], dev["x"], ex, cfg.k)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), idx_np)
    else:
        idx, gates, grp = moe.route_group(dev["logits"], cfg.k, bool(cfg.shared))
        y = moe.ffn_q(dev["x"], ex, idx, gates, grouping=grp)
        torch.cuda.synchronize()
    err = rel_l2_rows(y_to_f64(y), oracle_rows(lay, idx_np, gates_np))
    log(f"[batch-layout] {name}: max rel-L2 {err.max():.3e}")
    assert err.max() <= TOL_FAST
    ex.close()


def test_batch_layer_workspace_reuse():
    """One workspace through layer calls of different batches, then the first
    again: every call matches the oracle and the repeat is bit-identical
    (nothing of an earlier call's copy, grouping or counters leaks)."""
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    cfgs = [CONFIGS[4], CONFIGS[4].with_(T=37, qtype=3), CONFIGS[4].with_(T=9)]
    lays = [make_layer(c, seed=41 + i) for i, c in enumerate(cfgs)]
    devs = [upload(l) for l in lays]
    exs = [experts_of(l, d) for l, d in zip(lays, devs)]
    nbytes = max(int(moe.lib().moe_layer_workspace_size(ex.handle, c.T, c.k, 0)) for ex, c in zip(exs, cfgs))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    outs = []
    for i in [0, 1, 2, 0]:
        c = cfgs[i]
        log(f"[batch-reuse] call T={c.T} Q{c.qtype}")
        idx, gates, y = moe.layer(devs[i]["logits"], devs[i]["x"], exs[i], c.k, workspace=ws)
        torch.cuda.synchronize()
        idx_np, gates_np = oracle.route(lays[i]["logits"], c.k)
        assert np.array_equal(idx.cpu().numpy(), idx_np)
        err = rel_l2_rows(y_to_f64(y), oracle_rows(lays[i], idx_np, gates_np))
        assert err.max() <= TOL_FAST, (c.T, err.max())
        outs.append(y.clone())
    assert torch.equal(outs[0], outs[3]), "repeat of the first call differs"
    for ex in exs:
        ex.close()
