"""A stack of distinct layers captured once in a HIP graph and replayed.

Several decode steps of a model are one pass over its MoE layers; a graph
holds that pass as launches whose arguments never change ("Strata – the
details", How it works: drafts are checked by one pass over all 48 layers;
"strata-dualgpu (oss)", What changed: the draft chain sits in one CUDA graph).
The layers here are distinct seeded instances (weights, logits and x of their
own) that share one workspace, as the layers of a model would: four 4-token
decode windows (2-bit), one 64-token batched layer (3-bit, grouped path) and a
window that starts from hidden states (router product inside its launch).

Each replay must give exactly the eager results, and those the oracle's, with
eager calls on the same workspace and the outputs overwritten in between (so
a replay that wrote nothing, or left the window counters inconsistent for the
next call, fails).
"""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, make_layer, make_router
from gpu_util import experts_of, log, oracle_rows, rel_l2_rows, torch_cuda, upload, y_to_f64

pytestmark = pytest.mark.gpu

TOL_FAST = 1e-2


def _stack():
    specs = [(CONFIGS[1], 0), (CONFIGS[1], 1), (CONFIGS[1], 2), (CONFIGS[4], 3), (CONFIGS[1], 4),
             (CONFIGS[1], 5)]
    lays = [make_layer(cfg, seed=71, layer=i) for cfg, i in specs]
    w, bias = make_router(CONFIGS[1], 71, 5)   # the last layer starts from hidden states
    lays[-1] = dict(lays[-1], router=(w, bias))
    return lays


def test_graph_replay_of_distinct_layers():
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    lays = _stack()
    devs = [upload(l) for l in lays]
    exs = [experts_of(l, d) for l, d in zip(lays, devs)]
    L = moe.lib()
    ws_n = max(max(int(L.moe_layer_workspace_size(ex.handle, l["cfg"].T, l["cfg"].k, 0)),
                   int(L.moe_layer_hidden_workspace_size(ex.handle, l["cfg"].T, l["cfg"].k, 0)))
               for l, ex in zip(lays, exs))
    routers = [None if "router" not in l else
               (torch.from_numpy(l["router"][0].view(np.int16)).cuda(),
                torch.from_numpy(l["router"][1]).cuda(),
                torch.empty((l["cfg"].T, l["cfg"].E), dtype=torch.float32, device="cuda"))
               for l in lays]
    ws = torch.zeros(ws_n, dtype=torch.uint8, device="cuda")
    outs = []
    for l, d in zip(lays, devs):
        cfg = l["cfg"]
        outs.append((torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda"),
                     torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda"),
                     torch.empty((cfg.T, cfg.H), dtype=d["x"].dtype, device="cuda")))

    def run_all():
        for l, d, ex, o, r in zip(lays, devs, exs, outs, routers):
            if r is None:
                moe.layer(d["logits"], d["x"], ex, l["cfg"].k, workspace=ws, out=o)
            else:
                moe.layer_hidden(d["x"], r[0], r[1], ex, l["cfg"].k, workspace=ws, out=o, logits=r[2])

    log("[graph] eager pass over the stack")
    run_all()
    torch.cuda.synchronize()
    eager = [tuple(t.clone() for t in o) for o in outs]

    # the eager results meet the oracle
    for n, (l, e) in enumerate(zip(lays, eager)):
        cfg = l["cfg"]
        if "router" in l:   # routed on the oracle's own router product (no near-ties here)
            lg = oracle.router_logits(l["x"], *l["router"]).astype(np.float32)
        else:
            lg = l["logits"]
        idx_o, g_o = oracle.route(lg, cfg.k)
        assert np.array_equal(e[0].cpu().numpy(), idx_o), f"layer {n}"
        assert np.abs(e[1].cpu().numpy() - g_o).max() <= 1e-5, f"layer {n}"
        err = rel_l2_rows(y_to_f64(e[2]), oracle_rows(l, idx_o, g_o))
        log(f"[graph] layer {n} ({cfg.name}, T={cfg.T}): max rel-L2 {err.max():.3e}")
        assert err.max() <= TOL_FAST, f"layer {n}"

    log("[graph] capture")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    # an extra seeded window, called eagerly on the same workspace between replays
    extra = make_layer(CONFIGS[1], seed=72, layer=0)
    extra_d = upload(extra)
    extra_ex = experts_of(extra, extra_d)
    _, _, y_extra0 = moe.layer(extra_d["logits"], extra_d["x"], extra_ex, CONFIGS[1].k,
                               workspace=ws)
    torch.cuda.synchronize()

    for rep in range(3):
        for o in outs:
            o[0].fill_(-1)
            o[1].fill_(float("nan"))
            o[2].fill_(float("nan"))
        log(f"[graph] replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for n, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o[0], e[0]), f"replay {rep} layer {n}: idx"
            assert torch.equal(o[1], e[1]), f"replay {rep} layer {n}: gates"
            assert torch.equal(o[2].view(torch.int16), e[2].view(torch.int16)), \
                f"replay {rep} layer {n}: y differs from the eager call"
        _, _, y_extra = moe.layer(extra_d["logits"], extra_d["x"], extra_ex, CONFIGS[1].k,
                                  workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y_extra.view(torch.int16), y_extra0.view(torch.int16)), \
            f"eager window after replay {rep}"
    for ex in exs + [extra_ex]:
        ex.close()
