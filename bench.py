#!/usr/bin/env python3
"""Benchmark of the routed MoE layer over 2-bit block-quantized experts (one MI355X).

A step is one pass of the whole hot path over one batch: top-k routing, the
grouping of assignments by expert, and the expert FFN with combine (dequant,
gate/up, SwiGLU, down, gate-weighted sum, shared expert).

Default run (prints ONE JSON line):
  * decode: the 4-token verify-window layer (hidden 2048, 512 routed experts + 1
    shared, top-10, intermediate 512, Q2) over a stack of --rotation (48)
    distinct seeded layers, each with its own weights, logits and x (the layers
    are not chained: with these weight scales a chained y would fade to zero
    within a few layers), so the touched weights cannot stay in the 256 MB
    last-level cache between visits. One HIP graph holds a whole pass over the
    stack and is replayed. `value` is tokens/s of one layer step; "stack"
    gives the pass over all layers (end-to-end tokens/s of the decode window).
  * batched decode (16 streams x 4 tokens, Q3) under both readings of its
    logits: one Zipf ranking shared by the streams, and one per stream.
  * prefill: the 8,192-token chunk through the 48-layer stack (24,576 routed
    experts, ~29 GB of Q2 planes resident in HBM), and the 1,024-token chunk
    over 8 distinct layers; per-layer and end-to-end tokens/s.
  * roofline: the dominant kernel of each regime, timed with HIP events around
    its launches (an eager pass over the same steps), against MI355X's
    published peaks and against measured ones (a streaming copy and a loop of
    matrix-core products).
  * cpu_baseline: the CPU oracle on the decode steps, on all the host cores
    this process may use and on one core, plus the other workloads (configs in
    full, or bounded row samples scaled up where a full run would take minutes,
    each labelled).

Inputs are synthetic and seeded (package ``synth``); nothing is read from disk.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS_F16 = 2500.0  # MI355X dense fp16/bf16 matrix peak, published

SEPARATE_CALLS = False  # --separate-calls: moe_route_topk + moe_group instead of moe_route_group
LAYER_CALL = True       # decode steps call moe_layer (--stage-calls: route_group + ffn_q)

METRIC = "MoE-layer tokens/s (4-tok decode, 8K prefill); HBM GB/s and MFMA % of peak"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def expert_plane_bytes(cfg) -> dict:
    """Bytes of one expert's gate+up planes and of its down planes."""
    bits = 4 if cfg.qtype == 3 else 3   # code bits + 32 bits of (d, m) per 32 weights
    mat = cfg.H * cfg.I * bits // 8
    return {"gateup": 2 * mat, "down": mat}


class LayerInstance:
    """Device buffers and prebuilt C-ABI argument lists for one layer step."""

    def __init__(self, cfg, host: dict, ws_bytes_fn, router=None):
        import torch
        import bit_quantized_moe_topk_amd as moe
        self.cfg = cfg
        dev = "cuda"
        self.hidden = router is not None   # steps start from hidden states (moe_layer_hidden)
        if self.hidden:
            self.rw = torch.from_numpy(router[0].view(np.int16)).to(dev)
            self.rb = torch.from_numpy(router[1]).to(dev)
        self.logits = torch.from_numpy(host["logits"]).to(dev)
        x = torch.from_numpy(np.ascontiguousarray(host["x"]))
        if host["x"].dtype == np.uint16:
            x = x.view(torch.int16).view(torch.bfloat16)
        self.x = x.to(dev)
        self.codes = torch.from_numpy(host["codes"].reshape(-1)).to(dev)
        self.dm = torch.from_numpy(host["dm"].reshape(-1).view(np.int16)).to(dev)
        self.hi = None if host["hi"] is None else torch.from_numpy(host["hi"].reshape(-1)).to(dev)
        self.ex = moe.Experts(cfg.qtype, cfg.E, bool(cfg.shared), cfg.H, cfg.I, self.codes,
                              self.hi, self.dm)
        T, k, E = cfg.T, cfg.k, cfg.E
        A = T * (k + cfg.shared)
        i32 = torch.int32
        self.idx = torch.empty((T, k), dtype=i32, device=dev)
        self.gates = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E + 1, dtype=i32, device=dev)
        self.offsets = torch.empty(E + 2, dtype=i32, device=dev)
        self.perm = torch.empty(A, dtype=i32, device=dev)
        self.slot_of = torch.empty(A, dtype=i32, device=dev)
        self.y = torch.empty((T, cfg.H), dtype=self.x.dtype, device=dev)

    def bind(self, gws, fws, lws):
        """Fix the argument tuples for the three C-ABI calls (shared workspaces)."""
        P = lambda t: C.c_void_p(t.data_ptr())  # noqa: E731
        cfg = self.cfg
        xdt = 0 if self.x.dtype.is_floating_point and self.x.element_size() == 4 else 1
        self.a_route = (P(self.logits), cfg.T, cfg.E, cfg.k, P(self.idx), P(self.gates))
        self.a_route_group = (P(self.logits), cfg.T, cfg.E, cfg.k, cfg.shared, P(self.idx),
                              P(self.gates), P(self.counts), P(self.offsets), P(self.perm),
                              P(self.slot_of), P(gws) if gws is not None else None,
                              0 if gws is None else gws.numel())
        self.a_group = (P(self.idx), cfg.T, cfg.k, cfg.E, cfg.shared, P(self.counts),
                        P(self.offsets), P(self.perm), P(self.slot_of),
                        P(gws) if gws is not None else None, 0 if gws is None else gws.numel())
        self.a_layer = (P(self.logits), P(self.x), xdt, cfg.T, self.ex.handle, cfg.k, P(self.idx),
                        P(self.gates), P(self.y), 0, P(lws), lws.numel())
        if self.hidden:  # the router's logits land in the instance's logits buffer
            self.a_hidden = (P(self.x), xdt, cfg.T, P(self.rw), P(self.rb), self.ex.handle, cfg.k,
                             P(self.idx), P(self.gates), P(self.y), P(self.logits), 0, P(lws),
                             lws.numel())
        self.a_ffn = (P(self.x), xdt, cfg.T, self.ex.handle, P(self.idx), P(self.gates), cfg.k,
                      P(self.counts), P(self.offsets), P(self.perm), P(self.slot_of), P(self.y),
                      0, P(fws), fws.numel())

    def step(self, L, stream) -> None:
        if self.hidden:
            st = L.moe_layer_hidden(*self.a_hidden, stream)
            if st:
                raise RuntimeError(f"moe_layer_hidden failed: {st}")
            return
        if LAYER_CALL:
            st = L.moe_layer(*self.a_layer, stream)
            if st:
                raise RuntimeError(f"moe_layer failed: {st}")
            return
        if SEPARATE_CALLS:
            r = L.moe_route_topk(*self.a_route, stream)
            g = L.moe_group(*self.a_group, stream)
        else:
            r = 0
            g = L.moe_route_group(*self.a_route_group, stream)
        f = L.moe_ffn_q(*self.a_ffn, stream)
        if r or g or f:
            raise RuntimeError(f"C-ABI call failed: route={r} group={g} ffn={f}")


def build_instances(cfg, n: int, seed: int, keep_host: int = 0, hidden: bool = False):
    import torch
    import bit_quantized_moe_topk_amd as moe
    from synth import make_layer, make_router
    insts, hosts = [], []
    t0 = time.time()
    for i in range(n):
        host = make_layer(cfg, seed=seed, layer=i, threads=16)
        router = make_router(cfg, seed, layer=i) if hidden else None
        insts.append(LayerInstance(cfg, host, None, router))
        if i < keep_host:
            hosts.append(host)
        del host
    torch.cuda.synchronize()
    log(f"{cfg.name}: generated and uploaded {n} layer instances in {time.time() - t0:.1f}s")
    L = moe.lib()
    gws_n = L.moe_group_workspace_size(cfg.T, cfg.k, cfg.E)
    gws = torch.empty(gws_n, dtype=torch.uint8, device="cuda") if gws_n else None
    fws_n = insts[0].ex.workspace_size(cfg.T, cfg.k, 0)
    fws = torch.empty(fws_n, dtype=torch.uint8, device="cuda")
    lws_n = L.moe_layer_workspace_size(insts[0].ex.handle, cfg.T, cfg.k, 0)
    if hidden:
        lws_n = max(lws_n, L.moe_layer_hidden_workspace_size(insts[0].ex.handle, cfg.T, cfg.k, 0))
    lws = torch.zeros(lws_n, dtype=torch.uint8, device="cuda")  # head: window counters
    for it in insts:
        it.bind(gws, fws, lws)
    return insts, hosts, (gws, fws, lws)


def routing_stats(insts) -> list:
    """Per instance (from the idx the step wrote): experts on the GEMV path
    (1..4 assignments, batches under 256 tokens only), on the MFMA path, and
    the assignments on the MFMA path."""
    out = []
    for it in insts:
        cfg = it.cfg
        c = np.bincount(it.idx.cpu().numpy().reshape(-1), minlength=cfg.E).astype(np.int64)
        if cfg.shared:
            c = np.append(c, cfg.T)
        gmax = 4 if cfg.T < 256 else 0
        gemv = int(((c >= 1) & (c <= gmax)).sum())
        mf = c > gmax
        out.append({"gemv_experts": gemv, "mfma_experts": int(mf.sum()),
                    "mfma_assignments": int(c[mf].sum()), "touched": int((c > 0).sum())})
    return out


def gpu_hold(ms: float) -> None:
    """Keep the GPU busy for about `ms` so that launches queued meanwhile run
    back to back (their HIP events then time the GPU, not the host)."""
    import torch
    torch.cuda._sleep(int(ms * 1e-3 * 2.4e9))


def kernel_source_hash() -> str:
    """Digest of the HIP sources (a byte-counter summary is valid only for them)."""
    import hashlib
    d = os.path.join(ROOT, "bit_quantized_moe_topk_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 byte-counter summary, or
    None when there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel source hash") != kernel_source_hash():
        return None
    try:
        return int(vals["traffic bytes per launch"].replace(",", ""))
    except (KeyError, ValueError):
        return None


def kernel_profile(insts, L, stream, steps: int, chunk: int = 32) -> dict:
    import torch
    import bit_quantized_moe_topk_amd as moe
    torch.cuda.synchronize()
    moe.profile_begin(64 * steps + 64)
    for c0 in range(0, steps, chunk):
        gpu_hold(25.0)
        for s in range(c0, min(steps, c0 + chunk)):
            insts[s % len(insts)].step(L, stream)
    torch.cuda.synchronize()
    return moe.profile_end()


def run_decode(cfg, args, workload: str = "decode", hidden: bool = False):
    """Time K layer steps over a rotation of distinct layer instances (from
    logits, or from hidden states with the router product in the step)."""
    import torch
    import bit_quantized_moe_topk_amd as moe
    L = moe.lib()
    insts, hosts, keep = build_instances(cfg, args.rotation, args.seed, keep_host=args.cpu_layers,
                                         hidden=hidden)
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    for s in range(max(args.warmup, len(insts))):   # every instance runs once untimed
        insts[s % len(insts)].step(L, stream)
    torch.cuda.synchronize()
    stats = routing_stats(insts)

    K = args.steps
    n = len(insts)
    graphs = None
    if not args.eager:
        # one graph holds a full pass over the rotation; a second one the first
        # K mod n steps, so exactly K steps run in the timed region
        def capture(count):
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    cur = C.c_void_p(torch.cuda.current_stream().cuda_stream)
                    for s in range(count):
                        insts[s].step(L, cur)
            torch.cuda.current_stream().wait_stream(side)
            return g
        graphs = (capture(n), capture(K % n) if K % n else None)
        for g in graphs:
            if g is not None:
                g.replay()
        torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    if graphs is not None:
        for _ in range(K // n):
            graphs[0].replay()
        if graphs[1] is not None:
            graphs[1].replay()
    else:
        for s in range(K):
            insts[s % n].step(L, stream)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    ms_per_step = ms / K

    # eager pass with HIP events around every launch: per-kernel durations
    prof = kernel_profile(insts, L, stream, K)
    pb = expert_plane_bytes(cfg)
    step_layers = [stats[s % len(insts)] for s in range(K)]
    kname = max((k for k in prof
                 if k in ("win_layer", "win_layer_rt", "win_gateup", "gemv_gateup", "win_down",
                          "gemv_down", "bat_gateup", "bat_down")),
                key=lambda k: prof[k][1], default="")
    if not kname:
        raise RuntimeError(f"no decode expert kernel in the profile: {sorted(prof)}")
    if kname.startswith("win_layer"):  # the whole window in one kernel: gate/up and down planes
        unit = pb["gateup"] + pb["down"]
    else:
        unit = pb["gateup"] if "gateup" in kname else pb["down"]
    per_step_units = [st["touched"] if kname.startswith(("win", "bat")) else st["gemv_experts"]
                      for st in step_layers]
    k_bytes = sum(per_step_units) * unit
    if kname == "win_layer_rt":  # the router rows (bf16 [E][H]) are read in the same launch
        k_bytes += K * cfg.E * cfg.H * 2
    n_k, k_ms = prof[kname]
    touched_bytes = np.mean([st["touched"] for st in stats]) * (pb["gateup"] + pb["down"])
    kernels_us = {k: round(1e3 * v[1] / max(v[0], 1), 2) for k, v in prof.items()}
    res = {
        "tokens_per_s": cfg.T / (ms_per_step / 1e3),
        "ms_per_step": ms_per_step,
        "graph": graphs is not None,
        "kernels_us": kernels_us,
        "touched_experts_mean": float(np.mean([st["touched"] for st in stats])),
        "layer_weight_bytes_mean": float(touched_bytes),
        "layer_hbm_gbs": float(touched_bytes / (ms_per_step * 1e-3) / 1e9),
        "stack": {
            "layers": n,
            "us_per_pass": round(ms_per_step * n * 1e3, 2),
            "tokens_per_s_end_to_end": round(cfg.T / (ms_per_step * n * 1e-3), 1),
        },
        "roofline": {
            "kernel": kname,
            "bound": "hbm",
            "achieved": round(k_bytes / (k_ms * 1e-3) / 1e9, 1) if k_ms else None,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(k_bytes / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if k_ms else None,
            "traffic": measured_traffic(kname, workload),
            "launches": n_k,
            "avg_us": round(1e3 * k_ms / max(n_k, 1), 2),
            "bytes_per_launch": round(k_bytes / max(n_k, 1)),
            "unit_bytes": unit,
        },
    }
    del graphs
    return res, hosts, insts


def router_timing(args, reps: int = 50) -> dict:
    """The router product in front of the layer (moe_router_logits), timed
    with kernel-attached events at the decode window and the 8K chunk: not
    part of the layer step above, which starts from logits."""
    import torch
    import bit_quantized_moe_topk_amd as moe
    from synth import CONFIGS, make_router, make_x
    out = {}
    for name, cfg in (("decode_t4", CONFIGS[1]), ("prefill_t8192", CONFIGS[3])):
        w, bias = make_router(cfg, args.seed)
        x = torch.from_numpy(make_x(cfg, args.seed).view(np.int16)).cuda().view(torch.bfloat16)
        wt = torch.from_numpy(w.view(np.int16)).cuda()
        bt = torch.from_numpy(bias).cuda()
        for _ in range(3):
            moe.router_logits(x, wt, bt)
        torch.cuda.synchronize()
        moe.profile_begin(4 * reps)
        gpu_hold(5.0)
        for _ in range(reps):
            moe.router_logits(x, wt, bt)
        torch.cuda.synchronize()
        prof = moe.profile_end()
        kname, (n, ms) = max(prof.items(), key=lambda kv: kv[1][1])
        us = 1e3 * ms / max(n, 1)
        flops = 2.0 * cfg.T * cfg.H * cfg.E
        out[name] = {"kernel": kname, "us": round(us, 2), "router_bytes": cfg.E * cfg.H * 2,
                     "GB_s": round(cfg.E * cfg.H * 2 / (us * 1e-6) / 1e9, 1),
                     "TFLOP_s": round(flops / (us * 1e-6) / 1e12, 2)}
        if cfg.T >= 256:  # router product + top-k: one launch, against the two kernels
            for _ in range(3):
                moe.router_topk(x, wt, bt, cfg.k)
                moe.route_topk(moe.router_logits(x, wt, bt), cfg.k)
            torch.cuda.synchronize()
            moe.profile_begin(8 * reps)
            gpu_hold(5.0)
            for _ in range(reps):
                moe.router_topk(x, wt, bt, cfg.k)
            for _ in range(reps):
                moe.route_topk(moe.router_logits(x, wt, bt), cfg.k)
            torch.cuda.synchronize()
            prof = moe.profile_end()
            per = {kk: round(1e3 * v[1] / max(v[0], 1), 2) for kk, v in prof.items()}
            out[name]["fused_router_topk_us"] = per.get("router_topk")
            out[name]["separate_kernels_us"] = round(per.get("router_mfma", 0) + per.get("topk", 0), 2)
    return out


def run_prefill(cfg, args, n_layers: int, K: int, workload: str):
    """K passes over a stack of n_layers distinct layers of one prefill chunk."""
    import torch
    import bit_quantized_moe_topk_amd as moe
    L = moe.lib()
    insts, _, keep = build_instances(cfg, n_layers, args.seed)
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if not args.no_tiled:  # weight copy in the matrix-core tile order, built at load time
        t0 = time.time()
        for it in insts:
            it.ex.attach_tiled()
        torch.cuda.synchronize()
        log(f"prefill: tiled weight copies for {n_layers} layers in {time.time() - t0:.1f}s")
    for it in insts:           # warm-up: the whole stack once
        it.step(L, stream)
    torch.cuda.synchronize()
    stats = routing_stats(insts)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(K):
        for it in insts:
            it.step(L, stream)
    ev1.record()
    torch.cuda.synchronize()
    ms_stack = ev0.elapsed_time(ev1) / K
    prof = kernel_profile(insts, L, stream, len(insts))
    n_gu, gu_ms = prof.get("mfma_gateup", (0, 0.0))
    flops_gu = sum(2.0 * 2 * cfg.I * cfg.H * st["mfma_assignments"] for st in stats)
    total_flops = sum(2.0 * 3 * cfg.I * cfg.H * cfg.A for _ in stats)
    ms_layer = ms_stack / n_layers
    res = {
        "workload": f"prefill: {cfg.T}-token chunk through {n_layers} distinct MoE layers "
                    f"(hidden {cfg.H}, {cfg.E} routed + {cfg.shared} shared experts, top-{cfg.k}, "
                    f"intermediate {cfg.I}, Q{cfg.qtype}, bf16 activations)",
        "layers": n_layers,
        "weights": "canonical planes" if args.no_tiled else "canonical planes + tiled copy",
        "ms_per_chunk": ms_stack,
        "ms_per_layer": ms_layer,
        "tokens_per_s_end_to_end": cfg.T / (ms_stack * 1e-3),
        "tokens_per_s_per_layer": cfg.T / (ms_layer * 1e-3),
        "layer_tflops": total_flops / len(stats) / (ms_layer * 1e-3) / 1e12,
        "kernels_us": {k: round(1e3 * v[1] / max(v[0], 1), 1) for k, v in prof.items()},
        "roofline": {
            "kernel": "mfma_gateup",
            "bound": "mfma",
            "achieved": round(flops_gu / (gu_ms * 1e-3) / 1e12, 2) if gu_ms else None,
            "peak": MFMA_PEAK_TFLOPS_F16,
            "unit": "TFLOP/s",
            "frac": round(flops_gu / (gu_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS_F16, 4) if gu_ms else None,
            "traffic": measured_traffic("mfma_gateup", workload),
            "launches": n_gu,
            "avg_us": round(1e3 * gu_ms / max(n_gu, 1), 1),
            "flops_per_launch": flops_gu / max(n_gu, 1),
        },
    }
    for it in insts:
        it.ex.close()
    del insts, keep
    torch.cuda.empty_cache()
    return res


def fp8_variant(args, reps: int = 10) -> dict:
    """One expert's gate/up + SwiGLU over the 8,192-token chunk on the FP8
    matrix cores (moe_expert_gateup_fp8: operand preparation + the product
    kernel), beside the layer's fp16 tiles on the same work (moe_ffn_q with
    every token routed to that one expert; its gate/up kernel)."""
    import torch
    import bit_quantized_moe_topk_amd as moe
    from synth import CONFIGS
    from synth.gen import make_expert_planes, make_x
    cfg = CONFIGS[3]
    codes, hi, dm = make_expert_planes(cfg, args.seed, 0, cfg.E)  # the shared expert of layer 0
    dev = "cuda"
    ct = torch.from_numpy(np.ascontiguousarray(codes)).to(dev)
    ht = None if hi is None else torch.from_numpy(np.ascontiguousarray(hi)).to(dev)
    dt = torch.from_numpy(np.ascontiguousarray(dm).view(np.int16)).to(dev)
    ex = moe.Experts(cfg.qtype, 1, False, cfg.H, cfg.I, ct, ht, dt)
    x = torch.from_numpy(make_x(cfg, args.seed, 0).view(np.int16)).to(dev).view(torch.bfloat16)
    T = cfg.T
    idx = torch.zeros((T, 1), dtype=torch.int32, device=dev)
    gates = torch.ones((T, 1), dtype=torch.float32, device=dev)
    ws = torch.empty(int(moe.lib().moe_expert_gateup_fp8_workspace_size(ex.handle, T)),
                     dtype=torch.uint8, device=dev)
    moe.expert_gateup_fp8(x, ex, 0, workspace=ws)
    moe.ffn_q(x, ex, idx, gates, mode="fast")
    torch.cuda.synchronize()
    moe.profile_begin(64 * reps)
    gpu_hold(5.0)
    for _ in range(reps):
        moe.expert_gateup_fp8(x, ex, 0, workspace=ws)
    torch.cuda.synchronize()
    gpu_hold(5.0)
    for _ in range(reps):
        moe.ffn_q(x, ex, idx, gates, mode="fast")
    torch.cuda.synchronize()
    prof = moe.profile_end()
    ex.close()
    us = {k: round(1e3 * v[1] / max(v[0], 1), 1) for k, v in prof.items()}
    flops = 2.0 * 2 * cfg.I * cfg.H * T
    tf = lambda k: round(flops / (us[k] * 1e-6) / 1e12, 1) if us.get(k) else None  # noqa: E731
    return {
        "workload": f"gate/up + SwiGLU of one Q{cfg.qtype} expert (hidden {cfg.H}, intermediate "
                    f"{cfg.I}) over {T} tokens: {flops / 1e9:.1f} GFLOP",
        "kernels_us": us,
        "fp8_gateup_TFLOP_s": tf("fp8_gateup"),
        "fp16_tiles_gateup_TFLOP_s": tf("mfma_gateup"),
        "fp8_with_operand_prep_us": round(sum(us.get(k, 0.0) for k in ("fp8_codes", "fp8_x", "fp8_gateup")), 1),
        "accuracy": "per-row rel-L2 of h against the float64 oracle ~1e-5 (tests/test_gpu_fp8.py); "
                    "the fp16 tiles ~3e-3",
    }


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_share() -> int:
    """Host cores this process may use (at most 16, the CPU share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_step(host, cfg, threads: int, rows=None) -> None:
    """One layer step of the CPU oracle: top-k, grouping, expert FFN + combine
    (fp32 build, OpenMP over tokens)."""
    import oracle
    idx, gates = oracle.route(host["logits"], cfg.k)
    oracle.group(idx, cfg.E, bool(cfg.shared))
    oracle.layer_rows(host, idx, gates, rows=rows, prec="f32", threads=threads)


def time_oracle(hosts, cfg, threads: int, seconds: float, rows=None, max_steps: int = 1000):
    """Whole oracle steps (or steps over `rows` only) until `seconds` have passed
    (at least one): (steps, seconds, tokens per step)."""
    steps, t0 = 0, time.perf_counter()
    while True:
        oracle_step(hosts[steps % len(hosts)], cfg, threads, rows)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds or steps >= max_steps:
            break
    return steps, el, (cfg.T if rows is None else len(rows))


def cpu_baseline(cfg, hosts, args):
    """The CPU oracle on the decode steps (all cores, one core) and on the other
    workloads; configs in full unless a full run would take minutes (then a row
    sample, scaled and labelled)."""
    from synth import CONFIGS, make_layer
    share = cpu_share()
    used = lambda c: max(1, min(share, c.T))  # noqa: E731  (the oracle threads over tokens)
    out_cfgs = {}

    def record(name, c, threads, steps, el, tok, note):
        out_cfgs.setdefault(name, {})["1 core" if threads == 1 else "all cores"] = {
            "tokens_per_s": round(steps * tok / el, 3), "threads": threads,
            "sample": f"{steps} step(s) of {tok} token rows, {el:.1f}s wall; {note}"}

    steps, el, tok = time_oracle(hosts, cfg, used(cfg), args.cpu_seconds)
    head = {"value": round(steps * tok / el, 2), "unit": "tokens/s", "cores": used(cfg),
            "kind": "oracle",
            "sample": f"{steps} full decode layer steps ({cfg.T} tokens each) over {len(hosts)} "
                      f"seeded layer instances, fp32 oracle, {el:.1f}s wall; the oracle "
                      f"parallelises over the {cfg.T} tokens only"}
    s1, el1, tok1 = time_oracle(hosts, cfg, 1, args.cpu_seconds / 2)
    head["single_core"] = {"value": round(s1 * tok1 / el1, 3), "unit": "tokens/s", "cores": 1,
                           "sample": f"{s1} full decode layer steps, {el1:.1f}s wall"}
    head["cpu_model"] = cpu_model()
    head["host_cores_available"] = share

    full = args.cpu_full
    for cid in (0, 4, 2):
        c = CONFIGS[cid]
        h = [make_layer(c, seed=args.seed, layer=0, threads=share)]
        all_core_s = 0.0
        for threads in (used(c), 1):
            rows, note = None, "full layer step"
            # one core runs the whole step unless that projects to over a minute
            if threads == 1 and not full and all_core_s * used(c) > 60.0:
                rows = np.arange(128, dtype=np.int32)
                note = (f"rows 0..127 of the {c.T}-token step (a full step projects to "
                        f"{all_core_s * used(c):.0f}s on one core)")
            secs = 1.0 if cid == 0 else 0.0
            steps, el, tok = time_oracle(h, c, threads, secs, rows=rows)
            if threads > 1:
                all_core_s = el / steps
            record(c.name, c, threads, steps, el, tok, note)
        del h
    # one layer of the 8K chunk, extrapolated to the 48-layer stack
    c = CONFIGS[3]
    h = [make_layer(c, seed=args.seed, layer=0, threads=share)]
    n_rows = c.T if full else 2048
    rows = np.arange(n_rows, dtype=np.int32)
    steps, el, tok = time_oracle(h, c, used(c), 0.0, rows=rows)
    layer_s = el / steps * c.T / n_rows
    out_cfgs[c.name] = {"all cores": {
        "tokens_per_s_extrapolated": round(c.T / (layer_s * c.layers), 4),
        "threads": used(c), "layer_seconds_extrapolated": round(layer_s, 2),
        "sample": f"EXTRAPOLATED: {n_rows} of {c.T} token rows of one layer in {el:.1f}s, "
                  f"scaled to the whole chunk and x{c.layers} layers"}}
    del h
    head["configs"] = out_cfgs
    return head


def measured_peaks(reps: int = 5) -> dict:
    """Measured ceilings: a streaming copy (torch's copy kernel, bytes read +
    written) and the matrix-core loop of libmoe_peaks.so (bf16 and fp16
    operands), each timed with events on the stream it runs on."""
    import torch
    path = os.path.join(ROOT, "bit_quantized_moe_topk_amd", "libmoe_peaks.so")
    if not os.path.exists(path):
        raise RuntimeError("libmoe_peaks.so is not built (python -m bit_quantized_moe_topk_amd.build)")
    P = C.CDLL(path)
    P.peaks_mfma_loop.argtypes = [C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    P.peaks_mfma_loop_flops.argtypes = [C.c_int, C.c_int]
    P.peaks_mfma_loop_flops.restype = C.c_double
    P.peaks_mfma_loop_fp8_flops.argtypes = [C.c_int, C.c_int]
    P.peaks_mfma_loop_fp8_flops.restype = C.c_double
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 2 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(reps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * n * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del src, dst
    blocks, iters = 2048, 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {"copy_GBps": round(copy_gbs, 1), "copy_bytes": f"{reps} copies of 2 GiB, read + write"}
    for bf, name in ((1, "bf16"), (0, "f16"), (2, "fp8")):
        if P.peaks_mfma_loop(bf, blocks, iters, C.c_void_p(out.data_ptr()), stream):
            raise RuntimeError("peaks_mfma_loop failed")
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(reps):
            P.peaks_mfma_loop(bf, blocks, iters, C.c_void_p(out.data_ptr()), stream)
        ev1.record()
        torch.cuda.synchronize()
        fl = (P.peaks_mfma_loop_fp8_flops if bf == 2 else P.peaks_mfma_loop_flops)(blocks, iters) * reps
        res[f"mfma_loop_{name}_TFLOPs"] = round(fl / (ev0.elapsed_time(ev1) * 1e-3) / 1e12, 1)
    res["mfma_loop"] = (f"{blocks} workgroups x 4 waves, {iters} rounds of 8 independent "
                        "32x32x16 (bf16, f16) or 32x32x64 (fp8) products on register operands")
    return res


def with_measured(rf: dict, peaks: dict) -> dict:
    """A roofline object with the measured ceiling beside the published one."""
    if not rf or peaks is None or rf.get("achieved") is None:
        return rf
    rf = dict(rf)
    mp = peaks["copy_GBps"] if rf["bound"] == "hbm" else peaks["mfma_loop_f16_TFLOPs"]
    rf["measured_peak"] = mp
    rf["frac_of_measured"] = round(rf["achieved"] / mp, 4)
    return rf


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--rotation", type=int, default=48,
                    help="distinct decode layers (the stack) the steps cycle through")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graphs")
    ap.add_argument("--separate-calls", action="store_true",
                    help="route and group with two calls instead of moe_route_group")
    ap.add_argument("--stage-calls", action="store_true",
                    help="decode steps call route_group + ffn_q instead of moe_layer")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-hidden", action="store_true",
                    help="skip the decode stack that starts from hidden states")
    ap.add_argument("--no-batched", action="store_true", help="skip the config-4 batched decode")
    ap.add_argument("--prefill-layers", type=int, default=0, help="0 = all 48")
    ap.add_argument("--prefill-steps", type=int, default=3)
    ap.add_argument("--prefill-1k-layers", type=int, default=8,
                    help="distinct layers of the 1,024-token chunk (0 = skip it)")
    ap.add_argument("--prefill-1k-steps", type=int, default=5)
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured copy/MFMA peaks")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 matrix-core gate/up variant")
    ap.add_argument("--cpu-full", action="store_true",
                    help="run every CPU oracle workload in full (no row samples; takes minutes)")
    ap.add_argument("--no-tiled", action="store_true",
                    help="prefill on the canonical weight planes only (no tiled copy)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="first copy a buffer of this many MiB 5 times (a kernel of known "
                         "traffic for scaling hardware byte counters)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-layers", type=int, default=8)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    global SEPARATE_CALLS, LAYER_CALL
    SEPARATE_CALLS = args.separate_calls
    LAYER_CALL = not (args.stage_calls or args.separate_calls)
    import torch
    import bit_quantized_moe_topk_amd as moe
    from synth import CONFIGS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    moe.lib()
    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 5 copies of {args.copy_calibration_mb} MiB")
        del src, dst
    cfg = CONFIGS[1]
    dec, hosts, insts = run_decode(cfg, args)
    log(f"decode: {dec['tokens_per_s']:.0f} tokens/s, {dec['ms_per_step'] * 1e3:.1f} us/step, "
        f"gemv_gateup {dec['roofline']['achieved']} GB/s")
    for it in insts:
        it.ex.close()
    del insts
    torch.cuda.empty_cache()

    # the same stack from hidden states: router product, top-k and the window
    # in one launch per layer
    dech = None
    if not args.no_hidden:
        import copy
        hargs = copy.copy(args)
        hargs.cpu_layers = 0
        h, _, hinsts = run_decode(cfg, hargs, workload="decode_hidden", hidden=True)
        for it in hinsts:
            it.ex.close()
        del hinsts
        torch.cuda.empty_cache()
        dech = {"workload": "decode from hidden states: the router product (bf16 [512][2048] "
                            "router rows + Zipf bias) in front of the same layer step, over the "
                            "same 48-layer stack", **h}
        log(f"decode from hidden states: {h['tokens_per_s']:.0f} tokens/s, "
            f"{h['ms_per_step'] * 1e3:.1f} us/step, kernels {h['kernels_us']}")

    # batched decode (config 4: 16 streams x 4 tokens, Q3): reported beside the
    # headline, through the general path (route + group, GEMV and matrix-core
    # experts, combine)
    bat = bat_own = None
    if not args.no_batched:
        import copy
        bargs = copy.copy(args)
        bargs.rotation = 16
        bargs.cpu_layers = 0
        for reading in ("shared", "own"):
            bcfg = CONFIGS[4] if reading == "shared" else CONFIGS[4].with_(stream_ranking=True)
            wl = "batched_decode" if reading == "shared" else "batched_decode_stream_ranking"
            b, _, binsts = run_decode(bcfg, bargs, workload=wl)
            for it in binsts:
                it.ex.close()
            del binsts
            torch.cuda.empty_cache()
            rank = ("the 16 streams share the layer's Zipf ranking of the experts"
                    if reading == "shared" else
                    "each of the 16 streams ranks the experts by a Zipf bias of its own")
            b = {"workload": "batched decode: 16 streams x 4 tokens (T = 64) through one MoE layer "
                             "(hidden 2048, 512 routed + 1 shared experts, top-10, intermediate 512, "
                             f"Q3 weights, bf16 activations); {rank}; steps rotate over 16 seeded "
                             "layer instances", **b}
            log(f"batched decode ({reading} ranking): {b['tokens_per_s']:.0f} tokens/s, "
                f"{b['ms_per_step'] * 1e3:.1f} us/step, {b['touched_experts_mean']:.0f} experts, "
                f"layer {b['layer_hbm_gbs']:.0f} GB/s")
            if reading == "shared":
                bat = b
            else:
                bat_own = b

    pre = pre1k = None
    if not args.no_prefill:
        pre = run_prefill(CONFIGS[3], args, args.prefill_layers or CONFIGS[3].layers,
                          args.prefill_steps, "prefill_8k")
        log(f"prefill: {pre['tokens_per_s_end_to_end']:.0f} tokens/s end to end, "
            f"{pre['ms_per_layer']:.3f} ms/layer, mfma_gateup {pre['roofline']['achieved']} TFLOP/s")
        if args.prefill_1k_layers:
            pre1k = run_prefill(CONFIGS[2], args, args.prefill_1k_layers, args.prefill_1k_steps,
                                "prefill_1k")
            log(f"prefill 1K: {pre1k['tokens_per_s_per_layer']:.0f} tokens/s per layer, "
                f"{pre1k['ms_per_layer'] * 1e3:.1f} us/layer, mfma_gateup "
                f"{pre1k['roofline']['achieved']} TFLOP/s")

    peaks = None
    if not args.no_peaks:
        peaks = measured_peaks()
        log(f"measured peaks: {peaks}")
        for r in (dec, dech, bat, bat_own, pre, pre1k):
            if r is not None:
                r["roofline"] = with_measured(r["roofline"], peaks)

    router = router_timing(args)
    log(f"router: {router}")

    f8 = None
    if not args.no_fp8:
        f8 = fp8_variant(args)
        log(f"fp8 variant: {f8}")

    cpu = None
    if not args.no_cpu_baseline and hosts:
        cpu = cpu_baseline(cfg, hosts, args)
        log(f"cpu oracle: {cpu['value']} tokens/s on {cpu['cores']} threads, "
            f"{cpu['single_core']['value']} on one core ({cpu['cpu_model']})")

    rf = dict(dec["roofline"])
    line = {
        "metric": METRIC,
        "value": round(dec["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16/bf16",
        "arithmetic": "gate/up: fp16 matrix-core operands (each x row scaled by its own power "
                      "of two, weights dequantised to fp16), fp32 accumulation; h in bf16; "
                      "down: bf16 matrix-core operands, fp32 accumulation; x and y bf16",
        "data": "synthetic",
        "config": {
            "workload": f"decode: one MoE layer step over a {cfg.T}-token verify window "
                        f"(hidden {cfg.H}, {cfg.E} routed + {cfg.shared} shared experts, "
                        f"top-{cfg.k}, intermediate {cfg.I}, Q{cfg.qtype} weights, bf16 "
                        f"activations); steps cycle through a stack of {args.rotation} distinct "
                        f"seeded layers",
            "tokens_per_step": cfg.T,
            "launch": "one hip graph per pass over the stack" if dec["graph"] else "eager",
        },
        "roofline": rf,
        "cpu_baseline": cpu,
        "decode_detail": {k: v for k, v in dec.items() if k not in ("roofline",)},
        "decode_from_hidden": dech,
        "measured_peaks": peaks,
        "prefill_8k": pre,
        "prefill_1k": pre1k,
        "batched_decode_q3": bat,
        "batched_decode_q3_stream_ranking": bat_own,
        "router": router,
        "fp8_gateup_variant": f8,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
