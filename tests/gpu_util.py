"""Helpers shared by the GPU parity tests: upload seeded layers, compare rows."""
from __future__ import annotations

import os
import sys

import numpy as np

import oracle


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def upload(layer: dict, dev="cuda"):
    """Device tensors of a synth layer: logits, x, codes, hi, dm."""
    import torch
    x = layer["x"]
    xt = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        xt = xt.view(torch.int16).view(torch.bfloat16)
    out = {"logits": torch.from_numpy(layer["logits"]).to(dev), "x": xt.to(dev)}
    if "codes" in layer:
        out["codes"] = torch.from_numpy(layer["codes"].reshape(-1)).to(dev)
        out["dm"] = torch.from_numpy(layer["dm"].reshape(-1).view(np.int16)).to(dev)
        hi = layer.get("hi")
        out["hi"] = None if hi is None else torch.from_numpy(hi.reshape(-1)).to(dev)
    return out


def experts_of(layer: dict, dev_layer: dict):
    import bit_quantized_moe_topk_amd as moe
    cfg = layer["cfg"]
    return moe.Experts(cfg.qtype, cfg.E, bool(cfg.shared), cfg.H, cfg.I, dev_layer["codes"],
                       dev_layer["hi"], dev_layer["dm"])


def y_to_f64(y) -> np.ndarray:
    import torch
    return y.float().cpu().numpy().astype(np.float64)


def rel_l2_rows(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return num / np.maximum(den, 1e-300)


def oracle_rows(layer, idx, gates, rows=None):
    return oracle.layer_rows(layer, np.asarray(idx), np.asarray(gates), rows=rows, prec="f64",
                             threads=threads())
