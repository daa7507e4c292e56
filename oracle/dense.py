"""Dense float64 brute force of the routed MoE layer (NumPy).

TEST INFRASTRUCTURE ONLY. It pins the C oracle on tiny shapes by a different
route to the same numbers:

* probabilities are a softmax over all E logits, the top-k set is taken from a
  lexicographic sort (logit descending, index ascending), and the selected
  probabilities are renormalised to sum to one;
* every expert, selected or not, is evaluated densely on every token from a
  fully dequantised float64 weight tensor, and the routed mask zeroes the rest;
* y = sum over experts of mask * gate * o + the shared expert's o.

Cost is O(T * E * H * I): small shapes only.
"""
from __future__ import annotations

import numpy as np


def _half(u16: np.ndarray) -> np.ndarray:
    return np.asarray(u16, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant_expert(qtype: int, H: int, I: int, codes, hi, dm):
    """Float64 (Wg [I,H], Wu [I,H], Wd [H,I]) of one expert from its packed planes."""
    nb = 3 * H * I // 32
    c = np.asarray(codes, dtype=np.uint8).reshape(nb, 8)
    # 2-bit fields, least significant first: weight j of a block in byte j//4
    q = np.stack([(c >> s) & 3 for s in (0, 2, 4, 6)], axis=-1).reshape(nb, 32).astype(np.int64)
    if qtype == 3:
        hb = np.unpackbits(np.asarray(hi, dtype=np.uint8).reshape(nb, 4), axis=1,
                           bitorder="little")
        q = q + 4 * hb.astype(np.int64)
    pair = np.asarray(dm, dtype=np.uint16).reshape(nb, 2)
    d = _half(pair[:, 0])[:, None]
    m = _half(pair[:, 1])[:, None]
    w = (d * q + m).reshape(-1)
    n_gu = I * H
    wg = w[:n_gu].reshape(I, H)
    wu = w[n_gu:2 * n_gu].reshape(I, H)
    wd = w[2 * n_gu:].reshape(H, I)
    return wg, wu, wd


def x_float64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.float32:
        return x.astype(np.float64)
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def topk_mask_gates(logits: np.ndarray, k: int):
    """Mask [T,E] of the top-k experts and renormalised softmax gates [T,E] (f64)."""
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    mask = np.zeros((T, E), dtype=bool)
    ar = np.arange(E)
    for t in range(T):
        order = np.lexsort((ar, -np.asarray(logits[t], dtype=np.float32)))
        mask[t, order[:k]] = True
    g = np.where(mask, p, 0.0)
    g = g / g.sum(axis=1, keepdims=True)
    return mask, g


def dense_layer(layer: dict, k: int | None = None, logits=None):
    """y [T,H] float64 for a ``synth.make_layer`` dict, routing from its logits."""
    cfg = layer["cfg"]
    k = cfg.k if k is None else k
    logits = layer["logits"] if logits is None else logits
    x = x_float64(layer["x"])
    mask, gates = topk_mask_gates(logits, k)
    T = x.shape[0]
    y = np.zeros((T, cfg.H))
    hi = layer.get("hi")
    for e in range(cfg.E_tot):
        wg, wu, wd = dequant_expert(cfg.qtype, cfg.H, cfg.I, layer["codes"][e],
                                    None if hi is None else hi[e], layer["dm"][e])
        g = x @ wg.T
        u = x @ wu.T
        h = g / (1.0 + np.exp(-g)) * u
        o = h @ wd.T
        if e < cfg.E:
            y += gates[:, e:e + 1] * o      # zero where the expert is not routed
        else:
            y += o                          # shared expert, weight 1
    return y
