"""CPU oracle for the routed MoE FFN layer over block-quantized experts.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The product path never imports this
package, and this package never imports the product (the two share no code;
both read inputs from ``synth``).

Two independent implementations live here:

* ``liboracle.so`` (``moe_oracle.c``): plain C, per token, sequential
  accumulation in double (``*_f64``) or float (``*_f32``, the fp32 oracle);
* ``dense.py``: a NumPy float64 dense brute force used to pin the C oracle.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from .build import ensure_built

_lib = None


def bind(cdll: C.CDLL) -> C.CDLL:
    """Declare the C signatures on a loaded oracle library."""
    P = C.c_void_p
    i = C.c_int
    cdll.oracle_route.argtypes = [P, i, i, i, P, P]
    cdll.oracle_group.argtypes = [P, i, i, i, i, P, P, P, P]
    cdll.oracle_half_to_double.argtypes = [C.c_uint16]
    cdll.oracle_half_to_double.restype = C.c_double
    cdll.oracle_bf16_to_double.argtypes = [C.c_uint16]
    cdll.oracle_bf16_to_double.restype = C.c_double
    for s in ("f32", "f64"):
        getattr(cdll, f"oracle_dequant_row_{s}").argtypes = [i, P, P, P, i, P]
        getattr(cdll, f"oracle_expert_forward_{s}").argtypes = [i, i, i, P, P, P, P, P, P, P, P]
        getattr(cdll, f"oracle_layer_rows_{s}").argtypes = [i, i, i, i, i, i, i, i, P, P, P,
                                                            P, P, P, P, i, P, i]
    return cdll


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        _lib = bind(C.CDLL(ensure_built()))
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _acc(prec: str):
    if prec not in ("f32", "f64"):
        raise ValueError(prec)
    return np.float32 if prec == "f32" else np.float64


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 is the top half of a float32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def router_logits(x: np.ndarray, w_bits: np.ndarray, bias=None) -> np.ndarray:
    """Router scores in front of the top-k, float64 ``[T, E]``.

    The pages keep the routers on the GPU and route each token to the experts
    its router scores highest ("Strata - the details", "How it works"; Strata
    README, "How does it work?"); the score is the plain product of the
    token's hidden state with each expert's router row: ``logits[t, e] =
    sum_h x[t, h] * w[e, h] (+ bias[e])``. ``x``: float32, or uint16 bf16
    bits; ``w_bits``: uint16 bf16 bits ``[E, H]``; ``bias``: float32 ``[E]``
    or None. Products and sums in float64 (a matrix product as one step).
    """
    xd = _bf16_to_f64(x) if np.asarray(x).dtype == np.uint16 else np.asarray(x, dtype=np.float64)
    wd = _bf16_to_f64(w_bits)
    if xd.ndim != 2 or wd.ndim != 2 or xd.shape[1] != wd.shape[1]:
        raise ValueError("x [T, H] and w [E, H] must share H")
    out = xd @ wd.T
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float64)[None, :]
    return out


def route(logits: np.ndarray, k: int):
    """Top-k experts per token (ties to the lower index) and their softmax gates."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("k out of range")
    idx = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float32)
    lib().oracle_route(_p(logits), T, E, k, _p(idx), _p(gates))
    return idx, gates


def group(idx: np.ndarray, E: int, has_shared: bool):
    """Stable counting sort of assignments by expert -> counts, offsets, perm, slot_of."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    if idx.size and (idx.min() < 0 or idx.max() >= E):
        raise ValueError("expert index out of range")
    A = T * (k + int(bool(has_shared)))
    counts = np.empty(E + 1, dtype=np.int32)
    offsets = np.empty(E + 2, dtype=np.int32)
    perm = np.empty(A, dtype=np.int32)
    slot_of = np.empty(A, dtype=np.int32)
    lib().oracle_group(_p(idx), T, k, E, int(bool(has_shared)), _p(counts), _p(offsets),
                       _p(perm), _p(slot_of))
    return counts, offsets, perm, slot_of


def half_to_double(h: int) -> float:
    return lib().oracle_half_to_double(int(h))


def dequant_row(qtype: int, codes: np.ndarray, hi, dm: np.ndarray, K: int, prec: str = "f64"):
    """One row of K weights from its packed blocks."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    dm = np.ascontiguousarray(dm, dtype=np.uint16)
    hi = None if hi is None else np.ascontiguousarray(hi, dtype=np.uint8)
    if K % 32 or codes.size < K // 4 or dm.size < K // 16 or (qtype == 3 and (hi is None or hi.size < K // 8)):
        raise ValueError("plane too small for K")
    w = np.empty(K, dtype=_acc(prec))
    getattr(lib(), f"oracle_dequant_row_{prec}")(qtype, _p(codes), _p(hi), _p(dm), K, _p(w))
    return w


def expert_forward(qtype: int, H: int, I: int, codes, hi, dm, x, prec: str = "f64"):
    """One expert on one token: returns (o [H], g [I], u [I], h [I])."""
    at = _acc(prec)
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    dm = np.ascontiguousarray(dm, dtype=np.uint16).reshape(-1)
    hi = None if hi is None else np.ascontiguousarray(hi, dtype=np.uint8).reshape(-1)
    nb = 3 * H * I // 32
    if codes.size != nb * 8 or dm.size != nb * 2 or (qtype == 3 and hi.size != nb * 4):
        raise ValueError("plane sizes do not match H, I")
    x = np.ascontiguousarray(x, dtype=at)
    o = np.empty(H, dtype=at)
    g, u, h = (np.empty(I, dtype=at) for _ in range(3))
    getattr(lib(), f"oracle_expert_forward_{prec}")(qtype, H, I, _p(codes), _p(hi), _p(dm),
                                                     _p(x), _p(o), _p(g), _p(u), _p(h))
    return o, g, u, h


def layer_rows(layer: dict, idx: np.ndarray, gates: np.ndarray, rows=None, prec: str = "f64",
               threads: int = 0):
    """Layer output for the tokens ``rows`` (all tokens if None): array [len(rows), H].

    ``layer`` is a dict from ``synth.make_layer``; ``idx``/``gates`` are [T, k].
    """
    cfg = layer["cfg"]
    at = _acc(prec)
    T, k = idx.shape
    rows = np.arange(T, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    if rows.size and (rows.min() < 0 or rows.max() >= T):
        raise ValueError("row out of range")
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    if idx.size and (idx.min() < 0 or idx.max() >= cfg.E):
        raise ValueError("expert index out of range")
    gates = np.ascontiguousarray(gates, dtype=np.float32)
    x = np.ascontiguousarray(layer["x"])
    xdt = 0 if x.dtype == np.float32 else 1
    if xdt == 1 and x.dtype != np.uint16:
        raise TypeError("x must be float32 or bf16 bits (uint16)")
    y = np.empty((rows.size, cfg.H), dtype=at)
    codes = np.ascontiguousarray(layer["codes"])
    dm = np.ascontiguousarray(layer["dm"])
    hi = layer.get("hi")
    hi = None if hi is None else np.ascontiguousarray(hi)
    getattr(lib(), f"oracle_layer_rows_{prec}")(
        cfg.qtype, T, cfg.H, cfg.E, cfg.I, k, cfg.shared, xdt, _p(x), _p(idx), _p(gates),
        _p(codes), _p(hi), _p(dm), _p(rows), int(rows.size), _p(y), int(threads))
    return y


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))
