"""Routed MoE FFN over 2/3-bit block-quantized experts on one MI355X (gfx950).

Thin ctypes binding over ``libmoe.so`` (the C ABI in ``include/moe.h``). Every
step of the layer runs in the library's HIP kernels; this module only checks
tensor placement, allocates outputs and workspace with PyTorch and passes raw
device pointers plus the current HIP stream. There is no CPU fallback: without
the built library every call raises.

Calls, in the order a layer uses them:
    idx, gates = route_topk(logits, k)
    grp        = group(idx, E, has_shared)                  # optional
    ex         = Experts(qtype, E, has_shared, H, I, codes, hi, dm)
    y          = ffn_q(x, ex, idx, gates, grouping=grp, mode="fast" | "check")
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
Q2, Q3 = 2, 3
FAST, CHECK_F32 = 0, 2
MAX_E = 2048

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


def lib() -> C.CDLL:
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_quantized_moe_topk_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = C.c_char_p
        L.moe_router_logits.argtypes = [P, i32, i32, i32, P, P, i32, P, P]
        L.moe_router_logits.restype = C.c_int
        L.moe_route_topk.argtypes = [P, i32, i32, i32, P, P, P]
        L.moe_route_topk.restype = C.c_int
        L.moe_group_workspace_size.argtypes = [i32, i32, i32]
        L.moe_group_workspace_size.restype = sz
        L.moe_group.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, sz, P]
        L.moe_group.restype = C.c_int
        L.moe_route_group.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P, P, sz, P]
        L.moe_route_group.restype = C.c_int
        L.moe_experts_create.argtypes = [C.POINTER(P), i32, i32, i32, i32, i32, P, P, P]
        L.moe_experts_create.restype = C.c_int
        L.moe_experts_destroy.argtypes = [P]
        L.moe_experts_destroy.restype = C.c_int
        L.moe_experts_tiled_size.argtypes = [P]
        L.moe_experts_tiled_size.restype = sz
        L.moe_experts_attach_tiled.argtypes = [P, P, sz, P]
        L.moe_experts_attach_tiled.restype = C.c_int
        L.moe_ffn_q_workspace_size.argtypes = [P, i32, i32, i32]
        L.moe_ffn_q_workspace_size.restype = sz
        L.moe_ffn_q.argtypes = [P, i32, i32, P, P, P, i32, P, P, P, P, P, i32, P, sz, P]
        L.moe_ffn_q.restype = C.c_int
        L.moe_layer_workspace_size.argtypes = [P, i32, i32, i32]
        L.moe_layer_workspace_size.restype = sz
        L.moe_layer.argtypes = [P, P, i32, i32, P, i32, P, P, P, i32, P, sz, P]
        L.moe_layer.restype = C.c_int
        L.moe_layer_static.argtypes = [P, P, i32, i32, P, i32, P, P, P, i32, P]
        L.moe_layer_static.restype = C.c_int
        L.moe_router_topk.argtypes = [P, i32, i32, i32, P, P, i32, i32, P, P, P, P]
        L.moe_router_topk.restype = C.c_int
        L.moe_expert_gateup_fp8_workspace_size.argtypes = [P, i32]
        L.moe_expert_gateup_fp8_workspace_size.restype = sz
        L.moe_expert_gateup_fp8.argtypes = [P, i32, P, i32, P, P, sz, P]
        L.moe_expert_gateup_fp8.restype = C.c_int
        L.moe_layer_hidden_workspace_size.argtypes = [P, i32, i32, i32]
        L.moe_layer_hidden_workspace_size.restype = sz
        L.moe_layer_hidden.argtypes = [P, i32, i32, P, P, P, i32, P, P, P, P, i32, P, sz, P]
        L.moe_layer_hidden.restype = C.c_int
        L.moe_profile_begin.argtypes = [i32]
        L.moe_profile_begin.restype = C.c_int
        L.moe_profile_end.argtypes = []
        L.moe_profile_end.restype = C.c_int
        L.moe_profile_count.argtypes = []
        L.moe_profile_count.restype = i32
        L.moe_profile_get.argtypes = [i32, C.POINTER(C.c_char_p), C.POINTER(i32),
                                      C.POINTER(C.c_double)]
        L.moe_profile_get.restype = C.c_int
        _lib = L
    return _lib


def profile_begin(max_launches: int = 65536) -> None:
    """Record HIP events around every library launch from now on."""
    _check("moe_profile_begin", lib().moe_profile_begin(max_launches))


def profile_end() -> dict:
    """Stop recording; return {kernel name: (launches, total ms)}."""
    L = lib()
    _check("moe_profile_end", L.moe_profile_end())
    out = {}
    for i in range(L.moe_profile_count()):
        name, n, ms = C.c_char_p(), C.c_int32(), C.c_double()
        _check("moe_profile_get", L.moe_profile_get(i, C.byref(name), C.byref(n), C.byref(ms)))
        out[name.value.decode()] = (n.value, ms.value)
    return out


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise MoeError(fn, status)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need_cuda(name: str, t: torch.Tensor, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def router_logits(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None = None):
    """Router scores x . w[e] (+ bias[e]): float32 [T, E]. x: f32 or bf16 [T, H];
    w: bf16 [E, H] (or its uint16/int16 bit patterns); bias: f32 [E] or None."""
    _need_cuda("x", x, (torch.float32, torch.bfloat16))
    if w.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not w.is_cuda or not w.is_contiguous():
        raise ValueError("w must be a contiguous CUDA bf16 (or 16-bit pattern) tensor [E, H]")
    if bias is not None:
        _need_cuda("bias", bias, torch.float32)
    T, H = x.shape
    E = w.shape[0]
    if w.shape[1] != H or (bias is not None and bias.numel() != E):
        raise ValueError("shape mismatch between x, w and bias")
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    xdt = F32 if x.dtype == torch.float32 else BF16
    _check("moe_router_logits", lib().moe_router_logits(_ptr(x), xdt, T, H, _ptr(w),
                                                        _ptr(bias) if bias is not None else None,
                                                        E, _ptr(logits), _stream()))
    return logits


def router_topk(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None, k: int):
    """moe_router_topk: router product and top-k in one launch (bf16 x [T, H],
    w bf16 [E, H]): returns (idx int32 [T, k], gates f32 [T, k], logits f32 [T, E])."""
    _need_cuda("x", x, torch.bfloat16)
    if w.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not w.is_cuda or not w.is_contiguous():
        raise ValueError("w must be a contiguous CUDA bf16 (or 16-bit pattern) tensor [E, H]")
    if bias is not None:
        _need_cuda("bias", bias, torch.float32)
    T, H = x.shape
    E = w.shape[0]
    if w.shape[1] != H or (bias is not None and bias.numel() != E):
        raise ValueError("shape mismatch between x, w and bias")
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    gates = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check("moe_router_topk", lib().moe_router_topk(_ptr(x), BF16, T, H, _ptr(w),
                                                    _ptr(bias) if bias is not None else None, E, k,
                                                    _ptr(idx), _ptr(gates), _ptr(logits), _stream()))
    return idx, gates, logits


def route_topk(logits: torch.Tensor, k: int):
    """Top-k experts per token and their softmax gates: (idx int32 [T,k], gates f32 [T,k])."""
    _need_cuda("logits", logits, torch.float32)
    T, E = logits.shape
    idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    gates = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check("moe_route_topk", lib().moe_route_topk(_ptr(logits), T, E, k, _ptr(idx), _ptr(gates),
                                                  _stream()))
    return idx, gates


@dataclass
class Grouping:
    counts: torch.Tensor   # int32 [E+1]
    offsets: torch.Tensor  # int32 [E+2]
    perm: torch.Tensor     # int32 [A]
    slot_of: torch.Tensor  # int32 [A]


def group(idx: torch.Tensor, E: int, has_shared: bool) -> Grouping:
    """Stable grouping of the assignments of ``idx`` by expert."""
    _need_cuda("idx", idx, torch.int32)
    T, k = idx.shape
    dev = idx.device
    A = T * (k + int(bool(has_shared)))
    g = Grouping(torch.empty(E + 1, dtype=torch.int32, device=dev),
                 torch.empty(E + 2, dtype=torch.int32, device=dev),
                 torch.empty(max(A, 1), dtype=torch.int32, device=dev),
                 torch.empty(max(A, 1), dtype=torch.int32, device=dev))
    nbytes = lib().moe_group_workspace_size(T, k, E)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check("moe_group", lib().moe_group(_ptr(idx), T, k, E, int(bool(has_shared)), _ptr(g.counts),
                                        _ptr(g.offsets), _ptr(g.perm), _ptr(g.slot_of), _ptr(ws),
                                        nbytes, _stream()))
    g.perm = g.perm[:A]
    g.slot_of = g.slot_of[:A]
    return g


def route_group(logits: torch.Tensor, k: int, has_shared: bool):
    """Top-k routing and the grouping in one call: (idx, gates, Grouping)."""
    _need_cuda("logits", logits, torch.float32)
    T, E = logits.shape
    dev = logits.device
    A = T * (k + int(bool(has_shared)))
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    g = Grouping(torch.empty(E + 1, dtype=torch.int32, device=dev),
                 torch.empty(E + 2, dtype=torch.int32, device=dev),
                 torch.empty(max(A, 1), dtype=torch.int32, device=dev),
                 torch.empty(max(A, 1), dtype=torch.int32, device=dev))
    nbytes = lib().moe_group_workspace_size(T, k, E)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check("moe_route_group", lib().moe_route_group(
        _ptr(logits), T, E, k, int(bool(has_shared)), _ptr(idx), _ptr(gates), _ptr(g.counts),
        _ptr(g.offsets), _ptr(g.perm), _ptr(g.slot_of), _ptr(ws), nbytes, _stream()))
    g.perm = g.perm[:A]
    g.slot_of = g.slot_of[:A]
    return idx, gates, g


class Experts:
    """One layer's packed experts (device planes in the canonical layout)."""

    def __init__(self, qtype: int, E: int, has_shared: bool, H: int, I: int,
                 codes: torch.Tensor, hi: torch.Tensor | None, dm: torch.Tensor):
        _need_cuda("codes", codes, torch.uint8)
        _need_cuda("dm", dm, (torch.uint16, torch.int16))
        if hi is not None:
            _need_cuda("hi", hi, torch.uint8)
        E_tot = E + int(bool(has_shared))
        nb = 3 * H * I // 32
        if codes.numel() != E_tot * nb * 8 or dm.numel() != E_tot * nb * 2:
            raise ValueError("plane sizes do not match the shape")
        if qtype == Q3 and (hi is None or hi.numel() != E_tot * nb * 4):
            raise ValueError("Q3 needs a high-bit plane of E_tot * NB * 4 bytes")
        self.qtype, self.E, self.has_shared, self.H, self.I = qtype, E, bool(has_shared), H, I
        self._planes = (codes, hi, dm)  # keep alive for the handle's lifetime
        h = C.c_void_p()
        _check("moe_experts_create",
               lib().moe_experts_create(C.byref(h), qtype, E, int(bool(has_shared)), H, I,
                                        _ptr(codes), _ptr(hi), _ptr(dm)))
        self._h = h

    @property
    def handle(self) -> C.c_void_p:
        return self._h

    def attach_tiled(self) -> None:
        """Build the tiled weight copy that the prefill matrix-core tiles read
        (a device buffer as large as the planes, kept by this object)."""
        import torch
        nbytes = int(lib().moe_experts_tiled_size(self._h))
        buf = torch.empty(nbytes, dtype=torch.uint8, device=self._planes[0].device)
        stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
        _check("moe_experts_attach_tiled",
               lib().moe_experts_attach_tiled(self._h, _ptr(buf), nbytes, stream))
        self._tiled = buf

    def detach_tiled(self) -> None:
        _check("moe_experts_attach_tiled", lib().moe_experts_attach_tiled(self._h, None, 0, None))
        self._tiled = None

    def workspace_size(self, T: int, k: int, mode: int = FAST) -> int:
        return int(lib().moe_ffn_q_workspace_size(self._h, T, k, mode))

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().moe_experts_destroy(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_MODES = {"fast": FAST, "check": CHECK_F32, FAST: FAST, CHECK_F32: CHECK_F32}


def ffn_q(x: torch.Tensor, ex: Experts, idx: torch.Tensor, gates: torch.Tensor,
          grouping: Grouping | None = None, mode="fast", workspace: torch.Tensor | None = None,
          out: torch.Tensor | None = None) -> torch.Tensor:
    """Expert FFN + gate-weighted combine for every token of ``x``.

    ``x``: [T, H] float32 or bfloat16. Returns ``y`` [T, H] with x's dtype in
    fast mode, float32 in check mode.
    """
    mode = _MODES[mode]
    _need_cuda("x", x, (torch.float32, torch.bfloat16))
    _need_cuda("idx", idx, torch.int32)
    _need_cuda("gates", gates, torch.float32)
    T, H = x.shape
    k = idx.shape[1]
    if H != ex.H or idx.shape[0] != T or tuple(gates.shape) != (T, k):
        raise ValueError("shape mismatch between x, idx, gates and the experts")
    xdt = F32 if x.dtype == torch.float32 else BF16
    ydtype = torch.float32 if mode == CHECK_F32 else x.dtype
    y = out if out is not None else torch.empty((T, H), dtype=ydtype, device=x.device)
    _need_cuda("out", y, ydtype)
    nbytes = ex.workspace_size(T, k, mode)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    g = grouping
    _check("moe_ffn_q", lib().moe_ffn_q(
        _ptr(x), xdt, T, ex.handle, _ptr(idx), _ptr(gates), k,
        _ptr(g.counts) if g else None, _ptr(g.offsets) if g else None,
        _ptr(g.perm) if g else None, _ptr(g.slot_of) if g else None,
        _ptr(y), mode, _ptr(workspace), workspace.numel(), _stream()))
    return y


def layer(logits: torch.Tensor, x: torch.Tensor, ex: "Experts", k: int, mode="fast",
          workspace: torch.Tensor | None = None, out=None):
    """The whole layer (route, group, expert FFN, combine): returns (idx, gates, y).

    A caller-provided `workspace` (uint8, at least moe_layer_workspace_size
    bytes) must start zero-filled; the calls keep the counters in its first
    8192 bytes consistent from call to call. `out` = (idx, gates, y) writes
    into existing tensors (as a captured graph needs)."""
    mode = _MODES[mode]
    _need_cuda("logits", logits, torch.float32)
    _need_cuda("x", x, (torch.float32, torch.bfloat16))
    T, H = x.shape
    if H != ex.H or logits.shape[0] != T:
        raise ValueError("shape mismatch between logits, x and the experts")
    dev = x.device
    ydtype = torch.float32 if mode == CHECK_F32 else x.dtype
    if out is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        gates = torch.empty((T, k), dtype=torch.float32, device=dev)
        y = torch.empty((T, H), dtype=ydtype, device=dev)
    else:
        idx, gates, y = out
        _need_cuda("idx", idx, torch.int32)
        _need_cuda("gates", gates, torch.float32)
        _need_cuda("y", y, ydtype)
        if tuple(idx.shape) != (T, k) or tuple(gates.shape) != (T, k) or tuple(y.shape) != (T, H):
            raise ValueError("out tensors do not match (T, k) and (T, H)")
    nbytes = int(lib().moe_layer_workspace_size(ex.handle, T, k, mode))
    if workspace is None:  # zero-filled: its head holds the decode window's counters
        workspace = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=dev)
    xdt = F32 if x.dtype == torch.float32 else BF16
    _check("moe_layer", lib().moe_layer(_ptr(logits), _ptr(x), xdt, T, ex.handle, k, _ptr(idx),
                                        _ptr(gates), _ptr(y), mode, _ptr(workspace),
                                        workspace.numel(), _stream()))
    return idx, gates, y


def layer_hidden(x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor | None, ex: "Experts",
                 k: int, mode="fast", workspace: torch.Tensor | None = None, out=None,
                 logits: torch.Tensor | None = None):
    """moe_layer_hidden: the router product, then the whole layer, from the
    hidden states x [T, H]: returns (idx, gates, y, logits). w_router: bf16 [E, H]
    (or its 16-bit patterns); bias: f32 [E] or None. `logits` (f32 [T, E]) receives
    the router scores; when None, a new tensor does. `workspace` and `out` as
    for layer()."""
    mode = _MODES[mode]
    _need_cuda("x", x, (torch.float32, torch.bfloat16))
    if (w_router.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not w_router.is_cuda
            or not w_router.is_contiguous()):
        raise ValueError("w_router must be a contiguous CUDA bf16 (or 16-bit pattern) tensor [E, H]")
    if bias is not None:
        _need_cuda("bias", bias, torch.float32)
    T, H = x.shape
    if H != ex.H or tuple(w_router.shape) != (ex.E, H) or (bias is not None and bias.numel() != ex.E):
        raise ValueError("shape mismatch between x, w_router, bias and the experts")
    dev = x.device
    ydtype = torch.float32 if mode == CHECK_F32 else x.dtype
    if out is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        gates = torch.empty((T, k), dtype=torch.float32, device=dev)
        y = torch.empty((T, H), dtype=ydtype, device=dev)
    else:
        idx, gates, y = out
        _need_cuda("idx", idx, torch.int32)
        _need_cuda("gates", gates, torch.float32)
        _need_cuda("y", y, ydtype)
    if logits is None:
        logits = torch.empty((T, ex.E), dtype=torch.float32, device=dev)
    _need_cuda("logits", logits, torch.float32)
    nbytes = int(lib().moe_layer_hidden_workspace_size(ex.handle, T, k, mode))
    if workspace is None:  # zero-filled: its head holds the decode window's counters
        workspace = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=dev)
    xdt = F32 if x.dtype == torch.float32 else BF16
    _check("moe_layer_hidden", lib().moe_layer_hidden(
        _ptr(x), xdt, T, _ptr(w_router), _ptr(bias) if bias is not None else None, ex.handle, k,
        _ptr(idx), _ptr(gates), _ptr(y), _ptr(logits), mode, _ptr(workspace), workspace.numel(),
        _stream()))
    return idx, gates, y, logits


def expert_gateup_fp8(x: torch.Tensor, ex: "Experts", expert: int,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """moe_expert_gateup_fp8: h = silu(g) * u of one expert for every row of
    x (bf16 [T, H]) on the FP8 matrix cores (a measured variant): f32 [T, I]."""
    _need_cuda("x", x, torch.bfloat16)
    T, H = x.shape
    if H != ex.H:
        raise ValueError("x does not match the experts' H")
    h = torch.empty((T, ex.I), dtype=torch.float32, device=x.device)
    n = int(lib().moe_expert_gateup_fp8_workspace_size(ex.handle, T))
    if workspace is None:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=x.device)
    _check("moe_expert_gateup_fp8", lib().moe_expert_gateup_fp8(
        _ptr(x), T, ex.handle, expert, _ptr(h), _ptr(workspace), workspace.numel(), _stream()))
    return h


def layer_static(logits: torch.Tensor, x: torch.Tensor, ex: "Experts", k: int, mode="fast"):
    """moe_layer_static: the whole layer on the library's own per-GPU scratch
    (no workspace argument, nothing allocated by the library): (idx, gates, y)."""
    mode = _MODES[mode]
    _need_cuda("logits", logits, torch.float32)
    _need_cuda("x", x, (torch.float32, torch.bfloat16))
    T, H = x.shape
    if H != ex.H or logits.shape[0] != T:
        raise ValueError("shape mismatch between logits, x and the experts")
    dev = x.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    y = torch.empty((T, H), dtype=torch.float32 if mode == CHECK_F32 else x.dtype, device=dev)
    xdt = F32 if x.dtype == torch.float32 else BF16
    _check("moe_layer_static", lib().moe_layer_static(_ptr(logits), _ptr(x), xdt, T, ex.handle, k,
                                                      _ptr(idx), _ptr(gates), _ptr(y), mode,
                                                      _stream()))
    return idx, gates, y


__all__ = ["layer", "layer_static", "profile_begin", "profile_end", "router_logits", "route_topk", "route_group", "group", "Grouping", "Experts", "ffn_q", "lib", "status_string",
           "MoeError", "Q2", "Q3", "F32", "BF16", "FAST", "CHECK_F32", "MAX_E", "LIB_PATH"]
