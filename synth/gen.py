"""Seeded generators for router logits, activations and packed expert planes.

Every array is drawn from numpy's PCG64 with a SeedSequence keyed by
(seed, workload id, layer, stream, expert), so any one expert of any layer can
be regenerated on its own (the 48-layer prefill stack holds 24,624 experts).

Packed expert planes (the canonical layout both sides read)
-----------------------------------------------------------
The pages name 2-bit "Q2_0" expert packs and 3-bit packs ("Strata - the
details", "Speed (measured)" and "Which model?") but publish no bit layout, so
the layout is fixed here. A weight is ``w = d * q + m`` with one fp16 ``d`` and
one fp16 ``m`` per block of 32 consecutive weights along the contraction axis
and an unsigned code ``q`` (Q2: 0..3, Q3: 0..7).

* Expert order: routed experts ``0..E-1``, then the shared expert (index E).
* Matrix order inside an expert: gate ``[I][H]``, up ``[I][H]``, down ``[H][I]``,
  each row-major with blocks running along the row (the contraction axis).
  An expert therefore holds ``NB = 3*H*I/32`` blocks, numbered in that order.
* ``codes``: 8 bytes per block. Weight ``j`` (0..31) of a block sits in byte
  ``j // 4`` at bits ``2*(j % 4)`` (little-endian: u32 word ``j // 16``, bits
  ``2*(j % 16)``). For Q3 these are the low two bits of the code.
* ``hi`` (Q3 only): 4 bytes per block; bit ``j`` of the little-endian u32 is
  bit 2 of code ``j``.
* ``dm``: two uint16 per block, the fp16 bit patterns of ``d`` then ``m``.

Draw recipe (one seed generates everything)
-------------------------------------------
* codes and high bits: uniform random bytes, which is the same as independent
  uniform codes;
* ``d = fp16(|z| * 0.02)`` with ``z ~ N(0,1)``; ``m = fp16(-c * d)`` with
  ``c = 1.5`` for Q2 and ``c = 3.5`` for Q3 (the middle of the code range);
* activations ``N(0,1)``, rounded to bf16 (round-to-nearest-even) for the bf16
  workloads;
* router logits ``N(0,1)`` per token and expert, plus, for the skewed
  workloads, a per-layer bias ``-1.1 * ln(rank_e)`` where ``rank`` is a seeded
  permutation of ``1..E`` (a Zipf(1.1) expert popularity shared by every token
  and stream of the layer);
* for the router in front of the layer: a bf16 router matrix ``[E][H]`` with
  entries ``N(0,1)/sqrt(H)`` (so ``x . w_e`` is about ``N(0,1)`` for N(0,1)
  activations) and, for the skewed workloads, the same per-layer Zipf bias as
  a float32 vector ``[E]`` (zeros otherwise).
"""
from __future__ import annotations

import numpy as np

from .configs import LayerConfig

# SeedSequence stream tags
_S_LOGITS, _S_WEIGHTS, _S_ZIPF, _S_X, _S_ROUTER = 0, 1, 2, 3, 4


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(v) for v in key])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the uint16 bits.

    Inputs here are finite; NaN/inf are passed through by the same bit rule.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def plane_sizes(cfg: LayerConfig) -> dict:
    """Per-expert plane sizes in bytes / elements for a layer of ``cfg``'s shape."""
    nb = 3 * cfg.H * cfg.I // 32
    return {"blocks": nb, "codes": nb * 8, "hi": nb * 4 if cfg.qtype == 3 else 0,
            "dm": nb * 2}


def zipf_bias(cfg: LayerConfig, seed: int, layer: int = 0) -> np.ndarray:
    """Per-expert logit bias ``-1.1 * ln(rank)``, float64 ``[E]``."""
    rank = _rng(seed, cfg.cid, layer, _S_ZIPF).permutation(cfg.E) + 1
    return -1.1 * np.log(rank.astype(np.float64))


def stream_zipf_bias(cfg: LayerConfig, seed: int, layer: int, stream: int) -> np.ndarray:
    """The Zipf bias of one decode stream that ranks the experts on its own."""
    rank = _rng(seed, cfg.cid, layer, _S_ZIPF, 1 + stream).permutation(cfg.E) + 1
    return -1.1 * np.log(rank.astype(np.float64))


def make_logits(cfg: LayerConfig, seed: int, layer: int = 0) -> np.ndarray:
    """Router logits, float32 ``[T, E]``.

    With ``stream_ranking`` the T rows are ``streams`` consecutive windows and
    each window's rows take the Zipf bias of its own stream; otherwise every
    row shares the layer's one ranking."""
    noise = _rng(seed, cfg.cid, layer, _S_LOGITS).standard_normal((cfg.T, cfg.E))
    if cfg.zipf and cfg.stream_ranking and cfg.streams > 1:
        if cfg.T % cfg.streams:
            raise ValueError("T must be a whole number of stream windows")
        bias = np.stack([stream_zipf_bias(cfg, seed, layer, s) for s in range(cfg.streams)])
        noise = noise + np.repeat(bias, cfg.T // cfg.streams, axis=0)
    elif cfg.zipf:
        noise = noise + zipf_bias(cfg, seed, layer)[None, :]
    return noise.astype(np.float32)


def make_router(cfg: LayerConfig, seed: int, layer: int = 0):
    """Router inputs: ``(w uint16 bf16 bits [E, H], bias float32 [E])``."""
    w = _rng(seed, cfg.cid, layer, _S_ROUTER).standard_normal((cfg.E, cfg.H)) / np.sqrt(cfg.H)
    bias = zipf_bias(cfg, seed, layer) if cfg.zipf else np.zeros(cfg.E)
    return f32_to_bf16_bits(w.astype(np.float32)), bias.astype(np.float32)


def make_x(cfg: LayerConfig, seed: int, layer: int = 0) -> np.ndarray:
    """Activations ``[T, H]``: float32 for f32 workloads, uint16 bf16 bits otherwise."""
    x = _rng(seed, cfg.cid, layer, _S_X).standard_normal((cfg.T, cfg.H)).astype(np.float32)
    return x if cfg.xdtype == "f32" else f32_to_bf16_bits(x)


def make_expert_planes(cfg: LayerConfig, seed: int, layer: int, expert: int):
    """Packed planes of one expert: ``(codes u8[NB*8], hi u8[NB*4] or None, dm u16[NB*2])``."""
    nb = 3 * cfg.H * cfg.I // 32
    rng = _rng(seed, cfg.cid, layer, _S_WEIGHTS, expert)
    codes = np.frombuffer(rng.bytes(nb * 8), dtype=np.uint8)
    hi = np.frombuffer(rng.bytes(nb * 4), dtype=np.uint8) if cfg.qtype == 3 else None
    z = rng.standard_normal(nb, dtype=np.float32)
    d = (np.abs(z) * np.float32(0.02)).astype(np.float16)
    c = np.float32(1.5 if cfg.qtype == 2 else 3.5)
    m = (-c * d.astype(np.float32)).astype(np.float16)
    dm = np.empty((nb, 2), dtype=np.uint16)
    dm[:, 0] = d.view(np.uint16)
    dm[:, 1] = m.view(np.uint16)
    return codes, hi, dm.reshape(-1)


def make_layer(cfg: LayerConfig, seed: int = 0, layer: int = 0, weights: bool = True,
               threads: int = 8) -> dict:
    """All inputs of one layer step.

    Returns a dict with ``logits`` f32 [T,E], ``x`` [T,H] (f32 or bf16 bits),
    and, if ``weights``, ``codes`` u8 [E_tot, NB*8], ``hi`` u8 [E_tot, NB*4] or
    None, ``dm`` u16 [E_tot, NB*2].
    """
    out = {"cfg": cfg, "seed": seed, "layer": layer,
           "logits": make_logits(cfg, seed, layer), "x": make_x(cfg, seed, layer)}
    if not weights:
        return out
    ps = plane_sizes(cfg)
    n = cfg.E_tot
    codes = np.empty((n, ps["codes"]), dtype=np.uint8)
    dm = np.empty((n, ps["dm"]), dtype=np.uint16)
    hi = np.empty((n, ps["hi"]), dtype=np.uint8) if cfg.qtype == 3 else None

    def fill(e: int) -> None:
        c, h, q = make_expert_planes(cfg, seed, layer, e)
        codes[e] = c
        dm[e] = q
        if hi is not None:
            hi[e] = h

    if threads > 1 and n > 32:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(n)))
    else:
        for e in range(n):
            fill(e)
    out.update(codes=codes, hi=hi, dm=dm)
    return out
