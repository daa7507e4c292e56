"""GPU parity of the FP8 matrix-core gate/up variant (moe_expert_gateup_fp8).

The variant is the gfx950 analogue of the pages' 8-bit tensor-core prompt
kernels ("Strata - the details", "Speed (measured)"): codes as exact E4M3
values, each token row scaled by a power of two and split into two E4M3 parts,
d and m applied per 32-weight block in fp32. Its h = silu(g) * u must agree
with the oracle's expert forward (float64) within the fast-mode bar, 1e-2
relative L2 per token row; the measured error is logged (expected far below).
"""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, make_layer
from synth.gen import bf16_bits_to_f32, f32_to_bf16_bits
from gpu_util import experts_of, log, rel_l2_rows, threads, torch_cuda, upload

pytestmark = pytest.mark.gpu

TOL = 1e-2


def oracle_h(lay, expert, rows):
    cfg = lay["cfg"]
    nb = 3 * cfg.H * cfg.I // 32
    codes = lay["codes"].reshape(cfg.E_tot, -1)[expert]
    dm = lay["dm"].reshape(cfg.E_tot, -1)[expert]
    hi = None if lay["hi"] is None else lay["hi"].reshape(cfg.E_tot, -1)[expert]
    x = lay["x"]
    xf = bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)
    out = []
    for t in rows:
        out.append(oracle.expert_forward(cfg.qtype, cfg.H, cfg.I, codes, hi, dm, xf[t])[3])
    assert codes.size == nb * 8
    return np.array(out)


def run_case(cfg, expert, rows=None, scale_rows=False, seed=91):
    torch = torch_cuda()
    import bit_quantized_moe_topk_amd as moe
    lay = make_layer(cfg, seed=seed, threads=threads())
    if scale_rows:  # rows far outside fp16's range and far below it, beside ordinary rows
        sc = np.array([(1e5, 3e-9, 1.0, 2.5e4, 1e-6, 7e5, 1e-10, 0.5)[t % 8] for t in range(cfg.T)])
        x = (bf16_bits_to_f32(lay["x"]).astype(np.float64) * sc[:, None]).astype(np.float32)
        lay = dict(lay, x=f32_to_bf16_bits(x))
    dev = upload(lay)
    ex = experts_of(lay, dev)
    log(f"[fp8 gate/up] T={cfg.T} Q{cfg.qtype} expert {expert} scaled rows {scale_rows}")
    h = moe.expert_gateup_fp8(dev["x"], ex, expert)
    h2 = moe.expert_gateup_fp8(dev["x"], ex, expert)
    torch.cuda.synchronize()
    assert torch.equal(h, h2), "not reproducible"
    if rows is None:
        rows = np.arange(cfg.T)
    got = h.cpu().numpy().astype(np.float64)[rows]
    assert np.isfinite(got).all()
    ref = oracle_h(lay, expert, rows)
    err = rel_l2_rows(got, ref)
    log(f"[fp8 gate/up] T={cfg.T} Q{cfg.qtype}: max rel-L2 {err.max():.3e}, median {np.median(err):.3e} "
        f"over {len(rows)} rows")
    assert err.max() <= TOL
    ex.close()
    return err


@pytest.mark.parametrize("qtype", [2, 3])
def test_fp8_gateup_ragged_batch(qtype):
    cfg = CONFIGS[2].with_(T=200, qtype=qtype)
    run_case(cfg, expert=cfg.E)            # the shared expert
    run_case(cfg.with_(T=37), expert=5)


def test_fp8_gateup_8k_sampled():
    cfg = CONFIGS[3]
    rows = np.unique(np.random.default_rng(93).choice(cfg.T, 32, replace=False))
    run_case(cfg, expert=cfg.E, rows=rows)


def test_fp8_gateup_activation_range():
    run_case(CONFIGS[2].with_(T=64), expert=3, scale_rows=True)
