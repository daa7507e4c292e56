"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch.

Every call here either fails argument validation or has nothing to launch
(T == 0), so no HIP kernel is enqueued.
"""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

moe = pytest.importorskip("bit_quantized_moe_topk_amd")
if not os.path.exists(moe.LIB_PATH):
    pytest.skip("libmoe.so not built (run __graft_entry__.build())", allow_module_level=True)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert {"moe_route_topk", "moe_group", "moe_ffn_q", "moe_experts_create"} <= set(names)
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert moe.status_string(s) and moe.status_string(s) != "unknown status"
    assert moe.status_string(-99) == "unknown status"


FAKE = C.c_void_p(0x10000)  # 16-byte aligned, never dereferenced by the host checks


def test_route_validation():
    L = moe.lib()
    assert L.moe_route_topk(FAKE, 4, 16, 17, FAKE, FAKE, None) == moe.ERR_INVALID_ARG  # k > E
    assert L.moe_route_topk(FAKE, 4, 16, 0, FAKE, FAKE, None) == moe.ERR_INVALID_ARG   # k < 1
    assert L.moe_route_topk(FAKE, -1, 16, 2, FAKE, FAKE, None) == moe.ERR_INVALID_ARG  # T < 0
    assert L.moe_route_topk(FAKE, 4, 4096, 2, FAKE, FAKE, None) == moe.ERR_UNSUPPORTED  # E > max
    assert L.moe_route_topk(None, 4, 16, 2, FAKE, FAKE, None) == moe.ERR_INVALID_ARG   # null
    assert L.moe_route_topk(None, 0, 16, 2, None, None, None) == moe.OK                # T == 0


def test_group_validation():
    L = moe.lib()
    assert L.moe_group(FAKE, 4, 2, 16, 2, FAKE, FAKE, FAKE, FAKE, None, 0, None) == moe.ERR_INVALID_ARG
    assert L.moe_group(FAKE, 4, 0, 16, 1, FAKE, FAKE, FAKE, FAKE, None, 0, None) == moe.ERR_INVALID_ARG
    big_T = 100_000  # needs the multi-launch path and its scratch
    need = L.moe_group_workspace_size(big_T, 10, 512)
    assert need >= 512 * ((big_T * 10 + 1023) // 1024) * 4
    assert L.moe_group(FAKE, big_T, 10, 512, 1, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                       None) == moe.ERR_WORKSPACE
    assert L.moe_group_workspace_size(4, 10, 512) == 0   # one-workgroup path needs no scratch


def make_handle(qtype=2, E=16, shared=0, H=256, I=128, hi=None):
    h = C.c_void_p()
    st = moe.lib().moe_experts_create(C.byref(h), qtype, E, shared, H, I, FAKE, hi, FAKE)
    return st, h


def test_experts_validation_and_lifetime():
    L = moe.lib()
    st, h = make_handle()
    assert st == moe.OK and h.value
    assert L.moe_experts_destroy(h) == moe.OK
    assert make_handle(qtype=4)[0] == moe.ERR_INVALID_ARG
    assert make_handle(qtype=3)[0] == moe.ERR_INVALID_ARG            # Q3 without high bits
    assert make_handle(qtype=2, hi=FAKE)[0] == moe.ERR_INVALID_ARG   # Q2 with high bits
    assert make_handle(H=96)[0] == moe.ERR_UNSUPPORTED               # not a multiple of 64
    assert make_handle(E=5000)[0] == moe.ERR_UNSUPPORTED
    st = L.moe_experts_create(C.byref(C.c_void_p()), 2, 16, 0, 256, 128, C.c_void_p(0x10008),
                              None, FAKE)
    assert st == moe.ERR_INVALID_ARG                                  # misaligned plane


def test_ffn_validation_and_workspace():
    L = moe.lib()
    st, h = make_handle(E=512, shared=1, H=2048, I=512)
    assert st == moe.OK
    try:
        fast = L.moe_ffn_q_workspace_size(h, 1024, 10, moe.FAST)
        check = L.moe_ffn_q_workspace_size(h, 1024, 10, moe.CHECK_F32)
        A = 1024 * 11
        assert fast >= A * 2048 * 2 + A * 512 * 2      # o (bf16) + h (16-bit)
        assert check >= A * 2048 * 4 + A * 512 * 4
        assert L.moe_ffn_q_workspace_size(h, 1024, 10, 7) == 0
        args = lambda **kw: dict(dict(x=FAKE, xdt=moe.BF16, T=4, idx=FAKE, gates=FAKE, k=10,
                                      grp=(None,) * 4, y=FAKE, mode=moe.FAST, ws=FAKE,
                                      nb=10 ** 9), **kw)

        def call(a):
            return L.moe_ffn_q(a["x"], a["xdt"], a["T"], h, a["idx"], a["gates"], a["k"],
                               *a["grp"], a["y"], a["mode"], a["ws"], a["nb"], None)

        assert call(args(k=513)) == moe.ERR_INVALID_ARG
        assert call(args(xdt=5)) == moe.ERR_INVALID_ARG
        assert call(args(mode=1)) == moe.ERR_INVALID_ARG
        assert call(args(grp=(FAKE, None, None, None))) == moe.ERR_INVALID_ARG
        assert call(args(nb=100)) == moe.ERR_WORKSPACE
        assert call(args(x=C.c_void_p(0x10002))) == moe.ERR_INVALID_ARG
        assert call(args(T=0, x=None, idx=None, gates=None, y=None, ws=None, nb=0)) == moe.OK
    finally:
        L.moe_experts_destroy(h)


def test_tiled_copy_validation():
    L = moe.lib()
    assert L.moe_experts_tiled_size(None) == 0
    assert L.moe_experts_attach_tiled(None, FAKE, 1 << 30, None) == moe.ERR_INVALID_ARG
    for qtype, per_block in ((2, 12), (3, 16)):
        st, h = make_handle(qtype=qtype, E=16, shared=1, H=256, I=128,
                            hi=FAKE if qtype == 3 else None)
        assert st == moe.OK
        try:
            need = L.moe_experts_tiled_size(h)
            assert need == 17 * (3 * 256 * 128 // 32) * per_block
            assert L.moe_experts_attach_tiled(h, FAKE, need - 1, None) == moe.ERR_INVALID_ARG
            assert L.moe_experts_attach_tiled(h, C.c_void_p(0x10008), need,
                                              None) == moe.ERR_INVALID_ARG  # misaligned
            assert L.moe_experts_attach_tiled(h, None, 0, None) == moe.OK     # detach
        finally:
            L.moe_experts_destroy(h)


def test_router_validation():
    L = moe.lib()
    bf16 = 1
    # T == 0 launches nothing
    assert L.moe_router_logits(FAKE, bf16, 0, 256, FAKE, None, 16, FAKE, None) == moe.OK
    # H must be a multiple of 256; E within the limit; dtype known
    assert L.moe_router_logits(FAKE, bf16, 4, 128, FAKE, None, 16, FAKE, None) == moe.ERR_UNSUPPORTED
    assert L.moe_router_logits(FAKE, bf16, 4, 256, FAKE, None, 4096, FAKE, None) == moe.ERR_UNSUPPORTED
    assert L.moe_router_logits(FAKE, 7, 4, 256, FAKE, None, 16, FAKE, None) == moe.ERR_INVALID_ARG
    # missing or misaligned buffers
    assert L.moe_router_logits(None, bf16, 4, 256, FAKE, None, 16, FAKE, None) == moe.ERR_INVALID_ARG
    assert L.moe_router_logits(FAKE, bf16, 4, 256, None, None, 16, FAKE, None) == moe.ERR_INVALID_ARG
    assert L.moe_router_logits(C.c_void_p(0x10008), bf16, 4, 256, FAKE, None, 16, FAKE,
                               None) == moe.ERR_INVALID_ARG
    assert L.moe_router_logits(FAKE, bf16, -1, 256, FAKE, None, 16, FAKE, None) == moe.ERR_INVALID_ARG
