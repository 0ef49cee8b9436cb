"""The C-ABI library loads, exports every function the header declares, sizes
blobs and workspaces, and rejects bad arguments on the host before launching
anything (no GPU needed: every call here returns before any HIP call)."""
import ctypes
import os
import re

import pytest

import bit_expert_ffn_amd as moe
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 24   # an aligned address that is never dereferenced: validation fails first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from bit_expert_ffn_amd import build
        build.build()
    return moe.lib()


def test_header_symbols_are_exported(L):
    text = open(os.path.join(ROOT, "include", "moe_ffn.h")).read()
    names = sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))
    assert len(names) >= 10
    assert sorted(moe.EXPORTS) == names
    for n in names:
        getattr(L, n)           # dlsym; raises AttributeError if missing


def test_blob_bytes_agree_with_oracle(L):
    for qtype, H, FF in [(1, 2560, 640), (2, 2816, 704), (2, 2816, 2112), (2, 7168, 2048), (1, 256, 128)]:
        d = moe.expert_desc(H, FF, qtype, 1.5)
        assert moe.expert_blob_bytes(d) == oracle.blob_bytes(qtype, H, FF)
    assert moe.expert_blob_bytes(moe.expert_desc(2560, 640, 1, 1.5)) == 1382400
    assert moe.expert_blob_bytes(moe.expert_desc(100, 640, 1, 1.5)) == 0       # H not a multiple of 64
    assert moe.expert_blob_bytes(moe.expert_desc(2560, 640, 7, 1.5)) == 0      # unknown qtype


def test_workspace_sizes(L):
    d = moe.layer_desc(2560, 640, 1, 1.5, 512, 10)
    assert moe.layer_workspace_bytes(d, 1) > 0
    assert moe.layer_workspace_bytes(d, 8) > moe.layer_workspace_bytes(d, 1)
    assert moe.layer_workspace_bytes(d, 0) >= 0
    assert moe.layer_workspace_bytes(moe.layer_desc(2560, 640, 1, 1.5, 512, 600), 1) == 0   # k > E
    assert moe.expert_workspace_bytes(moe.expert_desc(256, 128, 1, 1.5), 4) > 0


def _status(fn, *args):
    return fn(*args)


def test_route_topk_rejects_bad_arguments(L):
    p = ctypes.c_void_p(FAKE)
    assert L.moe_route_topk(p, 4, 8, 9, 1, p, p, None) == 1           # k > E
    assert L.moe_route_topk(p, 4, 8, 0, 1, p, p, None) == 1           # k = 0
    assert L.moe_route_topk(p, 4, 2048, 8, 1, p, p, None) == 2        # E above the supported range
    assert L.moe_route_topk(p, 4, 64, 40, 1, p, p, None) == 2         # k above 32
    assert L.moe_route_topk(p, -1, 8, 2, 1, p, p, None) == 1          # T < 0
    assert L.moe_route_topk(p, 4, 8, 2, 2, p, p, None) == 1           # renormalize not 0/1
    assert L.moe_route_topk(None, 4, 8, 2, 1, p, p, None) == 1        # NULL logits
    assert L.moe_route_topk(None, 0, 8, 2, 1, None, None, None) == 0  # T = 0: nothing to do
    assert b"NULL" in L.moe_last_error() or len(L.moe_last_error()) >= 0
    assert moe.status_str(3) == "MOE_ERR_WORKSPACE"


def test_layer_forward_rejects_bad_arguments(L):
    p = ctypes.c_void_p(FAKE)
    ok = moe.layer_desc(2560, 640, 1, 1.5, 512, 10)

    def call(desc, shared=None, x_dtype=1, T=1, ws_bytes=1 << 30, x=p, table=p):
        return L.moe_layer_forward(ctypes.byref(desc), table, shared, x, x_dtype, p, T, p, None, None, p, ws_bytes,
                                   None)

    assert call(ok, ws_bytes=16) == 3                                          # workspace too small
    assert b"workspace" in L.moe_last_error()
    assert call(moe.layer_desc(2560, 640, 3, 1.5, 512, 10)) == 1               # unknown qtype
    assert call(moe.layer_desc(2500, 640, 1, 1.5, 512, 10)) == 1               # H not a multiple of 64
    assert call(moe.layer_desc(2560, 640, 1, 1.5, 512, 0)) == 1                # k = 0
    assert call(moe.layer_desc(2560, 640, 1, 1.5, 4096, 10)) == 2              # E above the supported range
    assert call(moe.layer_desc(2560, 640, 1, 1.5, 512, 10, shared_ff=640)) == 1   # shared_ff without a blob
    assert call(ok, shared=p) == 1                                             # a blob without shared_ff
    assert call(ok, x_dtype=5) == 1                                            # unknown activation dtype
    assert call(ok, T=-2) == 1
    assert call(ok, x=ctypes.c_void_p(FAKE + 2)) == 1                          # misaligned x
    assert call(ok, table=None) == 1                                           # NULL table
    assert call(ok, T=0) == 0                                                  # nothing to do
    bad_act = moe.layer_desc(2560, 640, 1, 1.5, 512, 10)
    bad_act.expert.act = 3
    assert call(bad_act) == 2
    big = moe.layer_desc(2560 * 8, 640, 1, 1.5, 512, 10)                      # 320 blocks per row
    assert call(big) == 2
    assert call(moe.layer_desc(2560, 640, 1, 1.25, 512, 10)) == 2             # zero point not a multiple of 0.5
    assert call(moe.layer_desc(2560, 640, 1, 70.0, 512, 10)) == 2             # zero point beyond 64
    assert call(moe.layer_desc(2560, 640, 1, -2.5, 512, 10), ws_bytes=16) == 3  # negative half-integer: accepted


def test_expert_ffn_rejects_bad_arguments(L):
    p = ctypes.c_void_p(FAKE)
    d = moe.expert_desc(256, 128, 1, 1.5)
    assert L.moe_expert_ffn(ctypes.byref(d), p, p, 0, 4, p, p, 16, None) == 3
    assert L.moe_expert_ffn(ctypes.byref(d), None, p, 0, 4, p, p, 1 << 30, None) == 1
    assert L.moe_expert_ffn(ctypes.byref(d), p, p, 9, 4, p, p, 1 << 30, None) == 1
    assert L.moe_expert_ffn(ctypes.byref(d), p, p, 0, 0, p, p, 0, None) == 0
    assert L.moe_dequant_matrix(ctypes.byref(d), p, 3, p, None) == 1
    assert L.moe_validate_table(None, 4, None) == 1


def test_layer_forward_timed_rejects_bad_arguments(L):
    p = ctypes.c_void_p(FAKE)
    ok = moe.layer_desc(2560, 640, 1, 1.5, 512, 10)
    nk = ctypes.c_int32(7)

    def call(events, n, ws_bytes=1 << 30, T=1):
        return L.moe_layer_forward_timed(ctypes.byref(ok), p, None, p, 1, p, T, p, None, None, p, ws_bytes, None,
                                         events, n, ctypes.byref(nk))

    assert call(None, 2) == 1                                     # events missing
    assert call((ctypes.c_void_p * 2)(FAKE, None), 2) == 1        # a NULL event
    assert call(None, -1) == 1                                    # negative count
    assert call(None, 0, ws_bytes=16) == 3                        # the layer checks still apply
    assert nk.value == 0
    assert call(None, 0, T=0) == 0                                # nothing to do, no kernel
    assert nk.value == 0


def test_max_tokens_and_prefill_limit(L):
    """moe_max_tokens states the largest T the matrix-core path's 32-bit
    offsets address; a call above it is rejected on the host."""
    d = moe.layer_desc(7168, 2048, 2, 7.5, 256, 8)
    lim = ((1 << 32) - 4096)
    assert moe.max_tokens(d) == min(lim // (4 * 7168), lim // (4 * 2048 * 8)) == 65535
    ds = moe.layer_desc(7168, 2048, 2, 7.5, 256, 8, shared_ff=4096)
    assert moe.max_tokens(ds) == min(lim // (4 * 7168), lim // (4 * 4096 * 9))
    assert moe.max_tokens(moe.layer_desc(2560, 640, 7, 1.5, 512, 10)) == 0      # invalid descriptor
    p = ctypes.c_void_p(FAKE)
    T = moe.max_tokens(d) + 1
    st = L.moe_layer_forward(ctypes.byref(d), p, None, p, 1, p, T, p, None, None, p, 1 << 62, None)
    assert st == 2 and b"T = 65536" in L.moe_last_error()
    e = moe.expert_desc(7168, 2048, 2, 7.5)
    t1 = min(lim // (4 * 7168), lim // (4 * 2048))
    assert L.moe_expert_ffn(ctypes.byref(e), p, p, 1, t1 + 1, p, p, 1 << 62, None) == 2


def test_workspace_check_rejects_bad_arguments(L):
    """Argument checks of moe_workspace_check run before any HIP call."""
    d = moe.layer_desc(2560, 640, 1, 1.5, 512, 10)
    assert L.moe_workspace_check(ctypes.byref(d), None, 1 << 20, None) == 1           # NULL workspace
    assert L.moe_workspace_check(ctypes.byref(d), ctypes.c_void_p(FAKE + 64), 1 << 20, None) == 1   # misaligned
    assert L.moe_workspace_check(ctypes.byref(d), ctypes.c_void_p(FAKE), 256, None) == 3            # too small
    assert L.moe_workspace_check(None, ctypes.c_void_p(FAKE), 1 << 20, None) == 1
    L.moe_debug_set_wait_limit(-1)     # host-side state only


def test_layer_options_and_router_reject_bad_arguments(L):
    """Host checks of moe_layer_forward_ex's options and of moe_router_logits."""
    p = ctypes.c_void_p(FAKE)
    d = moe.layer_desc(2560, 640, 1, 1.5, 512, 10)
    rt = moe.Router(FAKE, None, 1, 1e-6)

    def ex(opts, logits=p, T=1, desc=d):
        return L.moe_layer_forward_ex(ctypes.byref(desc), ctypes.byref(opts) if opts is not None else None, p, None,
                                      p, 1, logits, T, p, None, None, p, 1 << 30, None)

    O = moe.LayerOpts
    assert ex(O(ctypes.pointer(rt), None, None, FAKE, FAKE), logits=None) == 1   # router and ids_in together
    assert ex(O(None, None, None, FAKE, None)) == 1                               # ids_in without w_in
    assert ex(O(ctypes.pointer(rt), None, None, None, None)) == 1                 # router with logits given
    assert ex(O(None, FAKE, None, None, None)) == 1                               # logits_out without router
    assert ex(None, logits=None) == 1                                             # nothing to route from
    assert ex(O(None, None, FAKE + 2, None, None)) == 1                           # misaligned down_scale
    bad = moe.Router(FAKE, None, 2, 1e-6)
    assert ex(O(ctypes.pointer(bad), None, None, None, None), logits=None) == 1   # norm not 0/1
    bad = moe.Router(FAKE, None, 1, -1.0)
    assert ex(O(ctypes.pointer(bad), None, None, None, None), logits=None) == 1   # negative eps
    gelu = moe.layer_desc(2560, 640, 1, 1.5, 512, 10, act=moe.ACT_GEGLU_TANH)
    assert L.moe_layer_workspace_bytes(ctypes.byref(gelu), 1) > 0                 # GeGLU is a known activation
    assert ex(O(None, None, None, FAKE, FAKE), T=0) == 0                          # nothing to do
    f = L.moe_router_logits
    assert f(ctypes.byref(rt), 512, 2560, p, 1, 0, p, None) == 0                  # T = 0
    assert f(ctypes.byref(rt), 512, 2568, p, 1, 1, p, None) == 1                  # H not a multiple of 32
    assert f(None, 512, 2560, p, 1, 1, p, None) == 1
    assert f(ctypes.byref(moe.Router(FAKE + 8, None, 0, 0.0)), 512, 2560, p, 1, 1, p, None) == 1   # misaligned W
    assert f(ctypes.byref(rt), 512, 2560, p, 7, 1, p, None) == 1                  # unknown x dtype
    d3 = moe.layer_desc(2560, 640, 1, 1.5, 512, 10)
    d3.expert.act = 2
    assert ex(None, desc=d3) == 2                                                 # unknown activation
