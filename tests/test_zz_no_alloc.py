"""moe_layer_forward_noalloc, the entry point for callers that cannot allocate
(its workspace is a library-owned device array), through the C ABI: its
outputs equal moe_layer_forward's with a caller workspace bit for bit, on two
calls in a row with the second smaller, at the Strata verify/decode shape and
at the Gemma shape with its shared expert; shapes or token counts beyond the
array are rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

import bit_expert_ffn_amd as moe
from synth import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _fn():
    f = moe.lib().moe_layer_forward_noalloc
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.POINTER(moe.LayerDesc), vp, vp, vp, i32, vp, i32, vp, vp, vp, vp]
    return f


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _noalloc(desc, table, x, logits, shared=None):
    T = x.shape[0]
    y = torch.empty((T, desc.expert.hidden), dtype=torch.float32, device=DEV)
    ids = torch.empty((T, desc.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, desc.top_k), dtype=torch.float32, device=DEV)
    st = _fn()(ctypes.byref(desc), _p(table), _p(shared), _p(x), 1 if x.dtype == torch.bfloat16 else 0, _p(logits),
               T, _p(y), _p(ids), _p(w), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, moe.lib().moe_last_error()
    return y, ids, w


@pytest.mark.parametrize("name,sizes", [("verify_t8", (8, 3)), ("gemma_decode", (4, 1))])
def test_noalloc_matches_layer_forward(name, sizes):
    w = wl.WORKLOADS[name]
    arena = wl.DeviceArena(w, device=DEV, layers=[1])
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k, shared_ff=w.shared_ff)
    for i, T in enumerate(sizes):
        print(f"noalloc {name} call {i} T={T}", flush=True)
        x, logits = wl.device_inputs(w, 1, 7 + i, device=DEV, tokens=T)
        ids_ref = torch.empty((T, w.top_k), dtype=torch.int32, device=DEV)
        w_ref = torch.empty((T, w.top_k), dtype=torch.float32, device=DEV)
        y_ref = moe.layer_forward(desc, arena.tables[1], x, logits, shared=arena.shared_blob(1), ids=ids_ref,
                                  weights=w_ref)
        y, ids, wt = _noalloc(desc, arena.tables[1], x, logits, shared=arena.shared_blob(1))
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_ref) and torch.equal(wt, w_ref)
        assert torch.equal(y, y_ref), f"{name} call {i} (T={T}) differs from moe_layer_forward"


def test_noalloc_rejects_what_the_array_cannot_hold():
    f = _fn()
    p = ctypes.c_void_p(1 << 24)
    d = moe.layer_desc(2560, 640, 1, 1.5, 512, 10)
    assert f(ctypes.byref(d), p, None, p, 1, p, 9, p, None, None, None) == 2          # prefill-sized T
    assert b"T <= 8" in moe.lib().moe_last_error()
    big = moe.layer_desc(4096, 1024, 2, 7.5, 64, 32)                                  # > 4 MiB of workspace
    assert f(ctypes.byref(big), p, None, p, 1, p, 8, p, None, None, None) == 3
    assert b"device array" in moe.lib().moe_last_error()
    assert f(ctypes.byref(d), p, None, p, 1, p, 0, p, None, None, None) == 0          # T = 0: nothing to do
