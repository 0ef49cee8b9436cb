"""ORACLE -- test infrastructure only (ctypes wrapper over oracle.c).

A plain single-threaded float64 CPU implementation of the routed low-bit
expert FFN layer.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the GPU library never does, and the two share
no code.  See oracle.c for the pages each function follows.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

Q2 = 1   # 64 two-bit codes + fp16 scale per 18-byte block
Q4 = 2   # 32 four-bit codes + fp16 scale per 18-byte block


def build():
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           os.path.join(_HERE, "oracle.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("oracle library not built: call oracle.build() (or __graft_entry__.build())")
        L = ctypes.CDLL(_LIB_PATH)
        i32, i64, dbl, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.oracle_blob_bytes.restype = i64
        L.oracle_blob_bytes.argtypes = [ctypes.c_int, i64, i64]
        L.oracle_dequant_matrix.argtypes = [vp, ctypes.c_int, dbl, i64, i64, ctypes.c_int, vp]
        L.oracle_expert_ffn.restype = ctypes.c_int
        L.oracle_expert_ffn.argtypes = [vp, ctypes.c_int, dbl, i64, i64, vp, ctypes.c_int, i64, vp]
        L.oracle_route_topk.restype = ctypes.c_int
        L.oracle_route_topk.argtypes = [vp, i64, i32, i32, i32, vp, vp]
        L.oracle_layer_forward.restype = ctypes.c_int
        L.oracle_layer_forward.argtypes = [vp, i32, i32, i32, ctypes.c_int, dbl, i64, i64, vp, i64, vp,
                                           ctypes.c_int, vp, i64, vp, vp, vp]
        L.oracle_gelu_tanh.restype = None
        L.oracle_gelu_tanh.argtypes = [vp, i64, vp]
        L.oracle_expert_ffn_act.restype = ctypes.c_int
        L.oracle_expert_ffn_act.argtypes = [vp, ctypes.c_int, dbl, i64, i64, ctypes.c_int, vp, ctypes.c_int, i64, vp]
        L.oracle_router_logits.restype = ctypes.c_int
        L.oracle_router_logits.argtypes = [vp, i32, i64, vp, ctypes.c_int, i64, ctypes.c_int, dbl, vp, vp]
        L.oracle_layer_forward_ex.restype = ctypes.c_int
        L.oracle_layer_forward_ex.argtypes = [vp, i32, i32, i32, ctypes.c_int, dbl, i64, i64, ctypes.c_int, vp, i64,
                                              vp, vp, ctypes.c_int, vp, vp, vp, i64, vp, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data)


def _xinfo(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, 1
    if x.dtype == np.float32:
        return x, 0
    raise TypeError("x must be uint16 (bf16 bits) or float32")


def blob_bytes(qtype, H, FF):
    return int(lib().oracle_blob_bytes(qtype, H, FF))


def dequant_matrix(blob, qtype, z, H, FF, m):
    """Dense float64 matrix m (0 gate [FF,H], 1 up [FF,H], 2 down [H,FF]) of a blob."""
    rows, cols = [(FF, H), (FF, H), (H, FF)][m]
    out = np.empty((rows, cols), dtype=np.float64)
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    lib().oracle_dequant_matrix(_p(blob), qtype, float(z), H, FF, m, _p(out))
    return out


def expert_ffn(blob, qtype, z, H, FF, x, act=0):
    """act 0: SwiGLU; 1: GeGLU with the tanh form of GELU."""
    x, xd = _xinfo(x)
    T = x.shape[0]
    y = np.empty((T, H), dtype=np.float64)
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    if act == 0:
        rc = lib().oracle_expert_ffn(_p(blob), qtype, float(z), H, FF, _p(x), xd, T, _p(y))
    else:
        rc = lib().oracle_expert_ffn_act(_p(blob), qtype, float(z), H, FF, act, _p(x), xd, T, _p(y))
    if rc:
        raise ValueError("oracle_expert_ffn: invalid arguments")
    return y


def gelu_tanh(v):
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(v)
    lib().oracle_gelu_tanh(_p(v), v.size, _p(out))
    return out


def router_logits(wr_bits, x, norm=False, eps=1e-6, in_scale=None):
    """float64 logits [T][E] = W_r x' with W_r given as bf16 bits [E][H] (uint16)."""
    wr_bits = np.ascontiguousarray(wr_bits, dtype=np.uint16)
    E, H = wr_bits.shape
    x, xd = _xinfo(x)
    T = x.shape[0]
    sc = None if in_scale is None else np.ascontiguousarray(in_scale, dtype=np.float32)
    out = np.empty((T, E), dtype=np.float64)
    rc = lib().oracle_router_logits(_p(wr_bits), E, H, _p(x), xd, T, int(bool(norm)), float(eps),
                                    _p(sc) if sc is not None else None, _p(out))
    if rc:
        raise ValueError("oracle_router_logits: invalid arguments")
    return out


def route_topk(logits, k, renormalize=True):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    rc = lib().oracle_route_topk(_p(logits), T, E, k, int(bool(renormalize)), _p(ids), _p(w))
    if rc:
        raise ValueError("oracle_route_topk: invalid arguments")
    return ids, w


def layer_forward(blobs, k, qtype, z, H, FF, x, logits, shared=None, shared_ff=0, renormalize=True):
    """blobs: list of E uint8 arrays (or a [E, bytes] array)."""
    x, xd = _xinfo(x)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    blob_list = [np.ascontiguousarray(b, dtype=np.uint8) for b in blobs]
    assert len(blob_list) == E
    table = (ctypes.c_void_p * E)(*[b.ctypes.data for b in blob_list])
    y = np.empty((T, H), dtype=np.float64)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    sh = None
    if shared is not None:
        sh = np.ascontiguousarray(shared, dtype=np.uint8)
    rc = lib().oracle_layer_forward(ctypes.cast(table, ctypes.c_void_p), E, k, int(bool(renormalize)), qtype,
                                    float(z), H, FF, _p(sh) if sh is not None else None, shared_ff, _p(x), xd,
                                    _p(logits), T, _p(y), _p(ids), _p(w))
    if rc:
        raise ValueError("oracle_layer_forward: invalid arguments")
    return y, ids, w


def layer_forward_ex(blobs, k, qtype, z, H, FF, x, logits=None, shared=None, shared_ff=0, renormalize=True, act=0,
                     down_scale=None, ids_in=None, w_in=None):
    """The layer with the extended call's options: act (0 SwiGLU, 1 GeGLU-tanh),
    per-expert down_scale [E], and caller-supplied routing ids_in / w_in [T][k]
    (zero-weight slots skipped) instead of logits.  Returns (y, ids, w)."""
    x, xd = _xinfo(x)
    T = x.shape[0]
    E = len(blobs)
    blob_list = [np.ascontiguousarray(b, dtype=np.uint8) for b in blobs]
    table = (ctypes.c_void_p * E)(*[b.ctypes.data for b in blob_list])
    lg = None if logits is None else np.ascontiguousarray(logits, dtype=np.float32)
    ds = None if down_scale is None else np.ascontiguousarray(down_scale, dtype=np.float32)
    ii = None if ids_in is None else np.ascontiguousarray(ids_in, dtype=np.int32)
    wi = None if w_in is None else np.ascontiguousarray(w_in, dtype=np.float32)
    sh = None if shared is None else np.ascontiguousarray(shared, dtype=np.uint8)
    y = np.empty((T, H), dtype=np.float64)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    opt = lambda a: _p(a) if a is not None else None
    rc = lib().oracle_layer_forward_ex(ctypes.cast(table, ctypes.c_void_p), E, k, int(bool(renormalize)), qtype,
                                       float(z), H, FF, act, opt(sh), shared_ff, opt(ds), _p(x), xd, opt(lg),
                                       opt(ii), opt(wi), T, _p(y), _p(ids), _p(w))
    if rc == 2:
        raise ValueError("oracle_layer_forward_ex: a nonzero weight with an expert id outside [0, E)")
    if rc:
        raise ValueError("oracle_layer_forward_ex: invalid arguments")
    return y, ids, w
