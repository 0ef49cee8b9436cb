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


def expert_ffn(blob, qtype, z, H, FF, x):
    x, xd = _xinfo(x)
    T = x.shape[0]
    y = np.empty((T, H), dtype=np.float64)
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    rc = lib().oracle_expert_ffn(_p(blob), qtype, float(z), H, FF, _p(x), xd, T, _p(y))
    if rc:
        raise ValueError("oracle_expert_ffn: invalid arguments")
    return y


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
