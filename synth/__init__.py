"""Seeded synthetic inputs (ctypes wrapper over synth.c).

Holds none of the method's arithmetic: it draws code bytes, fp16 scales,
activations and router logits from a counter-based SplitMix64 generator so the
oracle and the GPU path see identical bytes.  Build with `synth.build()`.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

SHARED_EXPERT = 0xFFFFFF
QK = {"q2": 64, "q4": 32}


def build():
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           os.path.join(_HERE, "synth.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("synth library not built: call synth.build() (or __graft_entry__.build())")
        L = ctypes.CDLL(_LIB_PATH)
        u64, u32, i32, i64, dbl, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_int64,
                                       ctypes.c_double, ctypes.c_void_p)
        L.synth_stream.restype = u64
        L.synth_stream.argtypes = [u32, u32, u32, u32]
        L.synth_word.restype = u64
        L.synth_word.argtypes = [u64, u64, u64]
        L.synth_double_to_f16.restype = ctypes.c_uint16
        L.synth_double_to_f16.argtypes = [dbl]
        L.synth_double_to_bf16.restype = ctypes.c_uint16
        L.synth_double_to_bf16.argtypes = [dbl]
        L.synth_bytes.argtypes = [u64, u64, vp, ctypes.c_size_t]
        L.synth_activations.argtypes = [u64, u32, u32, i64, i64, ctypes.c_int, vp]
        L.synth_popularity_rank.argtypes = [u64, u32, i32, vp]
        L.synth_logits.argtypes = [u64, u32, u32, i64, i32, dbl, vp]
        L.synth_blob_bytes.restype = i64
        L.synth_blob_bytes.argtypes = [i32, i64, i64]
        L.synth_expert_blob.argtypes = [u64, u32, u32, i32, i64, i64, dbl, vp]
        L.synth_expert_blobs.argtypes = [u64, u32, u32, i32, i32, i64, i64, dbl, vp, i64]
        _lib = L
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def blob_bytes(qk, H, FF):
    return int(lib().synth_blob_bytes(qk, H, FF))


def expert_blob(seed, layer, expert, qk, H, FF, sigma):
    """One expert's blob as a uint8 numpy array."""
    out = np.empty(blob_bytes(qk, H, FF), dtype=np.uint8)
    lib().synth_expert_blob(seed, layer, expert, qk, H, FF, sigma, _ptr(out))
    return out


def expert_blobs(seed, layer, e_first, n_exp, qk, H, FF, sigma, out=None):
    """Blobs of experts [e_first, e_first+n_exp) of one layer, shape [n_exp, blob]."""
    nb = blob_bytes(qk, H, FF)
    if out is None:
        out = np.empty((n_exp, nb), dtype=np.uint8)
    assert out.dtype == np.uint8 and out.flags.c_contiguous and out.size >= n_exp * nb
    lib().synth_expert_blobs(seed, layer, e_first, n_exp, qk, H, FF, sigma, _ptr(out), nb)
    return out


def activations(seed, layer, step, T, H, dtype="bf16"):
    """T x H activations: 'bf16' -> uint16 raw bits, 'f32' -> float32."""
    if dtype == "bf16":
        out = np.empty((T, H), dtype=np.uint16)
        lib().synth_activations(seed, layer, step, T, H, 1, _ptr(out))
    else:
        out = np.empty((T, H), dtype=np.float32)
        lib().synth_activations(seed, layer, step, T, H, 0, _ptr(out))
    return out


def logits(seed, layer, step, T, E, zipf_s):
    out = np.empty((T, E), dtype=np.float32)
    lib().synth_logits(seed, layer, step, T, E, float(zipf_s), _ptr(out))
    return out


def popularity_rank(seed, layer, E):
    out = np.empty(E, dtype=np.int32)
    lib().synth_popularity_rank(seed, layer, E, _ptr(out))
    return out


def random_bytes(seed, stream, n):
    out = np.empty(n, dtype=np.uint8)
    lib().synth_bytes(seed, stream, _ptr(out), n)
    return out


def f16_bits(v):
    return int(lib().synth_double_to_f16(float(v)))


def bf16_bits(v):
    return int(lib().synth_double_to_bf16(float(v)))


def bf16_to_f32(bits):
    """Exact widening of raw bf16 bits (uint16 array) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
