"""Test-side helpers: packing codes into the blob format (the inverse of the
decoders under test), plain fp16 scale encoding, and tolerance checks."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


QK = {1: 64, 2: 32}
BITS = {1: 2, 2: 4}


def pack_block(codes, qtype):
    """16 code bytes from qk integer codes: code i goes to byte i*bits//8 at bit
    (i*bits) % 8, lowest bits first (the layout both decoders read)."""
    bits = BITS[qtype]
    out = np.zeros(16, dtype=np.uint8)
    for i, c in enumerate(codes):
        out[(i * bits) // 8] |= np.uint8((int(c) << ((i * bits) % 8)) & 0xFF)
    return out


def pack_matrix(codes, scale_bits, qtype):
    """codes [rows][cols] ints, scale_bits [rows][cols/qk] uint16 -> codes plane + scales plane bytes."""
    qk = QK[qtype]
    rows, cols = codes.shape
    nblk = cols // qk
    cplane = np.zeros((rows, nblk, 16), dtype=np.uint8)
    bits = BITS[qtype]
    per_byte = 8 // bits
    c = codes.reshape(rows, nblk, 16, per_byte).astype(np.uint32)
    acc = np.zeros((rows, nblk, 16), dtype=np.uint32)
    for j in range(per_byte):
        acc |= c[..., j] << (j * bits)
    cplane[:] = acc.astype(np.uint8)
    splane = np.ascontiguousarray(scale_bits, dtype='<u2').view(np.uint8).reshape(-1)
    return np.concatenate([cplane.reshape(-1), splane])


def pack_blob(mats, qtype):
    """mats: [(codes, scale_bits)] for gate, up, down."""
    return np.concatenate([pack_matrix(c, s, qtype) for c, s in mats])


def f16_bits_array(v):
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16_value(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def random_expert(rng, qtype, H, FF, sigma):
    """Random codes and fp16 scales for gate/up/down, plus the dense float64 weights they stand for."""
    qk = QK[qtype]
    z = 1.5 if qtype == 1 else 7.5
    mats, dense = [], []
    for rows, cols in [(FF, H), (FF, H), (H, FF)]:
        codes = rng.integers(0, 1 << BITS[qtype], size=(rows, cols))
        sb = f16_bits_array(np.abs(rng.normal(0, sigma, size=(rows, cols // qk))))
        mats.append((codes, sb))
        dense.append(np.repeat(f16_value(sb), qk, axis=1) * (codes - z))
    return pack_blob(mats, qtype), dense, z


def silu(v):
    return v / (1.0 + np.exp(-v))


def max_err_over_rms(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref)) / rms) if rms > 0 else float(np.max(np.abs(got - ref)))


def bf16_bits_array(v):
    """Round float values to bf16 (nearest-even) and return the raw 16-bit words."""
    f = np.ascontiguousarray(v, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def router_error_bound(wr_bits, xp):
    """A priori bound on the fp32 router logits' error against float64: with
    n = H products summed in fp32 (each FMA rounds once, relative 2^-24), plus
    the few roundings that form x' (norm factor, scale), the error of a logit is
    at most (H + 16) * 2^-24 * sum_h |W[e][h] x'[t][h]| (the recursive-summation
    bound gamma_n, Higham, Accuracy and Stability of Numerical Algorithms, 2002,
    ch. 3).  xp: the exact x' (float64) [T][H]."""
    W = (np.asarray(wr_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    H = W.shape[1]
    return (H + 16) * 2.0 ** -24 * (np.abs(xp) @ np.abs(W).T)
