"""Pins of the float64 oracle against facts the pages and the mathematics fix.

Each test is chosen so that a plausible slip in the oracle (a wrong bit order,
a transposed matrix, a dropped zero point, a sign error in the routing order,
a missing shared term) fails at least one of them.  None of these tests calls
the GPU library.
"""
import math

import numpy as np
import pytest

import oracle
from helpers import (QK, f16_bits_array, f16_value, golden, pack_blob, pack_block, random_expert, silu)


# --- format sizes: the pages' fixed facts ----------------------------------------------------

def test_blob_sizes_match_page_facts():
    g = golden("format_facts.json")
    q2 = g["q2_blob"]
    nb = oracle.blob_bytes(q2["qtype"], q2["H"], q2["FF"])
    assert nb == q2["bytes"] == 1382400
    assert nb * 8 / (3 * q2["H"] * q2["FF"]) == q2["bits_per_weight"]
    f = g["q2_layer_512_experts_MB"]
    assert abs(f["experts"] * nb / 1e6 - f["approx_MB"]) / f["approx_MB"] < f["rel_tol"]
    f = g["q2_arena_GB"]
    assert abs(f["layers"] * f["experts"] * nb / 1e9 - f["approx_GB"]) / f["approx_GB"] < f["rel_tol"]
    f = g["q2_token_480_experts_GB"]
    assert abs(f["experts"] * nb / 1e9 - f["approx_GB"]) / f["approx_GB"] < f["rel_tol"]
    f = g["q4_gemma_arena_GB"]
    nb4 = oracle.blob_bytes(f["qtype"], f["H"], f["FF"])
    assert nb4 == 3345408
    assert nb4 * 8 / (3 * f["H"] * f["FF"]) == 4.5
    assert abs(f["layers"] * f["experts"] * nb4 / 1e9 - f["approx_GB"]) / f["approx_GB"] < f["rel_tol"]


def test_blob_sizes_other_shapes():
    assert oracle.blob_bytes(1, 256, 128) == 27648           # 3 * 256*128/64 * 18
    assert oracle.blob_bytes(2, 2816, 2112) == 10036224      # shared expert of the 4-bit decode shape
    assert oracle.blob_bytes(2, 7168, 2048) == 24772608      # prefill shape
    assert oracle.blob_bytes(3, 256, 128) == -1              # unknown qtype


# --- block decoding: hand-built blocks ------------------------------------------------------

def _one_block_blob(qtype, block_bytes, scale_bits):
    """A blob with H = FF = qk whose gate row 0 is the given block; the rest is zero."""
    qk = QK[qtype]
    parts = []
    for m in range(3):
        cp = np.zeros((qk, 1, 16), dtype=np.uint8)
        sp = np.zeros((qk, 1), dtype='<u2')
        if m == 0:
            cp[0, 0] = block_bytes
            sp[0, 0] = scale_bits
        parts += [cp.reshape(-1), sp.view(np.uint8).reshape(-1)]
    return np.concatenate(parts), qk


def test_q2_block_golden():
    g = golden("q2_block.json")
    blk = np.frombuffer(bytes.fromhex(g["bytes_hex"]), dtype=np.uint8)
    for case in g["cases"]:
        blob, qk = _one_block_blob(1, blk, int(case["scale_bits"], 16))
        W = oracle.dequant_matrix(blob, 1, case["z"], qk, qk, 0)
        row = W[0]
        assert list(row[:16]) == case["weights_head16"]
        assert np.all(row[16:] == case["weight_rest"])
        # the page's own mapping: w = scale * (code - z), codes as listed in the fixture
        assert np.array_equal(row, case["scale"] * (np.array(g["codes"], dtype=np.float64) - case["z"]))


def test_q2_page_mapping_codes_0123_mean_minus1_to_2():
    """Codes {0,1,2,3} read as {-1,0,1,2} x scale with the page's offset of 1."""
    blk = pack_block([0, 1, 2, 3] * 16, 1)
    assert blk[0] == 0xE4
    blob, qk = _one_block_blob(1, blk, 0x3C00)
    assert list(oracle.dequant_matrix(blob, 1, 1.0, qk, qk, 0)[0][:4]) == [-1.0, 0.0, 1.0, 2.0]
    assert list(oracle.dequant_matrix(blob, 1, 1.5, qk, qk, 0)[0][:4]) == [-1.5, -0.5, 0.5, 1.5]


def test_q4_block_golden():
    g = golden("q4_block.json")
    blk = np.frombuffer(bytes.fromhex(g["bytes_hex"]), dtype=np.uint8)
    for case in g["cases"]:
        blob, qk = _one_block_blob(2, blk, int(case["scale_bits"], 16))
        W = oracle.dequant_matrix(blob, 2, case["z"], qk, qk, 0)
        assert list(W[0]) == [float(v) for v in case["weights"]]
        assert np.all(W[1:] == 0.0)


def test_all_zero_codes_give_minus_z_times_scale():
    for qtype, z in [(1, 1.5), (2, 7.5)]:
        blob, qk = _one_block_blob(qtype, np.zeros(16, np.uint8), 0x3555)   # 0x3555 = 0.333251953125
        s = 0.333251953125
        assert np.all(oracle.dequant_matrix(blob, qtype, z, qk, qk, 0)[0] == -z * s)


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(7)
    for qtype, H, FF in [(1, 128, 192), (2, 96, 64)]:
        qk = QK[qtype]
        mats = []
        codes_list = []
        for rows, cols in [(FF, H), (FF, H), (H, FF)]:
            c = rng.integers(0, 4 if qtype == 1 else 16, size=(rows, cols))
            codes_list.append(c)
            mats.append((c, np.full((rows, cols // qk), 0x3C00, dtype=np.uint16)))
        blob = pack_blob(mats, qtype)
        assert blob.size == oracle.blob_bytes(qtype, H, FF)
        for m in range(3):
            W = oracle.dequant_matrix(blob, qtype, 0.0, H, FF, m)
            assert np.array_equal(W, codes_list[m].astype(np.float64))


def test_word_based_unpack_of_the_page_equals_byte_based():
    """The page unpacks 64 codes from 8 little-endian 16-bit words, 8 codes per
    word; the oracle reads byte i/4 at bit 2*(i%4).  Both readings must agree."""
    rng = np.random.default_rng(3)
    raw = rng.integers(0, 256, size=16, dtype=np.uint8)
    words = raw.view('<u2')
    by_word = [(int(words[i]) >> (2 * j)) & 3 for i in range(8) for j in range(8)]
    blob, qk = _one_block_blob(1, raw, 0x3C00)
    got = oracle.dequant_matrix(blob, 1, 0.0, qk, qk, 0)[0]
    assert list(got) == [float(c) for c in by_word]


# --- top-k routing ----------------------------------------------------------------------------

def _brute_force_ids(l, k):
    """Full stable sort by (logit descending, index ascending); NaN last."""
    def key(e):
        v = float(l[e])
        return (1, 0.0, e) if math.isnan(v) else (0, -v, e)
    return sorted(range(len(l)), key=key)[:k]


def test_topk_equals_brute_force_full_sort():
    rng = np.random.default_rng(11)
    for E, k in [(8, 2), (64, 6), (512, 10), (128, 8), (256, 8), (16, 16), (33, 1)]:
        T = 40
        # few distinct values so that ties are common
        l = rng.integers(-4, 5, size=(T, E)).astype(np.float32) * np.float32(0.25)
        l[0] = rng.normal(size=E).astype(np.float32)
        ids, w = oracle.route_topk(l, k)
        for t in range(T):
            assert list(ids[t]) == _brute_force_ids(l[t], k)


def test_topk_special_cases():
    # k = E returns every expert in key order
    l = np.array([[0.5, -1.0, 2.0, 0.5, 3.0]], dtype=np.float32)
    ids, _ = oracle.route_topk(l, 5)
    assert list(ids[0]) == [4, 2, 0, 3, 1]
    # k = 1 is the argmax, lowest index on ties
    l = np.array([[1.0, 7.0, 7.0, -3.0]], dtype=np.float32)
    assert oracle.route_topk(l, 1)[0][0, 0] == 1
    # all-equal logits: ids 0..k-1 and weights exactly 1/k
    for k in (1, 3, 8):
        ids, w = oracle.route_topk(np.full((2, 16), 0.75, dtype=np.float32), k)
        assert list(ids[0]) == list(range(k))
        assert np.all(w == 1.0 / k)
    # -0 and +0 tie: the lower index wins whichever sign it carries
    l = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], dtype=np.float32)
    ids, w = oracle.route_topk(l, 2)
    assert list(ids[0]) == [0, 1] and list(ids[1]) == [0, 1]
    assert np.all(w == 0.5)
    # NaN ranks below every number, -inf included
    l = np.array([[np.nan, -np.inf, 1.0, np.nan]], dtype=np.float32)
    ids, _ = oracle.route_topk(l, 4)
    assert list(ids[0]) == [2, 1, 0, 3]


def test_topk_all_neg_inf_selection_gets_equal_weights():
    """Reading (ties, -0, NaN): a selection whose top logit is -inf gets equal
    weights.  Pinned to the limit it extends: k equal finite logits c give
    exactly 1/k whatever c (every term is exp(0)), so equal weights are the
    value of the softmax as c -> -inf; with renormalize = 0 the same limit over
    all E logits gives 1/E."""
    E = 6
    for k in (1, 3, 6):
        l = np.full((2, E), -np.inf, dtype=np.float32)
        ids, w = oracle.route_topk(l, k)
        assert list(ids[0]) == list(range(k))            # all tied: lowest indices first
        assert np.all(w == 1.0 / k)
        for c in (-1e3, -1e30, float(np.finfo(np.float32).min)):
            _, wc = oracle.route_topk(np.full((2, E), c, dtype=np.float32), k)
            assert np.array_equal(wc, w)
        _, w0 = oracle.route_topk(l, k, renormalize=False)
        assert np.all(w0 == 1.0 / E)
    # -inf on top and NaN below: the -inf experts first (by index), then the
    # NaNs; the whole selection gets equal weights
    l = np.array([[np.nan, -np.inf, np.nan, -np.inf]], dtype=np.float32)
    ids, w = oracle.route_topk(l, 3)
    assert list(ids[0]) == [1, 3, 0]
    assert np.all(w == 1.0 / 3)


def test_topk_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.route_topk(np.zeros((1, 4), np.float32), 5)
    with pytest.raises(ValueError):
        oracle.route_topk(np.zeros((1, 4), np.float32), 0)


def test_weights_sum_to_one_and_equal_renormalised_full_softmax():
    rng = np.random.default_rng(5)
    l = (rng.normal(size=(64, 512)) * 3).astype(np.float32)
    ids, w = oracle.route_topk(l, 10)
    assert np.all(np.abs(w.sum(1) - 1.0) < 1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)          # rank order = weight order
    full = np.exp(l.astype(np.float64) - l.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, ids.astype(np.int64), 1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-12, atol=0)
    # without renormalisation the weights are the full softmax at the selected experts
    _, w0 = oracle.route_topk(l, 10, renormalize=False)
    np.testing.assert_allclose(w0, sel, rtol=1e-12, atol=0)


# --- the expert FFN ---------------------------------------------------------------------------

def test_expert_ffn_equals_dense_matrix_product():
    rng = np.random.default_rng(21)
    for qtype, H, FF, T in [(1, 256, 128, 4), (2, 96, 160, 3), (1, 192, 64, 2)]:
        blob, (Wg, Wu, Wd), z = random_expert(rng, qtype, H, FF, 0.05)
        x = rng.normal(size=(T, H)).astype(np.float32)
        y = oracle.expert_ffn(blob, qtype, z, H, FF, x)
        X = x.astype(np.float64)
        ref = (silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T
        np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


def test_expert_ffn_bf16_input_is_exact_widening():
    rng = np.random.default_rng(22)
    H, FF = 128, 64
    blob, (Wg, Wu, Wd), z = random_expert(rng, 1, H, FF, 0.05)
    bits = rng.integers(0, 1 << 16, size=(2, H), dtype=np.uint16)
    bits = (bits & 0x3FFF) | 0x3C00 * (bits & 1)          # finite, moderate values
    x32 = (bits.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(oracle.expert_ffn(blob, 1, z, H, FF, bits), oracle.expert_ffn(blob, 1, z, H, FF, x32))


def test_expert_ffn_one_hot_closed_form():
    """z = 1, code 2 = +scale and code 1 = 0: one-hot rows make every projection a
    permutation, so y_j = s_d * silu(s_g x[pi(rho(j))]) * s_u x[sigma(rho(j))]."""
    rng = np.random.default_rng(9)
    H, FF = 128, 64
    pi, sg_perm, rho = rng.permutation(H)[:FF], rng.permutation(H)[:FF], rng.integers(0, FF, size=H)
    s_g, s_u, s_d = 0.5, 0.25, 2.0
    mats = []
    for rows, cols, hot, s in [(FF, H, pi, s_g), (FF, H, sg_perm, s_u), (H, FF, rho, s_d)]:
        codes = np.ones((rows, cols), dtype=np.int64)
        codes[np.arange(rows), hot] = 2
        mats.append((codes, np.full((rows, cols // 64), f16_bits_array(s)[()], dtype=np.uint16)))
    blob = pack_blob(mats, 1)
    x = rng.normal(size=(1, H)).astype(np.float32)
    y = oracle.expert_ffn(blob, 1, 1.0, H, FF, x)[0]
    X = x[0].astype(np.float64)
    for j in range(H):
        f = rho[j]
        g = s_g * X[pi[f]]
        u = s_u * X[sg_perm[f]]
        assert abs(y[j] - s_d * (g / (1 + math.exp(-g))) * u) <= 1e-14 * max(1.0, abs(y[j]))


def test_expert_ffn_brute_force_from_bytes():
    """Pure-Python loops over the blob bytes (word-based unpack, as on the page)."""
    rng = np.random.default_rng(4)
    H, FF = 64, 64
    blob = rng.integers(0, 256, size=oracle.blob_bytes(1, H, FF), dtype=np.uint8)
    # keep scales finite and small: overwrite each scales plane with |N(0,0.05)| fp16
    off = 0
    for rows in (FF, FF, H):
        nb = rows * 1
        off += nb * 16
        blob[off:off + 2 * nb] = f16_bits_array(np.abs(rng.normal(0, 0.05, nb))).view(np.uint8)
        off += 2 * nb
    x = rng.normal(size=(1, H)).astype(np.float32)[0].astype(np.float64)

    def weight(m_off, rows, r, k):
        codes = blob[m_off + r * 16: m_off + r * 16 + 16]
        word = int(codes[2 * (k // 8)]) | (int(codes[2 * (k // 8) + 1]) << 8)
        c = (word >> (2 * (k % 8))) & 3
        sbits = int(blob[m_off + rows * 16 + 2 * r]) | (int(blob[m_off + rows * 16 + 2 * r + 1]) << 8)
        s = float(np.array([sbits], dtype=np.uint16).view(np.float16)[0])
        return s * (c - 1.5)

    offs = [0, FF * 18, 2 * FF * 18]
    g = [sum(weight(offs[0], FF, f, k) * x[k] for k in range(H)) for f in range(FF)]
    u = [sum(weight(offs[1], FF, f, k) * x[k] for k in range(H)) for f in range(FF)]
    a = [gi / (1 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
    y = [sum(weight(offs[2], H, j, f) * a[f] for f in range(FF)) for j in range(H)]
    got = oracle.expert_ffn(blob, 1, 1.5, H, FF, x.astype(np.float32)[None])[0]
    np.testing.assert_allclose(got, y, rtol=1e-12, atol=1e-14)


# --- the layer --------------------------------------------------------------------------------

def _layer_inputs(rng, qtype, E, H, FF, T, sigma=0.05):
    blobs, denses = [], []
    for _ in range(E):
        b, d, z = random_expert(rng, qtype, H, FF, sigma)
        blobs.append(b)
        denses.append(d)
    x = rng.normal(size=(T, H)).astype(np.float32)
    logits = rng.normal(size=(T, E)).astype(np.float32)
    return blobs, denses, z, x, logits


def test_layer_equals_weighted_sum_of_dense_experts():
    rng = np.random.default_rng(31)
    E, k, H, FF, T = 8, 3, 128, 64, 5
    blobs, dens, z, x, logits = _layer_inputs(rng, 1, E, H, FF, T)
    y, ids, w = oracle.layer_forward(blobs, k, 1, z, H, FF, x, logits)
    X = x.astype(np.float64)
    for t in range(T):
        ref = np.zeros(H)
        for j in range(k):
            Wg, Wu, Wd = dens[ids[t, j]]
            ref += w[t, j] * (Wd @ (silu(Wg @ X[t]) * (Wu @ X[t])))
        np.testing.assert_allclose(y[t], ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())


def test_layer_identical_experts_ignore_routing():
    rng = np.random.default_rng(32)
    E, k, H, FF, T = 6, 2, 64, 64, 3
    b, _, z = random_expert(rng, 1, H, FF, 0.05)
    x = rng.normal(size=(T, H)).astype(np.float32)
    y_one = oracle.expert_ffn(b, 1, z, H, FF, x)
    for seed in range(3):
        logits = np.random.default_rng(seed).normal(size=(T, E)).astype(np.float32)
        y, _, _ = oracle.layer_forward([b] * E, k, 1, z, H, FF, x, logits)
        np.testing.assert_allclose(y, y_one, rtol=1e-12, atol=1e-14)


def test_layer_permutation_equivariance():
    rng = np.random.default_rng(33)
    E, k, H, FF, T = 8, 3, 64, 64, 4
    blobs, _, z, x, logits = _layer_inputs(rng, 1, E, H, FF, T)
    y, ids, w = oracle.layer_forward(blobs, k, 1, z, H, FF, x, logits)
    perm = rng.permutation(E)               # new expert i is old expert perm[i]
    y2, ids2, w2 = oracle.layer_forward([blobs[p] for p in perm], k, 1, z, H, FF, x, logits[:, perm])
    np.testing.assert_array_equal(perm[ids2], ids)
    np.testing.assert_array_equal(w2, w)
    np.testing.assert_array_equal(y2, y)


def _double_down_scales(blob, qtype, H, FF):
    """Double every down-projection scale exactly (fp16 exponent + 1, or 2x a subnormal mantissa)."""
    qk = QK[qtype]
    b = blob.copy()
    off = 2 * FF * (H // qk) * 18 + H * (FF // qk) * 16
    sc = b[off: off + 2 * H * (FF // qk)].view('<u2')
    exp = (sc >> 10) & 31
    assert np.all(exp < 30)
    sc[:] = np.where(exp == 0, (sc & 0x8000) | ((sc & 0x3FF) << 1), sc + 0x400)
    return b


def test_layer_doubling_down_scales_doubles_output_exactly():
    rng = np.random.default_rng(34)
    E, k, H, FF, T = 4, 2, 64, 64, 3
    blobs, _, z, x, logits = _layer_inputs(rng, 2, E, H, FF, T, sigma=0.02)
    y, _, _ = oracle.layer_forward(blobs, k, 2, z, H, FF, x, logits)
    y2, _, _ = oracle.layer_forward([_double_down_scales(b, 2, H, FF) for b in blobs], k, 2, z, H, FF, x, logits)
    np.testing.assert_array_equal(y2, 2.0 * y)


def test_layer_shared_expert_is_added():
    rng = np.random.default_rng(35)
    E, k, H, FF, T = 4, 2, 64, 64, 2
    b, _, z = random_expert(rng, 2, H, FF, 0.02)
    x = rng.normal(size=(T, H)).astype(np.float32)
    logits = rng.normal(size=(T, E)).astype(np.float32)
    y1 = oracle.expert_ffn(b, 2, z, H, FF, x)
    # every routed expert and the shared expert equal: y = 2 * expert(x)
    y, _, _ = oracle.layer_forward([b] * E, k, 2, z, H, FF, x, logits, shared=b, shared_ff=FF)
    np.testing.assert_allclose(y, 2 * y1, rtol=1e-12, atol=1e-14)
    # a shared expert with zero scales adds nothing; a wider shared expert adds its own FFN
    bs, _, _ = random_expert(rng, 2, H, 3 * FF, 0.02)
    yr, _, _ = oracle.layer_forward([b] * E, k, 2, z, H, FF, x, logits)
    ys, _, _ = oracle.layer_forward([b] * E, k, 2, z, H, FF, x, logits, shared=bs, shared_ff=3 * FF)
    np.testing.assert_allclose(ys - yr, oracle.expert_ffn(bs, 2, z, H, 3 * FF, x), rtol=1e-10, atol=1e-13)
    zero = bs.copy()
    zero[:] = 0
    y0, _, _ = oracle.layer_forward([b] * E, k, 2, z, H, FF, x, logits, shared=zero, shared_ff=3 * FF)
    np.testing.assert_array_equal(y0, yr)


# --- Gemma-faithful options: GeGLU (tanh GELU), per-expert down scale ---------------------------

def test_gelu_tanh_against_library_and_identities():
    """kairos-engine README ("Decode, 2026-09-28/29"): the model's GELU is the tanh
    form.  Pinned to torch's own tanh-approximate GELU in float64, to the
    identity gelu(v) - gelu(-v) = v that the tanh form keeps exactly, and to its
    distance from the erf GELU (a few 1e-4 at most)."""
    import torch
    from scipy.special import erf
    v = np.concatenate([np.linspace(-12, 12, 4001), [0.0, -0.0, 1e-12, -1e-12, 30.0, -30.0, 1e4, -1e4]])
    g = oracle.gelu_tanh(v)
    ref = torch.nn.functional.gelu(torch.from_numpy(v), approximate="tanh").numpy()
    np.testing.assert_allclose(g, ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(g - oracle.gelu_tanh(-v), v, rtol=1e-13, atol=1e-15)
    assert g[v == 0.0].tolist() == [0.0, 0.0, 0.0]
    exact = 0.5 * v * (1.0 + erf(v / np.sqrt(2.0)))
    assert np.max(np.abs(g - exact)) < 5e-4


def test_expert_ffn_geglu_equals_dense_product():
    import torch
    rng = np.random.default_rng(31)
    for qtype, H, FF in [(1, 128, 64), (2, 96, 64)]:
        blob, (Wg, Wu, Wd), z = random_expert(rng, qtype, H, FF, 0.1)
        x = rng.normal(size=(3, H)).astype(np.float32)
        xd = x.astype(np.float64)
        g = xd @ Wg.T
        a = torch.nn.functional.gelu(torch.from_numpy(g), approximate="tanh").numpy() * (xd @ Wu.T)
        np.testing.assert_allclose(oracle.expert_ffn(blob, qtype, z, H, FF, x, act=1), a @ Wd.T, rtol=1e-10,
                                   atol=1e-12)
        # act 0 of the extended function is the SwiGLU FFN, bit for bit
        np.testing.assert_array_equal(oracle.expert_ffn(blob, qtype, z, H, FF, x, act=0),
                                      oracle.expert_ffn(blob, qtype, z, H, FF, x))


def _small_layer_blobs(rng, E, qtype, H, FF, sigma):
    blobs, dense = [], []
    for _ in range(E):
        b, d, z = random_expert(rng, qtype, H, FF, sigma)
        blobs.append(b)
        dense.append(d)
    return blobs, dense, z


def test_layer_down_scale_per_expert():
    """kairos-engine README ("The MoE forward"): the down projection's scale is
    per expert.  Pins: scale 1 everywhere is the plain layer bit for bit; scale 2
    everywhere doubles y exactly; random scales equal sum_j w_j s_{e_j} y_{e_j}
    over dense experts."""
    rng = np.random.default_rng(41)
    E, k, H, FF = 8, 3, 128, 64
    blobs, dense, z = _small_layer_blobs(rng, E, 1, H, FF, 0.05)
    x = rng.normal(size=(4, H)).astype(np.float32)
    lg = rng.normal(size=(4, E)).astype(np.float32)
    y0, ids, w = oracle.layer_forward(blobs, k, 1, z, H, FF, x, lg)
    y1, _, _ = oracle.layer_forward_ex(blobs, k, 1, z, H, FF, x, lg, down_scale=np.ones(E))
    np.testing.assert_array_equal(y1, y0)
    y2, _, _ = oracle.layer_forward_ex(blobs, k, 1, z, H, FF, x, lg, down_scale=np.full(E, 2.0))
    np.testing.assert_array_equal(y2, 2.0 * y0)
    s = rng.uniform(0.2, 3.0, size=E).astype(np.float32)
    ys, _, _ = oracle.layer_forward_ex(blobs, k, 1, z, H, FF, x, lg, down_scale=s, act=1)
    import torch
    xd = x.astype(np.float64)
    ref = np.zeros((4, H))
    for t in range(4):
        for j in range(k):
            Wg, Wu, Wd = dense[ids[t, j]]
            a = torch.nn.functional.gelu(torch.from_numpy(Wg @ xd[t]), approximate="tanh").numpy() * (Wu @ xd[t])
            ref[t] += w[t, j] * float(s[ids[t, j]]) * (Wd @ a)
    np.testing.assert_allclose(ys, ref, rtol=1e-10, atol=1e-12)


# --- fixed top-k shape: caller-supplied routing, zero-weight slots skipped ------------------------

def test_routed_zero_weight_slot_is_skipped():
    """Krasis white paper 7.5: an omitted route keeps its slot with a dummy
    expert and a zero weight, and no expert work is done for it.  A dummy
    blob with NaN scales behind zero-weight slots (and an id outside [0, E))
    leaves y finite and equal to the dense sum over the remaining slots; all
    weights zero give y = 0 exactly; a nonzero weight on an id outside [0, E)
    is rejected."""
    rng = np.random.default_rng(43)
    E, k, H, FF = 6, 4, 128, 64
    blobs, dense, z = _small_layer_blobs(rng, E, 1, H, FF, 0.05)
    poison = blobs[5].copy()
    nb = FF * (H // 64)
    poison[nb * 16:nb * 18] = np.frombuffer(np.full(nb, 0x7E00, dtype='<u2').tobytes(), dtype=np.uint8)   # NaN scales
    blobs[5] = poison
    x = rng.normal(size=(3, H)).astype(np.float32)
    ids = np.array([[2, 5, 0, 5], [1, 3, 9, 4], [5, 5, 5, 5]], dtype=np.int32)
    w = np.array([[0.5, 0.0, 0.25, 0.0], [0.4, 0.3, 0.0, 0.3], [0, 0, 0, 0]], dtype=np.float32)
    y, ids_o, w_o = oracle.layer_forward_ex(blobs, k, 1, z, H, FF, x, ids_in=ids, w_in=w)
    assert np.all(np.isfinite(y))
    np.testing.assert_array_equal(ids_o, ids)
    xd = x.astype(np.float64)
    ref = np.zeros((3, H))
    for t in range(3):
        for j in range(k):
            if w[t, j] != 0:
                Wg, Wu, Wd = dense[ids[t, j]]
                ref[t] += float(w[t, j]) * (Wd @ ((Wg @ xd[t]) / (1 + np.exp(-(Wg @ xd[t]))) * (Wu @ xd[t])))
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)
    assert np.all(y[2] == 0.0)
    with pytest.raises(ValueError):
        oracle.layer_forward_ex(blobs, k, 1, z, H, FF, x, ids_in=np.where(ids == 9, 7, ids),
                                w_in=np.where(ids == 9, 0.2, w).astype(np.float32))


def test_routed_equals_logit_routing_with_the_same_weights():
    """Routing supplied as the oracle's own top-k ids and weights (rounded to
    fp32) gives the logit-routed layer up to that rounding."""
    rng = np.random.default_rng(47)
    E, k, H, FF = 16, 4, 96, 64
    blobs, _, z = _small_layer_blobs(rng, E, 2, H, FF, 0.02)
    x = rng.normal(size=(5, H)).astype(np.float32)
    lg = rng.normal(size=(5, E)).astype(np.float32)
    y0, ids, w = oracle.layer_forward(blobs, k, 2, z, H, FF, x, lg)
    y1, _, _ = oracle.layer_forward_ex(blobs, k, 2, z, H, FF, x, ids_in=ids, w_in=w.astype(np.float32))
    np.testing.assert_allclose(y1, y0, rtol=1e-6, atol=1e-6 * np.abs(y0).max())


# --- router GEMV front end -----------------------------------------------------------------------

def test_router_logits_equal_dense_product_and_norm_properties():
    """kairos-engine README ("The MoE forward"): the router GEMM gives the logits,
    reading its input through its own weightless norm and a per-input-dim scale.
    Pins: without the norm the logits equal a dense float64 product with the
    bf16 weights; with identity weights the logits are x' itself, which with the
    norm (eps 0) has unit mean square, is proportional to x and is invariant to
    scaling x by 4 (exact in binary floating point); the per-input-dim scale
    multiplies x' element by element."""
    import synth
    rng = np.random.default_rng(53)
    E, H, T = 24, 160, 3
    wr = np.array([synth.bf16_bits(v) for v in rng.normal(0, 0.05, size=E * H)], dtype=np.uint16).reshape(E, H)
    xb = np.array([synth.bf16_bits(v) for v in rng.normal(size=T * H)], dtype=np.uint16).reshape(T, H)
    W = synth.bf16_to_f32(wr).astype(np.float64)
    X = synth.bf16_to_f32(xb).astype(np.float64)
    np.testing.assert_allclose(oracle.router_logits(wr, xb), X @ W.T, rtol=1e-12, atol=1e-14)
    xf = rng.normal(size=(T, H)).astype(np.float32)
    np.testing.assert_allclose(oracle.router_logits(wr, xf), xf.astype(np.float64) @ W.T, rtol=1e-12, atol=1e-14)
    one = synth.bf16_bits(1.0)
    ident = np.zeros((H, H), dtype=np.uint16)
    ident[np.arange(H), np.arange(H)] = one
    xn = oracle.router_logits(ident, xf, norm=True, eps=0.0)
    np.testing.assert_allclose(np.mean(xn ** 2, axis=1), 1.0, rtol=1e-14)
    ratio = xn / xf.astype(np.float64)
    np.testing.assert_allclose(ratio, ratio[:, :1] * np.ones((1, H)), rtol=1e-14)
    np.testing.assert_array_equal(oracle.router_logits(ident, 4 * xf, norm=True, eps=0.0), xn)
    sc = rng.uniform(0.5, 2.0, size=H).astype(np.float32)
    np.testing.assert_allclose(oracle.router_logits(ident, xf, norm=True, eps=0.0, in_scale=sc),
                               xn * sc.astype(np.float64), rtol=1e-15)
    # eps only ever lowers |x'|
    assert np.all(np.abs(oracle.router_logits(ident, xf, norm=True, eps=1e-2)) <= np.abs(xn))
