"""GPU parity: the HIP path through the C ABI against the float64 oracle on the
same seeded inputs.  Expert ids must match exactly, routing weights within
1e-6, layer outputs within max|err| <= 2e-3 * rms(oracle output)."""
import numpy as np
import pytest
import torch

import bit_expert_ffn_amd as moe
import oracle
import synth
from helpers import f16_bits_array, max_err_over_rms, random_expert
from synth import workloads as wl

pytestmark = pytest.mark.gpu
TOL = 2e-3
DEV = "cuda"


def _bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _x_tensor(x):
    return _bf16_tensor(x) if x.dtype == np.uint16 else torch.from_numpy(x).to(DEV)


# --- routing ------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(1, 512, 10), (8, 512, 10), (5, 128, 8), (64, 256, 8), (3, 8, 2), (2, 1024, 32),
                                   (4, 64, 64 // 2), (7, 33, 33 // 2), (1, 1, 1), (3, 16, 16)])
def test_route_topk_matches_oracle(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    l = rng.integers(-3, 4, size=(T, E)).astype(np.float32) * np.float32(0.5)   # many ties
    l[0] = rng.normal(size=E).astype(np.float32)
    for renorm in (True, False):
        ids_ref, w_ref = oracle.route_topk(l, k, renorm)
        ids, w = moe.route_topk(torch.from_numpy(l).to(DEV), k, renorm)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
        assert np.max(np.abs(w.cpu().numpy() - w_ref)) <= 1e-6


def test_route_topk_special_values():
    l = np.array([[-0.0, 0.0, -1.0, np.nan, -np.inf, 2.0],
                  [np.nan, np.nan, -np.inf, -np.inf, np.nan, -np.inf],
                  [0.0, -0.0, 0.0, -0.0, 0.0, -0.0],
                  [-np.inf] * 6], dtype=np.float32)
    for k in (1, 3, 6):
        ids_ref, w_ref = oracle.route_topk(l, k)
        ids, w = moe.route_topk(torch.from_numpy(l).to(DEV), k)
        np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
        wg = w.cpu().numpy()
        finite = np.isfinite(w_ref)
        assert np.array_equal(np.isfinite(wg), finite)
        assert np.max(np.abs(wg[finite] - w_ref[finite])) <= 1e-6


def _top_heavy_rows(E, k, seed):
    """Logit rows built around how many logits reach the k-th largest maximum of
    the 64 strided lanes (lane l holds experts l, l + 64, ...): the largest
    logits crowded into one lane, exactly 64 and 65 logits tied at the top, and
    ties on a value just below a few clear winners."""
    rng = np.random.default_rng(seed)
    base = rng.normal(size=E).astype(np.float32)
    assert base.max() < 6.0
    per_lane = E // 64
    rows = []
    a = base.copy()
    a[3 + 64 * np.arange(per_lane)] = 10.0 + np.arange(per_lane, dtype=np.float32)
    rows.append(a)
    for n_tied in (64, 65):
        b = base.copy()
        b[rng.choice(E, n_tied, replace=False)] = 7.0
        rows.append(b)
    d = base.copy()
    d[rng.choice(E, 3 * k, replace=False)] = 5.5
    d[rng.choice(E, k // 2, replace=False)] = 9.0
    rows.append(d)
    e = base.copy()
    e[64 * np.arange(per_lane)] = 8.0          # lane 0 holds a tied block
    e[1 + 64 * np.arange(per_lane)] = 8.0      # and lane 1 another
    rows.append(e)
    return np.stack(rows)


@pytest.mark.parametrize("E,k", [(512, 10), (1024, 32), (256, 8), (128, 2)])
def test_route_topk_crowded_and_tied_tops(E, k):
    l = _top_heavy_rows(E, k, E + k)
    for renorm in (True, False):
        ids_ref, w_ref = oracle.route_topk(l, k, renorm)
        ids, w = moe.route_topk(torch.from_numpy(l).to(DEV), k, renorm)
        np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
        assert np.max(np.abs(w.cpu().numpy() - w_ref)) <= 1e-6


def test_layer_routing_crowded_and_tied_tops():
    """The fused decode kernel's own routing (T = 1 and a window of 5) on the same rows."""
    E, k, H, FF = 512, 10, 256, 128
    l = _top_heavy_rows(E, k, 5)
    rng = np.random.default_rng(11)
    blob = torch.from_numpy(random_expert(rng, 1, H, FF, 0.05)[0]).to(DEV)
    table = torch.full((E,), blob.data_ptr(), dtype=torch.int64, device=DEV)
    desc = moe.layer_desc(H, FF, 1, 1.5, E, k)
    x = torch.from_numpy(rng.normal(size=(l.shape[0], H)).astype(np.float32)).to(DEV)
    ids_ref, w_ref = oracle.route_topk(l, k, True)
    for rows in [[t] for t in range(l.shape[0])] + [list(range(l.shape[0]))]:
        T = len(rows)
        ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
        wts = torch.empty((T, k), dtype=torch.float32, device=DEV)
        moe.layer_forward(desc, table, x[rows].contiguous(), torch.from_numpy(l[rows]).to(DEV), ids=ids,
                          weights=wts)
        np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref[rows])
        assert np.max(np.abs(wts.cpu().numpy() - w_ref[rows])) <= 1e-6


def test_route_topk_zipf_logits():
    for s, E, k in [(1.0, 512, 10), (0.8, 128, 8), (0.6, 256, 8)]:
        l = synth.logits(0, 3, 0, 300, E, s)
        ids_ref, w_ref = oracle.route_topk(l, k)
        ids, w = moe.route_topk(torch.from_numpy(l).to(DEV), k)
        np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
        assert np.max(np.abs(w.cpu().numpy() - w_ref)) <= 1e-6


# --- block decoding ---------------------------------------------------------------------------

@pytest.mark.parametrize("qtype,H,FF", [(1, 256, 128), (2, 96, 64), (1, 2560, 640)])
def test_dequant_matches_oracle_exactly(qtype, H, FF):
    z = 1.5 if qtype == 1 else 7.5
    blob = synth.expert_blob(5, 0, 1, 64 if qtype == 1 else 32, H, FF, 0.05)
    # plant special scales: zero, the smallest subnormal, a mid subnormal, the largest finite
    nb = FF * (H // (64 if qtype == 1 else 32))
    sc = blob[nb * 16: nb * 18].view('<u2')
    sc[:4] = [0x0000, 0x0001, 0x0155, 0x7BFF]
    d = moe.expert_desc(H, FF, qtype, z)
    dev = torch.from_numpy(blob).to(DEV)
    for m in range(3):
        got = moe.dequant_matrix(d, dev, m).cpu().numpy().astype(np.float64)
        np.testing.assert_array_equal(got, oracle.dequant_matrix(blob, qtype, z, H, FF, m))


# --- one expert --------------------------------------------------------------------------------

@pytest.mark.parametrize("qtype,H,FF", [(1, 256, 128), (2, 256, 128), (1, 2560, 640), (2, 2816, 704),
                                        (2, 2816, 2112), (1, 192, 320), (2, 7168, 2048)])
@pytest.mark.parametrize("T", [1, 2, 3, 8])
@pytest.mark.parametrize("xd", ["bf16", "f32"])
def test_expert_ffn_matches_oracle(qtype, H, FF, T, xd):
    z = 1.5 if qtype == 1 else 7.5
    qk = 64 if qtype == 1 else 32
    blob = synth.expert_blob(7, 1, T, qk, H, FF, 0.05 if qtype == 1 else 0.02)
    x = synth.activations(7, 1, T, T, H, xd)
    d = moe.expert_desc(H, FF, qtype, z)
    y = moe.expert_ffn(d, torch.from_numpy(blob).to(DEV), _x_tensor(x)).cpu().numpy()
    ref = oracle.expert_ffn(blob, qtype, z, H, FF, x)
    assert max_err_over_rms(y, ref) <= TOL


def test_expert_ffn_page_mapping_z1():
    """The Strata page's own code mapping (z = 1) and a one-hot closed form."""
    rng = np.random.default_rng(2)
    H, FF = 128, 64
    blob, _, _ = random_expert(rng, 1, H, FF, 0.05)
    x = rng.normal(size=(2, H)).astype(np.float32)
    d = moe.expert_desc(H, FF, 1, 1.0)
    y = moe.expert_ffn(d, torch.from_numpy(blob).to(DEV), torch.from_numpy(x).to(DEV)).cpu().numpy()
    assert max_err_over_rms(y, oracle.expert_ffn(blob, 1, 1.0, H, FF, x)) <= TOL


# --- layers ------------------------------------------------------------------------------------

def _layer_parity(w, layers, steps, tokens=None, arena=None):
    arena = arena or wl.DeviceArena(w, device=DEV, layers=layers)
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k, shared_ff=w.shared_ff)
    T = w.tokens if tokens is None else tokens
    for l in layers:
        host_blobs = None
        for step in steps:
            x, logits = wl.device_inputs(w, l, step, device=DEV, tokens=T)
            ids = torch.empty((T, w.top_k), dtype=torch.int32, device=DEV)
            wt = torch.empty((T, w.top_k), dtype=torch.float32, device=DEV)
            y = moe.layer_forward(desc, arena.tables[l], x, logits, shared=arena.shared_blob(l), ids=ids,
                                  weights=wt)
            hx, hl = wl.host_inputs(w, l, step, tokens=T)
            ids_ref, w_ref = oracle.route_topk(hl, w.top_k)
            np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
            assert np.max(np.abs(wt.cpu().numpy() - w_ref)) <= 1e-6
            needed = sorted(set(ids_ref.reshape(-1).tolist()))
            if host_blobs is None:
                host_blobs = {}
            for e in needed:
                if e not in host_blobs:
                    host_blobs[e] = synth.expert_blob(w.seed, l, e, w.qk, w.hidden, w.ff, w.sigma)
            # experts never selected are never read: an all-zero stand-in keeps the oracle's table complete
            zero = np.zeros(w.blob_bytes, dtype=np.uint8)
            table = [host_blobs.get(e, zero) for e in range(w.experts)]
            y_ref, ids2, _ = oracle.layer_forward(table, w.top_k, w.qtype, w.zero_point, w.hidden, w.ff, hx, hl,
                                                  shared=wl.host_shared_blob(w, l), shared_ff=w.shared_ff)
            np.testing.assert_array_equal(ids2, ids_ref)
            err = max_err_over_rms(y.cpu().numpy(), y_ref)
            assert err <= TOL, f"{w.name} layer {l} step {step}: max|err|/rms {err:.3e}"
    return arena


def test_layer_tiny():
    _layer_parity(wl.WORKLOADS["tiny"], [0], [0, 1, 2])


def test_layer_strata_decode_two_layers():
    _layer_parity(wl.WORKLOADS["strata_decode"], [0, 47], [0, 1])


def test_layer_gemma_decode_two_layers():
    _layer_parity(wl.WORKLOADS["gemma_decode"], [0, 29], [0, 1])


@pytest.mark.parametrize("name", ["verify_t4", "verify_t8"])
def test_layer_verify_windows(name):
    _layer_parity(wl.WORKLOADS[name], [3], [0, 1])


@pytest.mark.parametrize("T", [2, 3, 5, 6, 7])
def test_layer_ragged_windows(T):
    _layer_parity(wl.WORKLOADS["verify_t8"], [1], [4], tokens=T)


def test_window_most_pairs_and_shared_groups():
    """The window kernel at its largest pair count (8 tokens x 32 slots = 256
    pairs over 48 experts, so most experts are split into several groups of
    two) and with a shared expert over an odd window (its last group holds
    one token), against the oracle."""
    rng = np.random.default_rng(21)
    H, FF, FFs, E = 128, 64, 96, 48
    blobs = [random_expert(rng, 2, H, FF, 0.02)[0] for _ in range(E)]
    shared = random_expert(rng, 2, H, FFs, 0.02)[0]
    dev = [torch.from_numpy(b).to(DEV) for b in blobs]
    table = torch.tensor([t.data_ptr() for t in dev], dtype=torch.int64, device=DEV)
    sh = torch.from_numpy(shared).to(DEV)
    for T, k, use_shared in [(8, 32, False), (5, 6, True), (7, 32, True)]:
        x = rng.normal(size=(T, H)).astype(np.float32)
        logits = rng.normal(size=(T, E)).astype(np.float32)
        desc = moe.layer_desc(H, FF, 2, 7.5, E, k, shared_ff=FFs if use_shared else 0)
        y = moe.layer_forward(desc, table, torch.from_numpy(x).to(DEV), torch.from_numpy(logits).to(DEV),
                              shared=sh if use_shared else None)
        y_ref, _, _ = oracle.layer_forward(blobs, k, 2, 7.5, H, FF, x, logits,
                                           shared=shared if use_shared else None, shared_ff=FFs if use_shared else 0)
        assert max_err_over_rms(y.cpu().numpy(), y_ref) <= TOL, (T, k, use_shared)


def test_window_more_chunks_than_workgroups():
    """A wide layer (H = 4608, FF = 8192, 4-bit) whose down rows fall into
    more chunks (576 of 8 rows) than the window kernel has workgroups, so
    that workgroups combine several chunks one after another, against the
    oracle."""
    rng = np.random.default_rng(33)
    H, FF, E = 4608, 8192, 2
    blobs = [random_expert(rng, 2, H, FF, 0.02)[0] for _ in range(E)]
    dev = [torch.from_numpy(b).to(DEV) for b in blobs]
    table = torch.tensor([t.data_ptr() for t in dev], dtype=torch.int64, device=DEV)
    for T, k in [(2, 1), (3, 2)]:
        x = rng.normal(size=(T, H)).astype(np.float32)
        logits = rng.normal(size=(T, E)).astype(np.float32)
        desc = moe.layer_desc(H, FF, 2, 7.5, E, k)
        y = moe.layer_forward(desc, table, torch.from_numpy(x).to(DEV), torch.from_numpy(logits).to(DEV))
        y_ref, _, _ = oracle.layer_forward(blobs, k, 2, 7.5, H, FF, x, logits)
        assert max_err_over_rms(y.cpu().numpy(), y_ref) <= TOL, (T, k)


# --- invariants of the GEMV path ----------------------------------------------------------------

def test_batch_invariance_and_determinism():
    """Token t's output is bitwise the same alone (T=1) and inside a window of 8,
    and identical from run to run."""
    w = wl.WORKLOADS["verify_t8"]
    arena = wl.DeviceArena(w, device=DEV, layers=[2])
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k)
    x, logits = wl.device_inputs(w, 2, 0, device=DEV)
    y8 = moe.layer_forward(desc, arena.tables[2], x, logits)
    y8b = moe.layer_forward(desc, arena.tables[2], x, logits)
    assert torch.equal(y8, y8b)
    for t in range(8):
        y1 = moe.layer_forward(desc, arena.tables[2], x[t:t + 1].contiguous(), logits[t:t + 1].contiguous())
        assert torch.equal(y1[0], y8[t]), f"token {t} differs between T=1 and T=8"
    for T in (2, 3, 4, 5):
        yT = moe.layer_forward(desc, arena.tables[2], x[:T].contiguous(), logits[:T].contiguous())
        assert torch.equal(yT, y8[:T])


@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_batch_invariance_gemma_shape(x_dtype):
    """The 4-bit shape with a shared expert, whose one-token gate/up lanes take
    two adjacent block columns each (88 columns a row): token t's output is
    still bitwise the same alone and inside a window of 8, and of 3."""
    w = wl.WORKLOADS["gemma_decode"]
    arena = wl.DeviceArena(w, device=DEV, layers=[1])
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k, shared_ff=w.shared_ff)
    x, logits = wl.device_inputs(w, 1, 0, device=DEV, tokens=8)
    if x_dtype == "f32":
        x = x.float()
    sh = arena.shared_blob(1)
    y8 = moe.layer_forward(desc, arena.tables[1], x, logits, shared=sh)
    for t in range(8):
        y1 = moe.layer_forward(desc, arena.tables[1], x[t:t + 1].contiguous(), logits[t:t + 1].contiguous(), shared=sh)
        assert torch.equal(y1[0], y8[t]), f"token {t} differs between T=1 and T=8"
    y3 = moe.layer_forward(desc, arena.tables[1], x[:3].contiguous(), logits[:3].contiguous(), shared=sh)
    assert torch.equal(y3, y8[:3])


def test_identical_experts_ignore_routing():
    w = wl.WORKLOADS["strata_decode"]
    blob = torch.from_numpy(synth.expert_blob(0, 0, 0, w.qk, w.hidden, w.ff, w.sigma)).to(DEV)
    table = torch.full((w.experts,), blob.data_ptr(), dtype=torch.int64, device=DEV)
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k)
    ed = moe.expert_desc(w.hidden, w.ff, w.qtype, w.zero_point)
    x, logits = wl.device_inputs(w, 0, 0, device=DEV, tokens=4)
    y_one = moe.expert_ffn(ed, blob, x).cpu().numpy()
    for s in range(3):
        lg = torch.randn((4, w.experts), device=DEV, generator=torch.Generator(device=DEV).manual_seed(s))
        y = moe.layer_forward(desc, table, x, lg).cpu().numpy()
        assert max_err_over_rms(y, y_one) <= 1e-5


def test_permutation_equivariance():
    w = wl.WORKLOADS["strata_decode"]
    arena = wl.DeviceArena(w, device=DEV, layers=[1])
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k)
    x, logits = wl.device_inputs(w, 1, 0, device=DEV)
    ids = torch.empty((1, w.top_k), dtype=torch.int32, device=DEV)
    y = moe.layer_forward(desc, arena.tables[1], x, logits, ids=ids)
    perm = torch.randperm(w.experts, generator=torch.Generator().manual_seed(0)).to(DEV)
    ids2 = torch.empty_like(ids)
    y2 = moe.layer_forward(desc, arena.tables[1][perm].contiguous(), x, logits[:, perm].contiguous(), ids=ids2)
    assert torch.equal(perm[ids2.long()].int(), ids)
    assert torch.equal(y, y2)


def test_doubling_down_scales_doubles_output():
    w = wl.WORKLOADS["gemma_decode"]
    H, FF = w.hidden, w.ff
    blob = synth.expert_blob(0, 0, 3, w.qk, H, FF, w.sigma)
    off = 2 * FF * (H // 32) * 18 + H * (FF // 32) * 16
    b2 = blob.copy()
    sc = b2[off: off + 2 * H * (FF // 32)].view('<u2')
    e = (sc >> 10) & 31
    sc[:] = np.where(e == 0, (sc & 0x8000) | ((sc & 0x3FF) << 1), sc + 0x400)
    d = moe.expert_desc(H, FF, w.qtype, w.zero_point)
    x, _ = wl.device_inputs(w, 0, 0, device=DEV, tokens=3)
    y1 = moe.expert_ffn(d, torch.from_numpy(blob).to(DEV), x)
    y2 = moe.expert_ffn(d, torch.from_numpy(b2).to(DEV), x)
    assert torch.equal(y2, 2 * y1)


def test_k_equals_e_and_single_expert():
    rng = np.random.default_rng(8)
    H, FF, E = 128, 64, 4
    blobs = [random_expert(rng, 2, H, FF, 0.02)[0] for _ in range(E)]
    dev = [torch.from_numpy(b).to(DEV) for b in blobs]
    table = torch.tensor([t.data_ptr() for t in dev], dtype=torch.int64, device=DEV)
    x = rng.normal(size=(3, H)).astype(np.float32)
    for k in (1, E):
        logits = rng.normal(size=(3, E)).astype(np.float32)
        desc = moe.layer_desc(H, FF, 2, 7.5, E, k)
        y = moe.layer_forward(desc, table, torch.from_numpy(x).to(DEV), torch.from_numpy(logits).to(DEV))
        y_ref, _, _ = oracle.layer_forward(blobs, k, 2, 7.5, H, FF, x, logits)
        assert max_err_over_rms(y.cpu().numpy(), y_ref) <= TOL
    desc = moe.layer_desc(H, FF, 2, 7.5, 1, 1)
    y = moe.layer_forward(desc, table[:1].contiguous(), torch.from_numpy(x).to(DEV),
                          torch.zeros((3, 1), device=DEV))
    assert max_err_over_rms(y.cpu().numpy(), oracle.expert_ffn(blobs[0], 2, 7.5, H, FF, x)) <= TOL


def _decode_fixed_bytes(k, hidden, ff, shared_ff, qk, small_t=8):
    """Bytes at the start of a layer workspace that the decode kernels keep
    between calls, each region 256-byte aligned: the sync words (the larger of
    the one-token kernel's 64-byte lines plus 16 replicas of its ready flags,
    and the window kernel's lines: 2, then 2 per group of small_t * k + 4,
    then 2 per chunk of 8 passes of down rows), then the `a` words of
    small_t * k pairs and of small_t shared-expert rows, then the window
    kernel's d words for small_t * k + small_t rows of hidden."""
    al = lambda v: (v + 255) // 256 * 256
    lines = 64 * (4 + small_t * k + small_t + 16)
    sync1 = (lines + 4095) // 4096 * 4096 + 16 * 4096
    chunk_rows = (256 // (ff // qk)) * 8
    n_chunks = (hidden + chunk_rows - 1) // chunk_rows
    syncw = 64 * (2 + 2 * (small_t * k + 4) + 2 * n_chunks)
    off = al(max(sync1, syncw))
    off = al(off + small_t * k * ff * 4)
    off = al(off + small_t * shared_ff * 4)
    return al(off + (small_t * k + small_t) * hidden * 4)


def test_workspace_shared_state_returns_to_zero():
    """One workspace serves decode calls of several sizes and a prefill call in
    between: every result equals the one on a fresh workspace, and the decode
    kernel's sync and `a` words are zero after every call (which also shows
    that no bounded wait ran out: that would have left the error word set)."""
    w = wl.WORKLOADS["gemma_decode"]
    arena = wl.DeviceArena(w, device=DEV, layers=[0])
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k, shared_ff=w.shared_ff)
    sizes = (1, 3, 8, 20, 1, 8, 2)
    ws = moe.workspace(max(moe.layer_workspace_bytes(desc, T) for T in sizes), DEV)
    fixed = _decode_fixed_bytes(w.top_k, w.hidden, w.ff, w.shared_ff, 64 if w.qtype == 1 else 32)
    assert fixed <= moe.layer_workspace_bytes(desc, 1)
    for i, T in enumerate(sizes):
        x, logits = wl.device_inputs(w, 0, 50 + i, device=DEV, tokens=T)
        y = moe.layer_forward(desc, arena.tables[0], x, logits, shared=arena.shared_blob(0), ws=ws)
        y_fresh = moe.layer_forward(desc, arena.tables[0], x, logits, shared=arena.shared_blob(0))
        torch.cuda.synchronize()
        assert torch.equal(y, y_fresh), f"call {i} (T={T}) differs from a fresh workspace"
        assert int((ws[:fixed] != 0).sum().item()) == 0, f"shared words not zero after call {i} (T={T})"


def test_graph_replays_match_eager():
    """Calls captured in a HIP graph give, on every replay, the eager result."""
    w = wl.WORKLOADS["strata_decode"]
    arena = wl.DeviceArena(w, device=DEV, layers=[0, 1, 2])
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k)
    ws = moe.workspace(moe.layer_workspace_bytes(desc, 1), DEV)
    inputs = [wl.device_inputs(w, l, 9, device=DEV) for l in range(3)]
    ys = [torch.empty((1, w.hidden), device=DEV) for _ in range(3)]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for l in range(3):
            moe.layer_forward(desc, arena.tables[l], *inputs[l], y=ys[l], ws=ws, stream=stream)
    stream.synchronize()
    eager = [y.clone() for y in ys]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for l in range(3):
                moe.layer_forward(desc, arena.tables[l], *inputs[l], y=ys[l], ws=ws, stream=stream)
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        stream.synchronize()
        for l in range(3):
            assert torch.equal(ys[l], eager[l]), f"replay {rep} layer {l}"
        # eager work between replays
        moe.layer_forward(desc, arena.tables[0], *inputs[1], ws=moe.workspace(moe.layer_workspace_bytes(desc, 1), DEV))
        torch.cuda.synchronize()
    assert int((ws[:_decode_fixed_bytes(w.top_k, w.hidden, w.ff, 0, 64 if w.qtype == 1 else 32)] != 0).sum().item()) == 0
