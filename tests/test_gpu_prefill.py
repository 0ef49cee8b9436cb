"""GPU parity of the prefill (matrix-core) path, T > 8 tokens, against the
float64 oracle: full outputs at small sizes (several tiles, ragged per-expert
counts, shared expert, fp32 and bf16 activations, both block formats), and
sampled tokens of the full 4,096-token, 256-expert layer."""
import numpy as np
import pytest
import torch

import bit_expert_ffn_amd as moe
import oracle
import synth
from helpers import max_err_over_rms
from synth import workloads as wl

pytestmark = pytest.mark.gpu
TOL = 2e-3
DEV = "cuda"


def _x_tensor(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(x).to(DEV)


@pytest.mark.parametrize("qtype,H,FF,T,xd", [(2, 256, 128, 9, "bf16"), (2, 256, 192, 130, "bf16"), (1, 256, 128, 40, "bf16"),
                                             (2, 160, 96, 77, "f32"), (1, 192, 320, 300, "f32"),
                                             (2, 2816, 704, 64, "bf16"),
                                             # rows of a multiple of 8 blocks (scales in 16-byte loads), every
                                             # format and activation plane count, gate/up and down
                                             (1, 1024, 512, 70, "bf16"), (1, 512, 512, 33, "f32"),
                                             (2, 512, 256, 50, "f32")])
def test_expert_ffn_prefill_matches_oracle(qtype, H, FF, T, xd):
    qk = 64 if qtype == 1 else 32
    z = 1.5 if qtype == 1 else 7.5
    blob = synth.expert_blob(3, 2, T, qk, H, FF, 0.05 if qtype == 1 else 0.02)
    x = synth.activations(3, 2, T, T, H, xd)
    d = moe.expert_desc(H, FF, qtype, z)
    y = moe.expert_ffn(d, torch.from_numpy(blob).to(DEV), _x_tensor(x)).cpu().numpy()
    ref = oracle.expert_ffn(blob, qtype, z, H, FF, x)
    assert max_err_over_rms(y, ref) <= TOL


def _scales(blob, qk, H, FF, m):
    """Writable fp16 view [rows][nblk] of the scales plane of matrix m (0 gate,
    1 up, 2 down) of an expert blob: each matrix is a codes plane [rows][nblk]
    of 16 bytes followed by its scales."""
    rows, cols = (FF, FF, H), (H, H, FF)
    off = sum(rows[i] * (cols[i] // qk) * 18 for i in range(m))
    nblk = cols[m] // qk
    start = off + rows[m] * nblk * 16
    return blob[start:start + rows[m] * nblk * 2].view(np.float16).reshape(rows[m], nblk)


@pytest.mark.parametrize("qtype,z", [(2, 15.5), (2, 16.0), (2, -0.5), (2, -1.0), (1, 14.0), (1, -14.0)])
def test_prefill_zero_point_range(qtype, z):
    """bf16 activations with zero points away from the formats' centres (z a
    multiple of 0.5 in [-64, 64]): the matrix-core weight operands 2(c - z) stay
    exact fp16 integers at either end of the code range."""
    qk = 64 if qtype == 1 else 32
    H, FF, T = 512, 192, 70
    blob = synth.expert_blob(11, 0, 1, qk, H, FF, 0.05 if qtype == 1 else 0.02)
    x = synth.activations(11, 0, 1, T, H, "bf16")
    d = moe.expert_desc(H, FF, qtype, z)
    y = moe.expert_ffn(d, torch.from_numpy(blob).to(DEV), _x_tensor(x)).cpu().numpy()
    ref = oracle.expert_ffn(blob, qtype, z, H, FF, x)
    assert max_err_over_rms(y, ref) <= TOL


@pytest.mark.parametrize("qtype", [2, 1])
def test_prefill_large_block_scales(qtype):
    """Gate and up block scales times 2^17 (exact in fp16, up to 26,432): large
    and small scales mixed along each row, with outputs far from unit size, keep
    the oracle's relative accuracy through the per-block fp32 scaling."""
    qk = 64 if qtype == 1 else 32
    z = 1.5 if qtype == 1 else 7.5
    H, FF, T = 512, 192, 40
    blob = synth.expert_blob(12, 0, 2, qk, H, FF, 0.05 if qtype == 1 else 0.02)
    for m in (0, 1):
        sc = _scales(blob, qk, H, FF, m)
        big = sc.astype(np.float64) * 2.0 ** 17
        assert np.all(np.abs(big) <= 65504.0)
        sc[...] = big.astype(np.float16)
        frac = np.mean(np.abs(sc.astype(np.float64)) >= 1024.0)
        assert 0.3 < frac < 1.0, frac   # large and small scales mixed
    x = synth.activations(12, 0, 2, T, H, "bf16")
    d = moe.expert_desc(H, FF, qtype, z)
    y = moe.expert_ffn(d, torch.from_numpy(blob).to(DEV), _x_tensor(x)).cpu().numpy()
    ref = oracle.expert_ffn(blob, qtype, z, H, FF, x)
    assert np.all(np.isfinite(y))
    assert max_err_over_rms(y, ref) <= TOL


def _small_layer(qtype, E, k, H, FF, T, xd, shared_ff, zipf, seed):
    qk = 64 if qtype == 1 else 32
    z = 1.5 if qtype == 1 else 7.5
    sigma = 0.05 if qtype == 1 else 0.02
    blobs = synth.expert_blobs(seed, 0, 0, E, qk, H, FF, sigma)
    shared = synth.expert_blob(seed, 0, synth.SHARED_EXPERT, qk, H, shared_ff, sigma) if shared_ff else None
    x = synth.activations(seed, 0, 0, T, H, xd)
    logits = synth.logits(seed, 0, 0, T, E, zipf)
    dev = torch.from_numpy(blobs).to(DEV)
    table = torch.tensor([dev.data_ptr() + e * blobs.shape[1] for e in range(E)], dtype=torch.int64, device=DEV)
    desc = moe.layer_desc(H, FF, qtype, z, E, k, shared_ff=shared_ff)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    sh = torch.from_numpy(shared).to(DEV) if shared is not None else None
    y = moe.layer_forward(desc, table, _x_tensor(x), torch.from_numpy(logits).to(DEV), shared=sh, ids=ids, weights=w)
    y_ref, ids_ref, w_ref = oracle.layer_forward(list(blobs), k, qtype, z, H, FF, x, logits, shared=shared,
                                                 shared_ff=shared_ff)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    assert np.max(np.abs(w.cpu().numpy() - w_ref)) <= 1e-6
    return y.cpu().numpy(), y_ref


@pytest.mark.parametrize("qtype,E,k,H,FF,T,xd,shared_ff,zipf", [
    (2, 16, 4, 256, 128, 100, "bf16", 0, 0.6),
    (2, 16, 4, 256, 128, 257, "bf16", 192, 0.0),
    (1, 8, 2, 256, 128, 64, "f32", 0, 0.0),
    (2, 64, 8, 512, 256, 300, "bf16", 0, 1.2),
    # 37 experts (6-bit ids, not a power of two), 2,350 pairs: three placement
    # blocks, the last ragged, with skewed routing
    (1, 37, 5, 256, 128, 470, "bf16", 0, 1.0),
])
def test_layer_prefill_matches_oracle(qtype, E, k, H, FF, T, xd, shared_ff, zipf):
    y, y_ref = _small_layer(qtype, E, k, H, FF, T, xd, shared_ff, zipf, seed=T)
    assert max_err_over_rms(y, y_ref) <= TOL


def test_prefill_is_deterministic():
    a, _ = _small_layer(2, 16, 4, 256, 128, 200, "bf16", 128, 0.6, seed=5)
    b, _ = _small_layer(2, 16, 4, 256, 128, 200, "bf16", 128, 0.6, seed=5)
    np.testing.assert_array_equal(a, b)


def test_prefill_full_layer_sampled_tokens():
    """The full prefill shape (4,096 tokens, 256 experts, top-8, H 7168, FF 2048,
    4-bit): routing of every token exactly, outputs of sampled tokens (covering
    the hottest and the coldest experts) against the oracle."""
    w = wl.WORKLOADS["prefill"]
    arena = wl.DeviceArena(w, device=DEV, layers=[0])
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k)
    x, logits = wl.device_inputs(w, 0, 0, device=DEV)
    ids = torch.empty((w.tokens, w.top_k), dtype=torch.int32, device=DEV)
    wt = torch.empty((w.tokens, w.top_k), dtype=torch.float32, device=DEV)
    y = moe.layer_forward(desc, arena.tables[0], x, logits, ids=ids, weights=wt)
    torch.cuda.synchronize()
    hx, hl = wl.host_inputs(w, 0, 0)
    ids_ref, w_ref = oracle.route_topk(hl, w.top_k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    assert np.max(np.abs(wt.cpu().numpy() - w_ref)) <= 1e-6
    counts = np.bincount(ids_ref.reshape(-1), minlength=w.experts)
    hot, cold = int(np.argmax(counts)), int(np.argmin(counts))
    # 64 tokens: ones routed to the hottest and the coldest expert, the last
    # token, and a deterministic spread over the prompt.
    must = [int(np.nonzero((ids_ref == hot).any(1))[0][0]), int(np.nonzero((ids_ref == cold).any(1))[0][0]),
            w.tokens - 1]
    spread = [t for t in range(0, w.tokens, w.tokens // 61) if t not in must]
    sample = sorted(must + spread[:64 - len(must)])
    assert len(sample) == 64
    need = sorted(set(ids_ref[sample].reshape(-1).tolist()))
    blobs = {e: synth.expert_blob(w.seed, 0, e, w.qk, w.hidden, w.ff, w.sigma) for e in need}
    zero = np.zeros(w.blob_bytes, dtype=np.uint8)
    y_ref, _, _ = oracle.layer_forward([blobs.get(e, zero) for e in range(w.experts)], w.top_k, w.qtype,
                                       w.zero_point, w.hidden, w.ff, hx[sample], hl[sample])
    assert max_err_over_rms(y.cpu().numpy()[sample], y_ref) <= TOL


@pytest.mark.parametrize("T,expect", [(3, 1), (150, 6)])
def test_timed_entry_point_matches_and_records(T, expect):
    """moe_layer_forward_timed does the same work as moe_layer_forward (bitwise
    equal outputs) and records one event per kernel boundary, in order."""
    E, k, H, FF = 16, 4, 256, 128
    blobs = synth.expert_blobs(9, 0, 0, E, 32, H, FF, 0.02)
    x = synth.activations(9, 0, 0, T, H, "bf16")
    logits = synth.logits(9, 0, 0, T, E, 0.6)
    dev = torch.from_numpy(blobs).to(DEV)
    table = torch.tensor([dev.data_ptr() + e * blobs.shape[1] for e in range(E)], dtype=torch.int64, device=DEV)
    desc = moe.layer_desc(H, FF, 2, 7.5, E, k)
    xt, lt = _x_tensor(x), torch.from_numpy(logits).to(DEV)
    ws = moe.workspace(moe.layer_workspace_bytes(desc, T), DEV)
    y0 = moe.layer_forward(desc, table, xt, lt, ws=ws)
    s = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    for e in evs:
        e.record(s)
    y1, n = moe.layer_forward_timed(desc, table, xt, lt, evs, ws=ws)
    torch.cuda.synchronize()
    assert n == expect
    np.testing.assert_array_equal(y0.cpu().numpy(), y1.cpu().numpy())
    times = [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]
    assert all(t >= 0.0 for t in times) and evs[0].elapsed_time(evs[n]) > 0.0
