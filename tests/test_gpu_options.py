"""GPU parity of the layer options against the float64 oracle:
GeGLU (tanh GELU) and the per-expert down scale (kairos-engine README, "The
MoE forward" and "Decode, 2026-09-28/29"), caller-supplied routing with
zero-weight slots skipped (Krasis white paper 7.5), and the router front end
(kairos-engine README, "The MoE forward") -- on the decode (T = 1), verify
window (T = 2..8) and matrix-core (T > 8) paths."""
import numpy as np
import pytest
import torch

import bit_expert_ffn_amd as moe
import oracle
import synth
from helpers import bf16_bits_array, max_err_over_rms, router_error_bound
from synth import workloads as wl

pytestmark = pytest.mark.gpu
TOL = 2e-3
DEV = "cuda"


def _x_tensor(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _layer(qtype, E, H, FF, shared_ff, seed):
    qk = 64 if qtype == 1 else 32
    sigma = 0.05 if qtype == 1 else 0.02
    blobs = synth.expert_blobs(seed, 0, 0, E, qk, H, FF, sigma)
    shared = synth.expert_blob(seed, 0, synth.SHARED_EXPERT, qk, H, shared_ff, sigma) if shared_ff else None
    dev = torch.from_numpy(blobs).to(DEV)
    table = torch.tensor([dev.data_ptr() + e * blobs.shape[1] for e in range(E)], dtype=torch.int64, device=DEV)
    sh = torch.from_numpy(shared).to(DEV) if shared is not None else None
    return blobs, shared, dev, table, sh


# --- GeGLU and the per-expert down scale ----------------------------------------------------------

@pytest.mark.parametrize("qtype,H,FF,T", [(2, 2816, 704, 1), (2, 2816, 704, 4), (1, 256, 128, 40), (2, 256, 192, 8)])
def test_expert_ffn_geglu_matches_oracle(qtype, H, FF, T):
    qk = 64 if qtype == 1 else 32
    z = 1.5 if qtype == 1 else 7.5
    blob = synth.expert_blob(11, 1, T, qk, H, FF, 0.05 if qtype == 1 else 0.02)
    x = synth.activations(11, 1, T, T, H, "bf16")
    d = moe.expert_desc(H, FF, qtype, z, act=moe.ACT_GEGLU_TANH)
    y = moe.expert_ffn(d, torch.from_numpy(blob).to(DEV), _x_tensor(x)).cpu().numpy()
    assert max_err_over_rms(y, oracle.expert_ffn(blob, qtype, z, H, FF, x, act=1)) <= TOL


@pytest.mark.parametrize("T", [1, 4, 8, 48])
def test_gemma_faithful_layer_geglu_down_scale(T):
    """The Gemma shape (128 experts of H 2816, FF 704, top-8, shared FF 2112,
    4-bit) with GeGLU everywhere and a per-expert down scale."""
    w = wl.WORKLOADS["gemma_decode"]
    arena = wl.DeviceArena(w, device=DEV, layers=[2])
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k, shared_ff=w.shared_ff,
                          act=moe.ACT_GEGLU_TANH)
    rng = np.random.default_rng(T)
    ds = rng.uniform(0.25, 2.0, size=w.experts).astype(np.float32)
    x, logits = wl.device_inputs(w, 2, 30 + T, device=DEV, tokens=T)
    y = moe.layer_forward_ex(desc, arena.tables[2], x, logits, shared=arena.shared_blob(2),
                             down_scale=torch.from_numpy(ds).to(DEV)).cpu().numpy()
    hx, hl = wl.host_inputs(w, 2, 30 + T, tokens=T)
    ids, _ = oracle.route_topk(hl, w.top_k)
    zero = np.zeros(w.blob_bytes, dtype=np.uint8)
    need = set(ids.reshape(-1).tolist())
    blobs = [synth.expert_blob(w.seed, 2, e, w.qk, w.hidden, w.ff, w.sigma) if e in need else zero
             for e in range(w.experts)]
    y_ref, _, _ = oracle.layer_forward_ex(blobs, w.top_k, w.qtype, w.zero_point, w.hidden, w.ff, hx, hl,
                                          shared=wl.host_shared_blob(w, 2), shared_ff=w.shared_ff, act=1,
                                          down_scale=ds)
    assert max_err_over_rms(y, y_ref) <= TOL


def test_down_scale_keeps_batch_invariance():
    """With a down scale, a token's output is still bitwise the same alone and
    inside a window (the weight and the scale are multiplied first on both paths)."""
    w = wl.WORKLOADS["verify_t8"]
    arena = wl.DeviceArena(w, device=DEV, layers=[4])
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k, act=moe.ACT_GEGLU_TANH)
    ds = torch.from_numpy(np.random.default_rng(2).uniform(0.5, 1.5, w.experts).astype(np.float32)).to(DEV)
    x, logits = wl.device_inputs(w, 4, 1, device=DEV)
    y8 = moe.layer_forward_ex(desc, arena.tables[4], x, logits, down_scale=ds)
    for t in (0, 3, 7):
        y1 = moe.layer_forward_ex(desc, arena.tables[4], x[t:t + 1].contiguous(), logits[t:t + 1].contiguous(),
                                  down_scale=ds)
        assert torch.equal(y1[0], y8[t]), t


# --- caller-supplied routing: the fixed top-k shape --------------------------------------------

def _poisoned_routing(T, k, E, dummy, rng):
    """Routing of T tokens: k distinct experts each (never the dummy), weights
    renormalised, then about a third of the slots (never all of a token's but
    the last token's, which keeps none) set to the dummy expert with weight 0."""
    ids = np.stack([rng.choice([e for e in range(E) if e != dummy], size=k, replace=False) for _ in range(T)])
    w = rng.uniform(0.1, 1.0, size=(T, k))
    w /= w.sum(1, keepdims=True)
    drop = rng.random((T, k)) < 0.35
    drop[:, 0] = False
    if T > 1:
        drop[-1] = True
    ids = np.where(drop, dummy, ids).astype(np.int32)
    w = np.where(drop, 0.0, w).astype(np.float32)
    w[drop & (rng.random((T, k)) < 0.5)] = -0.0
    return ids, w


@pytest.mark.parametrize("T,shared_ff", [(1, 0), (1, 192), (5, 0), (8, 192), (40, 0), (130, 192)])
def test_routed_zero_weight_slots_skip_a_nan_dummy(T, shared_ff):
    """A dummy expert whose scales are all NaN sits behind every zero-weight
    slot: y stays finite and equals the oracle over the remaining slots."""
    E, k, H, FF = 24, 6, 256, 128
    blobs, shared, dev, table, sh = _layer(2, E, H, FF, shared_ff, seed=T)
    dummy = E - 1
    nb = FF * (H // 32)
    for m in range(3):   # every scale of the dummy's three matrices
        rows, cols = [(FF, H), (FF, H), (H, FF)][m]
        off = m * FF * (H // 32) * 18 + rows * (cols // 32) * 16
        blobs[dummy][off:off + 2 * rows * (cols // 32)] = np.frombuffer(
            np.full(rows * (cols // 32), 0x7E00, '<u2').tobytes(), np.uint8)
    dev[dummy].copy_(torch.from_numpy(blobs[dummy]))
    rng = np.random.default_rng(100 + T)
    ids, w = _poisoned_routing(T, k, E, dummy, rng)
    x = synth.activations(5, 0, T, T, H, "bf16")
    desc = moe.layer_desc(H, FF, 2, 7.5, E, k, shared_ff=shared_ff)
    ids_o = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w_o = torch.empty((T, k), dtype=torch.float32, device=DEV)
    y = moe.layer_forward_ex(desc, table, _x_tensor(x), shared=sh, ids_in=torch.from_numpy(ids).to(DEV),
                             w_in=torch.from_numpy(w).to(DEV), ids=ids_o, weights=w_o).cpu().numpy()
    assert np.all(np.isfinite(y))
    np.testing.assert_array_equal(ids_o.cpu().numpy(), ids)
    np.testing.assert_array_equal(w_o.cpu().numpy().view(np.uint32), w.view(np.uint32))
    y_ref, _, _ = oracle.layer_forward_ex(list(blobs), k, 2, 7.5, H, FF, x, shared=shared, shared_ff=shared_ff,
                                          ids_in=ids, w_in=w)
    if shared_ff == 0 and T > 1:
        assert np.all(y[-1] == 0.0)            # every slot skipped, no shared expert
    assert max_err_over_rms(y, y_ref) <= TOL


def test_routed_bad_id_is_reported():
    E, k, H, FF = 16, 4, 128, 64
    blobs, shared, dev, table, sh = _layer(2, E, H, FF, 0, seed=3)
    desc = moe.layer_desc(H, FF, 2, 7.5, E, k)
    for T in (1, 4, 20):
        ids = np.tile(np.arange(k, dtype=np.int32), (T, 1))
        w = np.full((T, k), 0.25, dtype=np.float32)
        ids[T // 2, 1] = E + 3                  # an id outside [0, E) with a nonzero weight
        ws = moe.workspace(moe.layer_workspace_bytes(desc, T), DEV)
        x = _x_tensor(synth.activations(3, 0, T, T, H, "bf16"))
        y = moe.layer_forward_ex(desc, table, x, ids_in=torch.from_numpy(ids).to(DEV),
                                 w_in=torch.from_numpy(w).to(DEV), ws=ws)
        torch.cuda.synchronize()
        assert torch.isnan(y).all(), T
        with pytest.raises(moe.MoeError) as ei:
            moe.workspace_check(desc, ws)
        assert "outside [0, E)" in str(ei.value)
        moe.workspace_check(desc, ws)


def test_routed_window_is_batch_invariant():
    w = wl.WORKLOADS["verify_t8"]
    arena = wl.DeviceArena(w, device=DEV, layers=[6])
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k)
    rng = np.random.default_rng(6)
    ids, wt = _poisoned_routing(8, w.top_k, w.experts, 0, rng)
    x, _ = wl.device_inputs(w, 6, 2, device=DEV)
    ii, wi = torch.from_numpy(ids).to(DEV), torch.from_numpy(wt).to(DEV)
    y8 = moe.layer_forward_ex(desc, arena.tables[6], x, ids_in=ii, w_in=wi)
    for t in range(8):
        y1 = moe.layer_forward_ex(desc, arena.tables[6], x[t:t + 1].contiguous(), ids_in=ii[t:t + 1].contiguous(),
                                  w_in=wi[t:t + 1].contiguous())
        assert torch.equal(y1[0], y8[t]), t


# --- the router front end ------------------------------------------------------------------------

def _router_inputs(E, H, T, seed, xd="bf16"):
    rng = np.random.default_rng(seed)
    wr = bf16_bits_array(rng.normal(0, 0.02, size=(E, H)))
    sc = rng.uniform(0.5, 1.5, size=H).astype(np.float32)
    x = synth.activations(seed, 9, 0, T, H, xd)
    return wr, sc, x


def _xprime(x, norm, sc, eps):
    xd = synth.bf16_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)
    if norm:
        xd = xd / np.sqrt(np.mean(xd * xd, axis=1, keepdims=True) + eps)
    return xd * sc.astype(np.float64) if sc is not None else xd


@pytest.mark.parametrize("T,xd", [(1, "bf16"), (3, "f32"), (8, "bf16"), (100, "bf16"), (65, "f32")])
@pytest.mark.parametrize("norm,scaled", [(False, False), (True, True)])
def test_router_logits_within_fp32_bound(T, xd, norm, scaled):
    E, H = 200, 2560
    wr, sc, x = _router_inputs(E, H, T, seed=T, xd=xd)
    sc = sc if scaled else None
    rt = moe.router(_x_tensor(wr.view(np.uint16)).view(torch.bfloat16),
                    torch.from_numpy(sc).to(DEV) if sc is not None else None, norm=norm, eps=1e-6)
    got = moe.router_logits(rt, E, _x_tensor(x)).cpu().numpy().astype(np.float64)
    ref = oracle.router_logits(wr, x, norm=norm, eps=1e-6, in_scale=sc)
    bound = router_error_bound(wr, _xprime(x, norm, sc, 1e-6))
    assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.parametrize("T,xd", [(8, "f32"), (5, "bf16"), (1, "f32")])
def test_router_logits_wide_rows_and_token_tiles(T, xd):
    """H = 7168: each lane's weight row takes two sets of chunks, and fp32 rows
    of 8 tokens exceed the LDS budget, so tokens are split over tiles."""
    E, H = 96, 7168
    wr, sc, x = _router_inputs(E, H, T, seed=300 + T, xd=xd)
    rt = moe.router(_x_tensor(wr.view(np.uint16)).view(torch.bfloat16), torch.from_numpy(sc).to(DEV), norm=True,
                    eps=1e-6)
    got = moe.router_logits(rt, E, _x_tensor(x)).cpu().numpy().astype(np.float64)
    ref = oracle.router_logits(wr, x, norm=True, eps=1e-6, in_scale=sc)
    assert np.all(np.abs(got - ref) <= router_error_bound(wr, _xprime(x, True, sc, 1e-6)))


def test_router_logits_batch_invariant():
    E, H = 512, 2560
    wr, sc, x = _router_inputs(E, H, 8, seed=77)
    rt = moe.router(_x_tensor(wr.view(np.uint16)).view(torch.bfloat16), torch.from_numpy(sc).to(DEV), norm=True)
    xt = _x_tensor(x)
    l8 = moe.router_logits(rt, E, xt)
    for t in range(8):
        assert torch.equal(moe.router_logits(rt, E, xt[t:t + 1].contiguous())[0], l8[t])


def _near_tie_free(ref, k, margin):
    """Tokens whose oracle top-k (and its order) cannot change under logit
    perturbations below `margin`: adjacent sorted logits through rank k differ
    by more than 2 margin."""
    s = -np.sort(-ref, axis=1)[:, :k + 1]
    return np.all(s[:, :-1] - s[:, 1:] > 2 * margin, axis=1)


@pytest.mark.parametrize("name,T,norm,act", [("strata_decode", 1, False, 0), ("verify_t8", 8, False, 0),
                                             ("gemma_decode", 1, True, 1), ("gemma_decode", 5, True, 1),
                                             ("gemma_decode", 24, True, 1)])
def test_layer_with_router_matches_oracle(name, T, norm, act):
    """The router inside the layer call: its logits within the fp32 bound of
    the oracle's; ids equal the oracle's (routing on its own float64 logits,
    rounded to fp32) wherever no near tie can reorder them, and where one can,
    the selection is a valid top-k of the oracle's logits within the bound;
    outputs within tolerance on the tokens with equal ids."""
    w = wl.WORKLOADS[name]
    layer = 1
    arena = wl.DeviceArena(w, device=DEV, layers=[layer])
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k, shared_ff=w.shared_ff, act=act)
    wr, sc, _ = _router_inputs(w.experts, w.hidden, 1, seed=T + 5)
    sc = sc if norm else None
    rt = moe.router(_x_tensor(wr.view(np.uint16)).view(torch.bfloat16),
                    torch.from_numpy(sc).to(DEV) if sc is not None else None, norm=norm, eps=1e-6)
    hx, _ = wl.host_inputs(w, layer, 60 + T, tokens=T)
    x = _x_tensor(hx)
    lg = torch.empty((T, w.experts), dtype=torch.float32, device=DEV)
    ids = torch.empty((T, w.top_k), dtype=torch.int32, device=DEV)
    y = moe.layer_forward_ex(desc, arena.tables[layer], x, shared=arena.shared_blob(layer), rt=rt, logits_out=lg,
                             ids=ids).cpu().numpy()
    ref = oracle.router_logits(wr, hx, norm=norm, eps=1e-6, in_scale=sc)
    bound = router_error_bound(wr, _xprime(hx, norm, sc, 1e-6))
    got = lg.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= bound)
    ids = ids.cpu().numpy()
    ids_ref, _ = oracle.route_topk(ref.astype(np.float32), w.top_k)
    # Each GPU logit lies within `err` of the oracle's float64 one, and the
    # oracle routes on those rounded to fp32: an order between two logits can
    # differ only where they are closer than twice that (a near tie).
    err = np.abs(got - ref).max(axis=1) + 2.0 ** -23 * np.abs(ref).max(axis=1)
    clean = np.array([_near_tie_free(ref[t:t + 1], w.top_k, err[t])[0] for t in range(T)])
    assert clean.mean() >= 0.5
    np.testing.assert_array_equal(ids[clean], ids_ref[clean])
    for t in np.nonzero(~clean)[0]:
        sel = ref[t, ids[t]]
        rest = np.delete(ref[t], ids[t])
        assert sel.min() >= rest.max() - 2 * err[t]
    need = set(ids_ref.reshape(-1).tolist())
    zero = np.zeros(w.blob_bytes, dtype=np.uint8)
    blobs = [synth.expert_blob(w.seed, layer, e, w.qk, w.hidden, w.ff, w.sigma) if e in need else zero
             for e in range(w.experts)]
    y_ref, _, _ = oracle.layer_forward_ex(blobs, w.top_k, w.qtype, w.zero_point, w.hidden, w.ff, hx,
                                          logits=ref.astype(np.float32), shared=wl.host_shared_blob(w, layer),
                                          shared_ff=w.shared_ff, act=act)
    assert max_err_over_rms(y[clean], y_ref[clean]) <= TOL
