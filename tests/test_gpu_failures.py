"""Failures inside a layer call reach the caller: with every bounded wait
forced to give up (debug wait limit 0; every kernel still exits normally),
the outputs the waits served are NaN, the error word is reported by
moe_workspace_check, which resets the workspace, later calls on an unchecked
workspace write NaN, and a checked workspace gives the same results as a
fresh one."""
import numpy as np
import pytest
import torch

import bit_expert_ffn_amd as moe
from synth import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture
def wait_limit_restored():
    yield
    moe.debug_set_wait_limit(-1)


@pytest.mark.parametrize("T", [1, 4])
def test_forced_timeouts_are_reported_and_cleared(T, wait_limit_restored):
    w = wl.WORKLOADS["verify_t8"]
    arena = wl.DeviceArena(w, device=DEV, layers=[5])
    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k)
    x, logits = wl.device_inputs(w, 5, 3, device=DEV, tokens=T)
    y_ok = moe.layer_forward(desc, arena.tables[5], x, logits)
    torch.cuda.synchronize()
    assert torch.isfinite(y_ok).all()

    ws = moe.workspace(moe.layer_workspace_bytes(desc, T), DEV)
    moe.workspace_check(desc, ws)                       # a fresh workspace is clean
    print(f"forced timeouts, T={T}", flush=True)
    moe.debug_set_wait_limit(0)
    y = moe.layer_forward(desc, arena.tables[5], x, logits, ws=ws)
    torch.cuda.synchronize()
    moe.debug_set_wait_limit(-1)
    assert torch.isnan(y).all(), "every output row was served by a wait that gave up"
    # an unchecked failure: the next call writes NaN and does nothing else
    y2 = moe.layer_forward(desc, arena.tables[5], x, logits, ws=ws)
    torch.cuda.synchronize()
    assert torch.isnan(y2).all()
    # ... also on the matrix-core path sharing the workspace
    wsb = moe.workspace(max(ws.numel(), moe.layer_workspace_bytes(desc, 12)), DEV)
    wsb[:ws.numel()].copy_(ws)
    x12, l12 = wl.device_inputs(w, 5, 4, device=DEV, tokens=12)
    y12 = moe.layer_forward(desc, arena.tables[5], x12, l12, ws=wsb)
    torch.cuda.synchronize()
    assert torch.isnan(y12).all()
    with pytest.raises(moe.MoeError) as ei:
        moe.workspace_check(desc, ws)
    assert ei.value.status == 4 and "wait gave up" in str(ei.value)
    moe.workspace_check(desc, ws)                       # reset: clean now
    y3 = moe.layer_forward(desc, arena.tables[5], x, logits, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y3, y_ok)
    moe.workspace_check(desc, ws)


def test_decode_then_window_with_16_slots_leave_workspace_zero():
    """k = 16 without a shared expert (the prefetch-hint words then share 64-byte
    lines with the window kernel's group counters): a one-token call, then a
    window call, then a one-token call on one workspace; each equals a fresh
    workspace's result and the shared region is zero after each."""
    rng = np.random.default_rng(4)
    E, k, H, FF = 64, 16, 256, 128
    from helpers import random_expert
    blobs = [random_expert(rng, 1, H, FF, 0.05)[0] for _ in range(E)]
    dev = [torch.from_numpy(b).to(DEV) for b in blobs]
    table = torch.tensor([t.data_ptr() for t in dev], dtype=torch.int64, device=DEV)
    desc = moe.layer_desc(H, FF, 1, 1.5, E, k)
    ws = moe.workspace(moe.layer_workspace_bytes(desc, 8), DEV)
    fixed = moe.layer_workspace_bytes(desc, 0)   # T = 0: exactly the shared region (no id/weight scratch)
    for i, T in enumerate((1, 4, 1, 8, 1)):
        x = torch.from_numpy(rng.normal(size=(T, H)).astype(np.float32)).to(DEV)
        lg = torch.from_numpy(rng.normal(size=(T, E)).astype(np.float32)).to(DEV)
        y = moe.layer_forward(desc, table, x, lg, ws=ws)
        y_fresh = moe.layer_forward(desc, table, x, lg)
        torch.cuda.synchronize()
        assert torch.equal(y, y_fresh), f"call {i} (T={T})"
        assert int((ws[:fixed] != 0).sum().item()) == 0, f"shared words not zero after call {i} (T={T})"
    moe.workspace_check(desc, ws)
