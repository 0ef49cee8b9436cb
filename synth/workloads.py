"""The five measured workloads and device arenas built from the seeded generator.

Only input construction lives here (shapes, seeds, host->device upload); none of
the method's arithmetic.  Shapes follow the pages' models: the Strata 48 x 512
Q2_0 expert stack (H 2560, FF 640, top-10), a Gemma-style 30 x 128 4-bit stack
with an always-on shared expert (H 2816, FF 704, top-8, shared FF 2112), verify
windows of 4 and 8 tokens over the Strata shape, and a 4,096-token prefill over
256 experts of H 7168, FF 2048, top-8.
"""
from dataclasses import dataclass

import numpy as np

import synth


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    experts: int
    hidden: int
    ff: int
    top_k: int
    qtype: int          # 1 = 2-bit/64, 2 = 4-bit/32
    zero_point: float
    sigma: float        # scales are |N(0, sigma)| in fp16
    tokens: int
    x_dtype: str        # "bf16" or "f32"
    zipf_s: float       # 0 = N(0,1) logits
    shared_ff: int = 0
    seed: int = 0

    @property
    def qk(self):
        return 64 if self.qtype == 1 else 32

    @property
    def blob_bytes(self):
        return synth.blob_bytes(self.qk, self.hidden, self.ff)

    @property
    def shared_blob_bytes(self):
        return synth.blob_bytes(self.qk, self.hidden, self.shared_ff) if self.shared_ff else 0


WORKLOADS = {
    "tiny": Workload("tiny", 1, 8, 256, 128, 2, 1, 1.5, 0.05, 4, "f32", 0.0),
    "strata_decode": Workload("strata_decode", 48, 512, 2560, 640, 10, 1, 1.5, 0.05, 1, "bf16", 1.0),
    "gemma_decode": Workload("gemma_decode", 30, 128, 2816, 704, 8, 2, 7.5, 0.02, 1, "bf16", 0.8, shared_ff=2112),
    "verify_t4": Workload("verify_t4", 48, 512, 2560, 640, 10, 1, 1.5, 0.05, 4, "bf16", 1.0),
    "verify_t8": Workload("verify_t8", 48, 512, 2560, 640, 10, 1, 1.5, 0.05, 8, "bf16", 1.0),
    "prefill": Workload("prefill", 4, 256, 7168, 2048, 8, 2, 7.5, 0.02, 4096, "bf16", 0.6),
    # Measurement aids, not workloads of the pages: the Strata routing (512
    # experts, top-10, Zipf s = 1.0) and layer structure with experts so small
    # (H 256, FF 64) that their bytes and arithmetic are negligible, so a layer
    # call's time is the fixed cost of its dependent steps.
    "strata_floor": Workload("strata_floor", 48, 512, 256, 64, 10, 1, 1.5, 0.05, 1, "bf16", 1.0),
    "verify_t8_floor": Workload("verify_t8_floor", 48, 512, 256, 64, 10, 1, 1.5, 0.05, 8, "bf16", 1.0),
}


def host_layer_blobs(w: Workload, layer: int, experts=None):
    """[n, blob] uint8 numpy array of the given experts (default: all) of one layer."""
    if experts is None:
        return synth.expert_blobs(w.seed, layer, 0, w.experts, w.qk, w.hidden, w.ff, w.sigma)
    out = np.empty((len(experts), w.blob_bytes), dtype=np.uint8)
    for i, e in enumerate(experts):
        out[i] = synth.expert_blob(w.seed, layer, int(e), w.qk, w.hidden, w.ff, w.sigma)
    return out


def host_shared_blob(w: Workload, layer: int):
    if not w.shared_ff:
        return None
    return synth.expert_blob(w.seed, layer, synth.SHARED_EXPERT, w.qk, w.hidden, w.shared_ff, w.sigma)


def host_inputs(w: Workload, layer: int, step: int, tokens=None):
    """(x, logits) of one layer and step: x uint16 bf16 bits or float32, logits float32."""
    T = w.tokens if tokens is None else tokens
    x = synth.activations(w.seed, layer, step, T, w.hidden, w.x_dtype)
    logits = synth.logits(w.seed, layer, step, T, w.experts, w.zipf_s)
    return x, logits


class DeviceArena:
    """All experts of all layers resident in HBM: one [E, blob] uint8 tensor per
    layer, plus an int64 table of blob addresses per layer."""

    def __init__(self, w: Workload, device="cuda", layers=None, progress=None):
        import torch
        self.w = w
        self.layers = list(range(w.layers)) if layers is None else list(layers)
        self.blobs, self.tables, self.shared = {}, {}, {}
        pinned = torch.empty((w.experts, w.blob_bytes), dtype=torch.uint8, pin_memory=True)
        host = pinned.numpy()
        for l in self.layers:
            synth.expert_blobs(w.seed, l, 0, w.experts, w.qk, w.hidden, w.ff, w.sigma, out=host)
            dev = torch.empty((w.experts, w.blob_bytes), dtype=torch.uint8, device=device)
            dev.copy_(pinned)
            self.blobs[l] = dev
            base = dev.data_ptr()
            self.tables[l] = torch.tensor([base + e * w.blob_bytes for e in range(w.experts)], dtype=torch.int64,
                                          device=device)
            if w.shared_ff:
                self.shared[l] = torch.from_numpy(host_shared_blob(w, l)).to(device)
            if progress:
                progress(l)
        torch.cuda.synchronize()

    def shared_blob(self, layer):
        return self.shared.get(layer)


def device_inputs(w: Workload, layer: int, step: int, device="cuda", tokens=None):
    import torch
    x, logits = host_inputs(w, layer, step, tokens)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if w.x_dtype == "bf16" else torch.from_numpy(x)
    return xt.to(device), torch.from_numpy(logits).to(device)
