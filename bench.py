"""Benchmark of the routed low-bit expert FFN hot path on one MI355X.

A step is one pass of the whole path over one batch: for every layer of the
workload, routing + bucketing, dequant-fused gate/up + SwiGLU, down and the
weighted combine, layer after layer on one stream (no cross-layer lookahead:
layer l+1's call is enqueued after layer l's and reads its own fresh inputs).
All experts of all layers are resident in HBM and every step's activations and
logits are generated and uploaded before the timed region.  The timed region
replays a HIP graph holding the K steps.

Prints one JSON line (rank 0).  Default workload: the 48-layer x 512-expert
2-bit decode stack, one token per step.  `--workload prefill` measures the
matrix-core path instead: a step is the 4,096-token prompt through all 4
layers (256 experts, top-8, H 7168, FF 2048, 4-bit), launched eagerly with HIP
events at every kernel boundary, reported as prompt tokens/s and as the
dominant kernel's algorithmic TFLOP/s against the dense bf16 MFMA peak.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE decode tokens/s (expert stack) + achieved HBM GB/s as % of 8 TB/s"
PREFILL_METRIC = "MoE prefill prompt tokens/s + grouped-GEMM TFLOP/s as % of dense bf16 MFMA peak"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PREFILL_KERNELS = ["route_topk_kernel", "prefill_count_kernel", "prefill_place_kernel", "prefill_gateup_kernel",
                   "prefill_down_kernel", "prefill_combine_kernel"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes_per_layer(w, ids_np):
    """Bytes the method must move for one layer call: each distinct selected
    expert's blob once, the shared expert, activations in, logits in, fp32
    outputs out."""
    uniq = len(np.unique(ids_np))
    return (uniq * w.blob_bytes + w.shared_blob_bytes + w.tokens * w.hidden * (2 if w.x_dtype == "bf16" else 4)
            + w.tokens * w.experts * 4 + w.tokens * w.hidden * 4), uniq


def gpu_clocks():
    """Current shader (sclk) and memory (mclk) clocks in MHz of the first GPU,
    read from the amdgpu sysfs DPM tables (the level marked '*'), else from
    rocm-smi; None where neither is readable."""
    import glob
    import re
    out = {}
    for name in ("sclk", "mclk"):
        for f in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{name}")):
            try:
                for line in open(f):
                    if "*" in line:
                        m = re.search(r"(\d+)\s*Mhz", line, re.I)
                        if m:
                            out[name + "_mhz"] = int(m.group(1))
            except OSError:
                pass
            if name + "_mhz" in out:
                break
    if len(out) < 2:
        try:
            import subprocess
            r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
            d = json.loads(r.stdout)
            card = d[sorted(d)[0]]
            for key, v in card.items():
                k = key.lower()
                for name in ("sclk", "mclk"):
                    if f"({name})" in k and name + "_mhz" not in out:
                        m = re.search(r"(\d+)", str(v))
                        if m:
                            out[name + "_mhz"] = int(m.group(1))
        except Exception:
            pass
    return {"sclk_mhz": out.get("sclk_mhz"), "mclk_mhz": out.get("mclk_mhz"), "sampled": "after the timed repeats"}


def host_cores():
    """Host CPUs: os.cpu_count() and the CPUs this process may run on."""
    return {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


class one_core:
    """Runs the enclosed code pinned to one CPU (the first this process may
    use), restoring the affinity afterwards."""

    def __enter__(self):
        self.saved = os.sched_getaffinity(0)
        self.cpu = min(self.saved)
        os.sched_setaffinity(0, {self.cpu})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.saved)
        return False


def kernel_source_hash():
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "bit_expert_ffn_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by a copy-kernel
    calibration), or None when the kernel sources changed since the counters
    were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.loads(f.readline())
    return t["traffic_bytes_per_launch"] if t.get("source_hash") == kernel_source_hash() else None


def cpu_baseline(w, x_host, l_host, budget_s=12.0):
    """The float64 oracle, single-threaded, on a bounded sample: whole decode
    steps (all layers, all tokens of the step) until the budget is spent."""
    import oracle
    import synth
    from synth import workloads as wl
    t_total = 0.0
    steps = 0
    ref = None
    while t_total < budget_s:
        for l in range(w.layers):
            ids_ref, _ = oracle.route_topk(l_host[steps][l], w.top_k)
            need = sorted(set(ids_ref.reshape(-1).tolist()))
            zero = np.zeros(w.blob_bytes, dtype=np.uint8)
            blobs = {e: synth.expert_blob(w.seed, l, e, w.qk, w.hidden, w.ff, w.sigma) for e in need}
            table = [blobs.get(e, zero) for e in range(w.experts)]
            shared = wl.host_shared_blob(w, l)
            t0 = time.perf_counter()
            y, _, _ = oracle.layer_forward(table, w.top_k, w.qtype, w.zero_point, w.hidden, w.ff,
                                           x_host[steps][l], l_host[steps][l], shared=shared, shared_ff=w.shared_ff)
            t_total += time.perf_counter() - t0
            if steps == 0 and l == w.layers - 1:
                ref = y
        steps += 1
        if steps >= len(x_host):
            break
    tok = steps * w.tokens
    return {"value": tok / t_total, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full step(s) x {w.layers} layers x {w.tokens} token(s) of the same workload, "
                      f"float64 oracle single-threaded, pinned to one CPU, {t_total:.1f} s",
            "host": host_cores()}, ref


def router_timing(args, w, arena, x_step, desc, ws, stream, n_layers, eager_layer_ms):
    """The router front end's added time at this workload (the logits are
    otherwise an input): synthetic bf16 router weights N(0, 0.02) per layer
    (the Gemma-shaped workload also runs the weightless norm and a
    per-input-dim scale); HIP events on the launch stream around (a) the router
    alone and (b) the layer call with the router inside it, eagerly per layer,
    three passes.  The eager layer without the router is `eager_layer_ms`."""
    import torch

    import bit_expert_ffn_amd as moe
    gen = torch.Generator(device="cuda").manual_seed(1234)
    wr = [(torch.randn((w.experts, w.hidden), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
          for _ in range(n_layers)]
    gemma = w.shared_ff > 0
    scale = torch.rand((w.hidden,), generator=gen, device="cuda") + 0.5 if gemma else None
    rts = [moe.router(wr[l], scale, norm=gemma, eps=1e-6) for l in range(n_layers)]
    lg = torch.empty((w.tokens, w.experts), dtype=torch.float32, device="cuda")
    y = torch.empty((w.tokens, w.hidden), dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_layers)]
    t_router, t_layer = [], []
    for rep in range(4):
        for which in ("router", "layer"):
            with torch.cuda.stream(stream):
                for l in range(n_layers):
                    evs[l][0].record(stream)
                    if which == "router":
                        moe.router_logits(rts[l], w.experts, x_step[l], logits=lg, stream=stream)
                    else:
                        moe.layer_forward_ex(desc, arena.tables[l], x_step[l], shared=arena.shared_blob(l), rt=rts[l],
                                             y=y, ws=ws, stream=stream)
                    evs[l][1].record(stream)
            torch.cuda.synchronize()
            if rep > 0:   # the first pass warms up
                (t_router if which == "router" else t_layer).extend(a.elapsed_time(b) for a, b in evs)
    r_us, l_us = float(np.mean(t_router)) * 1e3, float(np.mean(t_layer)) * 1e3
    r_bytes = w.experts * w.hidden * 2 + w.tokens * w.hidden * (2 if w.x_dtype == "bf16" else 4) + \
        w.tokens * w.experts * 4 + (w.hidden * 4 if gemma else 0)
    return {"kernel": "router_gemv_kernel", "options": "weightless RMS norm + per-input-dim scale" if gemma
            else "plain", "router_us": round(r_us, 3), "router_bytes": int(r_bytes),
            "router_gbps": round(r_bytes / (r_us * 1e-6) / 1e9, 1),
            "layer_with_router_us": round(l_us, 3), "layer_eager_us": round(eager_layer_ms * 1e3, 3),
            "added_us_per_layer": round(l_us - eager_layer_ms * 1e3, 3),
            "timing": "eager, HIP events per call on the launch stream, 3 passes x all layers"}


def prefill_flops(w, n_slots, T):
    """Algorithmic flops of one layer's two grouped GEMM stages: gate and up are
    2 x (H x FF) multiply-adds per routed slot, down one more (plus the shared
    expert's per token)."""
    gu = 2 * 2 * w.hidden * (w.ff * n_slots + w.shared_ff * T)
    dn = 2 * w.hidden * (w.ff * n_slots + w.shared_ff * T)
    return gu, dn


def prefill_sample(w, l0, n=64):
    """A deterministic sample of n prompt tokens of layer 0: a token routed to
    the hottest expert, one routed to the coldest, then the first tokens."""
    import oracle
    ids, _ = oracle.route_topk(l0, w.top_k)
    counts = np.bincount(ids.reshape(-1), minlength=w.experts)
    hot, cold = int(np.argmax(counts)), int(np.argmin(counts))
    pick = [int(np.nonzero((ids == hot).any(1))[0][0]), int(np.nonzero((ids == cold).any(1))[0][0])]
    for t in range(w.tokens):
        if len(pick) >= n:
            break
        if t not in pick:
            pick.append(t)
    return sorted(pick), hot, cold


def prefill_cpu_baseline(w, x0, l0, got, n=64):
    """The float64 oracle, single-threaded, on a bounded sample of layer 0 of
    the prompt: 64 tokens including ones routed to the hottest and the coldest
    expert (each token's routing and experts are independent of the others).
    Also returns the GPU output's max |err| / rms on the sampled tokens."""
    import oracle
    import synth
    from synth import workloads as wl
    sample, hot, cold = prefill_sample(w, l0, n)
    zero = np.zeros(w.blob_bytes, dtype=np.uint8)
    cache = {}
    t_total, refs = 0.0, []
    for c in range(0, len(sample), 4):
        rows = sample[c:c + 4]
        x, lg = x0[rows], l0[rows]
        ids_ref, _ = oracle.route_topk(lg, w.top_k)
        for e in set(ids_ref.reshape(-1).tolist()):
            if e not in cache:
                cache[e] = synth.expert_blob(w.seed, 0, e, w.qk, w.hidden, w.ff, w.sigma)
        table = [cache.get(e, zero) for e in range(w.experts)]
        t0 = time.perf_counter()
        y, _, _ = oracle.layer_forward(table, w.top_k, w.qtype, w.zero_point, w.hidden, w.ff, x, lg,
                                       shared=wl.host_shared_blob(w, 0), shared_ff=w.shared_ff)
        t_total += time.perf_counter() - t0
        refs.append(y)
    ref = np.concatenate(refs)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got[sample] - ref))) / rms
    return ({"value": len(sample) / t_total, "unit": "tokens/s", "cores": 1, "kind": "oracle",
             "sample": f"{len(sample)} of the {w.tokens} prompt tokens of layer 0 (tokens routed to the hottest "
                       f"expert {hot} and the coldest expert {cold}, then the first tokens), float64 oracle "
                       f"single-threaded, pinned to one CPU, {t_total:.1f} s",
             "host": host_cores()},
            err, len(sample))


def bench_prefill(args, w):
    import torch

    import bit_expert_ffn_amd as moe
    from synth import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K = args.steps if args.steps is not None else 10
    W = args.warmup if args.warmup is not None else 2
    nsteps = K + W
    t0 = time.time()
    arena = wl.DeviceArena(w, device=dev, progress=lambda l: log(f"arena layer {l + 1}/{w.layers}"))
    log(f"arena ready: {w.layers} x {w.experts} x {w.blob_bytes} B in {time.time() - t0:.1f} s")

    x_dt = torch.bfloat16 if w.x_dtype == "bf16" else torch.float32
    xs = torch.empty((nsteps, w.layers, w.tokens, w.hidden), dtype=x_dt, device=dev)
    lg = torch.empty((nsteps, w.layers, w.tokens, w.experts), dtype=torch.float32, device=dev)
    x0 = l0 = None
    for s in range(nsteps):
        for l in range(w.layers):
            xh, lh = wl.host_inputs(w, l, s)
            if s == W and l == 0:
                x0, l0 = xh, lh
            xs[s, l].copy_(torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16) if w.x_dtype == "bf16"
                           else torch.from_numpy(xh))
            lg[s, l].copy_(torch.from_numpy(lh))
    log(f"inputs resident: {nsteps} steps x {w.layers} layers x {w.tokens} tokens")

    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k, shared_ff=w.shared_ff)
    ws = moe.workspace(moe.layer_workspace_bytes(desc, w.tokens), dev)
    y = torch.empty((2, w.tokens, w.hidden), dtype=torch.float32, device=dev)
    y_first = torch.empty((w.tokens, w.hidden), dtype=torch.float32, device=dev)
    ids = torch.empty((nsteps, w.layers, w.tokens, w.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((nsteps, w.layers, w.tokens, w.top_k), dtype=torch.float32, device=dev)
    nk = len(PREFILL_KERNELS)
    stream = torch.cuda.Stream()
    # One event per kernel boundary of every timed layer call; each is recorded
    # once up front so that its HIP event exists before the library records it.
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(w.layers)]
           for _ in range(K)]
    with torch.cuda.stream(stream):
        for a in evs:
            for b in a:
                for e in b:
                    e.record(stream)

    def layer(s, l, events=None):
        out = y_first if (s == W and l == 0) else y[l % 2]
        if events is None:
            moe.layer_forward(desc, arena.tables[l], xs[s, l], lg[s, l], shared=arena.shared_blob(l), y=out,
                              ids=ids[s, l], weights=wts[s, l], ws=ws, stream=stream)
        else:
            _, n = moe.layer_forward_timed(desc, arena.tables[l], xs[s, l], lg[s, l], events,
                                           shared=arena.shared_blob(l), y=out, ids=ids[s, l], weights=wts[s, l],
                                           ws=ws, stream=stream)
            assert n == nk, n

    with torch.cuda.stream(stream):
        for s in range(W):
            for l in range(w.layers):
                layer(s, l)
    torch.cuda.synchronize()
    # The K timed steps, run `repeats` times, each run bracketed by HIP events
    # on the launch stream and a device synchronisation; value = the median
    # run.  Per-kernel durations come from the boundary events of every run.
    reps_ms = []
    dur = np.zeros((args.repeats, K, w.layers, nk))
    t_wall = time.perf_counter()
    for rep in range(args.repeats):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            ev0.record(stream)
            for i, s in enumerate(range(W, nsteps)):
                for l in range(w.layers):
                    layer(s, l, evs[i][l])
            ev1.record(stream)
        torch.cuda.synchronize()
        reps_ms.append(ev0.elapsed_time(ev1))
        for i in range(K):
            for l in range(w.layers):
                for j in range(nk):
                    dur[rep, i, l, j] = evs[i][l][j].elapsed_time(evs[i][l][j + 1])
        log(f"repeat {rep + 1}/{args.repeats}: {reps_ms[-1] / K:.3f} ms per step")
    t_wall = (time.perf_counter() - t_wall) / args.repeats
    clocks = gpu_clocks()
    ms_total = float(np.median(reps_ms))
    ms_step = ms_total / K
    tok_s = K * w.tokens / (ms_total / 1e3)
    avg_ms = dur.mean(axis=(0, 1, 2))
    n_slots = w.tokens * w.top_k
    gu, dn = prefill_flops(w, n_slots, w.tokens)
    layer_flops = gu + dn
    step_tflops = w.layers * layer_flops / (ms_step / 1e3) / 1e12
    stages = {}
    for j, name in enumerate(PREFILL_KERNELS):
        st = {"avg_us": round(avg_ms[j] * 1e3, 2), "share": round(float(avg_ms[j] / avg_ms.sum()), 4)}
        if name == "prefill_gateup_kernel":
            st["tflops"] = round(gu / (avg_ms[j] / 1e3) / 1e12, 1)
        if name == "prefill_down_kernel":
            st["tflops"] = round(dn / (avg_ms[j] / 1e3) / 1e12, 1)
        stages[name] = st
    j_dom = 3 if avg_ms[3] >= avg_ms[4] else 4
    dom = PREFILL_KERNELS[j_dom]
    dom_flops = gu if j_dom == 3 else dn
    achieved = dom_flops / (avg_ms[j_dom] / 1e3) / 1e12

    ids_np = ids[W:].cpu().numpy()
    uniq = float(np.mean([len(np.unique(ids_np[i, l])) for i in range(K) for l in range(w.layers)]))
    # Algorithmic HBM bytes of the dominant kernel: the weights it multiplies
    # (gate+up, or down, of every expert with tokens) once, its gathered inputs
    # once, its outputs once.
    mat_bytes = w.blob_bytes // 3
    if j_dom == 3:
        dom_bytes = uniq * 2 * mat_bytes + n_slots * w.hidden * 2 + n_slots * w.ff * 4
    else:
        dom_bytes = uniq * mat_bytes + n_slots * w.ff * 4 + n_slots * w.hidden * 4

    result = {
        "metric": PREFILL_METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "experts": w.experts, "hidden": w.hidden, "ff": w.ff,
                   "top_k": w.top_k, "tokens_per_step": w.tokens, "format": "4-bit/32 + fp16 scale"
                   if w.qtype == 2 else "2-bit/64 + fp16 scale", "shared_ff": w.shared_ff, "graph": False},
        "step_tflops": round(step_tflops, 1), "mfma_frac_step": round(step_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "flops_per_layer": int(layer_flops), "distinct_experts_per_layer": round(uniq, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(w.name), "kernel": dom,
                     "launch_us": round(avg_ms[j_dom] * 1e3, 2), "flops_per_launch": int(dom_flops),
                     "bytes_per_launch": int(dom_bytes)},
        "stages": stages,
        "wall_s": round(t_wall, 4),
        "repeats": args.repeats, "median_ms_per_step": round(ms_step, 4),
        "min_ms_per_step": round(min(reps_ms) / K, 4),
        "max_tokens_per_s": round(K * w.tokens / (min(reps_ms) / 1e3), 1),
        "repeat_ms": [round(r, 3) for r in reps_ms], "clocks": clocks, "host_cores": host_cores(),
    }
    if not args.no_cpu_baseline:
        got = y_first.cpu().numpy()
        with one_core():
            base, err, n = prefill_cpu_baseline(w, x0, l0, got)
        result["cpu_baseline"] = base
        result["parity_max_err_over_rms"] = err
        result["parity_tokens"] = n
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 100 decode, 10 prefill)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 10 decode, 2 prefill)")
    ap.add_argument("--workload", default="strata_decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--repeats", type=int, default=5, help="timed repeats of the K steps (value = median)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run only a plain fp32 elementwise copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--calibrate-copy64", type=int, default=0, metavar="MIB",
                    help="run only a copy of MIB MiB read as 64-byte runs, one per 128 bytes of a source twice "
                         "as large (counter calibration for kernels whose requests are 64 B) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (expert parallelism is a design note "
              "only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        # A plain copy kernel of known size: reads and writes MIB MiB once per launch.
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "fp32 neg copy", "bytes_read": 4 * n, "bytes_written": 4 * n,
                          "launches": 3}), flush=True)
        return
    if args.calibrate_copy64:
        # Reads 16 of every 32 floats (one 64-byte run per 128 bytes) and writes them packed.
        n = args.calibrate_copy64 * (1 << 20) // 4
        src = torch.ones((n // 16, 32), dtype=torch.float32, device="cuda")
        dst = torch.empty((n // 16, 16), dtype=torch.float32, device="cuda")
        for _ in range(3):
            dst.copy_(src[:, :16])
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "fp32 copy of 64-byte runs", "bytes_read": 4 * n, "bytes_written": 4 * n,
                          "launches": 3}), flush=True)
        return

    import bit_expert_ffn_amd as moe
    from synth import workloads as wl

    w = wl.WORKLOADS[args.workload]
    if w.tokens > 8:
        bench_prefill(args, w)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K = args.steps if args.steps is not None else 100
    W = args.warmup if args.warmup is not None else 10
    nsteps = K + W

    t0 = time.time()
    arena = wl.DeviceArena(w, device=dev, progress=lambda l: log(f"arena layer {l + 1}/{w.layers}")
                           if (l + 1) % 12 == 0 else None)
    log(f"arena ready: {w.layers} x {w.experts} x {w.blob_bytes} B in {time.time() - t0:.1f} s")

    # Fresh activations and logits for every (step, layer), resident before timing.
    x_host, l_host = [], []
    xs = torch.empty((nsteps, w.layers, w.tokens, w.hidden),
                     dtype=torch.bfloat16 if w.x_dtype == "bf16" else torch.float32, device=dev)
    lg = torch.empty((nsteps, w.layers, w.tokens, w.experts), dtype=torch.float32, device=dev)
    for s in range(nsteps):
        xr, lr = [], []
        for l in range(w.layers):
            xh, lh = wl.host_inputs(w, l, s)
            xr.append(xh)
            lr.append(lh)
            xs[s, l].copy_(torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16) if w.x_dtype == "bf16"
                           else torch.from_numpy(xh))
            lg[s, l].copy_(torch.from_numpy(lh))
        x_host.append(xr)
        l_host.append(lr)

    desc = moe.layer_desc(w.hidden, w.ff, w.qtype, w.zero_point, w.experts, w.top_k, shared_ff=w.shared_ff)
    ws = moe.workspace(moe.layer_workspace_bytes(desc, w.tokens), dev)
    y = torch.empty((nsteps, w.layers, w.tokens, w.hidden), dtype=torch.float32, device=dev)
    ids = torch.empty((nsteps, w.layers, w.tokens, w.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((nsteps, w.layers, w.tokens, w.top_k), dtype=torch.float32, device=dev)

    def run_steps(s0, s1, stream):
        for s in range(s0, s1):
            for l in range(w.layers):
                moe.layer_forward(desc, arena.tables[l], xs[s, l], lg[s, l], shared=arena.shared_blob(l),
                                  y=y[s, l], ids=ids[s, l], weights=wts[s, l], ws=ws, stream=stream)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    if args.no_graph:
        def replay_warm():
            run_steps(0, W, stream)

        def replay_timed():
            run_steps(W, nsteps, stream)
    else:
        g_warm, g_timed = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            # one eager pass first (library initialisation outside capture)
            run_steps(0, 1, stream)
            stream.synchronize()
            with torch.cuda.graph(g_warm, stream=stream):
                run_steps(0, W, stream)
            with torch.cuda.graph(g_timed, stream=stream):
                run_steps(W, nsteps, stream)

        def replay_warm():
            with torch.cuda.stream(stream):
                g_warm.replay()

        def replay_timed():
            with torch.cuda.stream(stream):
                g_timed.replay()

    replay_warm()
    torch.cuda.synchronize()
    # The K timed steps, replayed `repeats` times; each replay is bracketed by
    # HIP events on the launch stream and a device synchronisation on both
    # sides.  value = the median replay; the minimum is reported beside it.
    reps_ms = []
    t_wall = time.perf_counter()
    for _ in range(args.repeats):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        replay_timed()
        ev1.record(stream)
        torch.cuda.synchronize()
        reps_ms.append(ev0.elapsed_time(ev1))
    t_wall = (time.perf_counter() - t_wall) / args.repeats
    clocks = gpu_clocks()
    ms_total = float(np.median(reps_ms))
    ms_step = ms_total / K
    tok_s = K * w.tokens / (ms_total / 1e3)

    # Algorithmic bytes of the timed steps, from the routing the GPU produced.
    ids_np = ids.cpu().numpy()
    bytes_steps, uniq_tot = 0, 0
    for s in range(W, nsteps):
        for l in range(w.layers):
            b, u = algorithmic_bytes_per_layer(w, ids_np[s, l])
            bytes_steps += b
            uniq_tot += u
    gbps = bytes_steps / (ms_total / 1e3) / 1e9

    # The dominant (and only) kernel of a decode step is the fused layer kernel,
    # launched once per layer: its average duration over the timed region is
    # the step time divided by the layers.
    layer_ms = ms_step / w.layers
    bytes_layer = bytes_steps / (K * w.layers)
    achieved = bytes_layer / (layer_ms / 1e3) / 1e9

    # Eager launches with one HIP event pair per layer call, on the launch stream.
    n_ev = min(w.layers, 48)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    durs = []
    for rep in range(3):
        s = W + (rep % K)
        with torch.cuda.stream(stream):
            for l in range(n_ev):
                evs[l][0].record(stream)
                moe.layer_forward(desc, arena.tables[l], xs[s, l], lg[s, l], shared=arena.shared_blob(l),
                                  y=y[s, l], ids=ids[s, l], weights=wts[s, l], ws=ws, stream=stream)
                evs[l][1].record(stream)
        torch.cuda.synchronize()
        durs += [a.elapsed_time(b) for a, b in evs]
    eager_layer_ms = float(np.mean(durs))
    router = router_timing(args, w, arena, xs[W], desc, ws, stream, n_ev, eager_layer_ms)

    result = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "experts": w.experts, "hidden": w.hidden, "ff": w.ff,
                   "top_k": w.top_k, "tokens_per_step": w.tokens,
                   "format": "2-bit/64 + fp16 scale" if w.qtype == 1 else "4-bit/32 + fp16 scale",
                   "shared_ff": w.shared_ff, "graph": not args.no_graph},
        "hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "bytes_per_step": int(bytes_steps / K), "distinct_experts_per_layer": round(uniq_tot / (K * w.layers), 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(w.name),
                     "kernel": ("decode_layer_kernel" if w.tokens == 1 else "window_layer_kernel") + " (one launch per layer)",
                     "launch_us": round(layer_ms * 1e3, 3),
                     "bytes_per_launch": int(bytes_layer), "eager_launch_us": round(eager_layer_ms * 1e3, 3)},
        "wall_s": round(t_wall, 4),
        "router": router,
        "repeats": args.repeats, "median_ms_per_step": round(ms_step, 5),
        "min_ms_per_step": round(min(reps_ms) / K, 5),
        "max_tokens_per_s": round(K * w.tokens / (min(reps_ms) / 1e3), 2),
        "repeat_ms": [round(r, 4) for r in reps_ms], "clocks": clocks, "host_cores": host_cores(),
    }
    if not args.no_cpu_baseline:
        with one_core():
            base, ref = cpu_baseline(w, x_host, l_host)
        result["cpu_baseline"] = base
        got = y[0, w.layers - 1].cpu().numpy()
        rms = float(np.sqrt(np.mean(ref ** 2)))
        result["parity_max_err_over_rms"] = float(np.max(np.abs(got - ref)) / rms)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
