"""Build libmoe_ffn.so (HIP for gfx950) in-tree with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_ffn.so")
SOURCES = ["moe_api.hip", "moe_route.hip", "moe_router.hip", "moe_gemv.hip", "moe_window.hip", "moe_prefill.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                       # every fused multiply-add is written explicitly
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",         # MFMA results in VGPRs: no accumulator-register copies
    "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose=False):
    """Each source compiled to an object in parallel (every kernel is
    self-contained: no relocatable device code), then linked."""
    from concurrent.futures import ThreadPoolExecutor
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    cflags = [f for f in FLAGS if f != "-shared"]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        jobs.append((obj, [HIPCC] + cflags + ["-c", os.path.join(CSRC, src), "-o", obj]))
    if verbose:
        for _, c in jobs:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda j: _run(j[1]), jobs))
    for (obj, _), (rc, out) in zip(jobs, results):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(obj)}:\n" + out)
        if out.strip() and verbose:
            print(out)
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for o, _ in jobs] + ["-o", LIB + ".tmp"]
    rc, out = _run(link)
    if rc != 0:
        raise RuntimeError("hipcc link failed:\n" + out)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
