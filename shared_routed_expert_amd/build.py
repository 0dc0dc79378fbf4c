"""Build libsrmoe.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m shared_routed_expert_amd.build

Each source is compiled to its own object in parallel (every translation unit holds
its kernels and their host launchers), then the objects are linked into the library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsrmoe.so")
SOURCES = ["api.hip", "router.hip", "route.hip", "align.hip", "quant.hip", "ffn.hip", "ffn_decode.hip",
           "ffn_expert_decode.hip", "ffn_tile.hip", "front.hip", "qknorm.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)  # the host pass does not know that feature
    return r.returncode, msgs


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for s in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(s)[0] + ".o")
        jobs.append((s, obj, [HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", obj]))
    if verbose:
        print(f"{HIPCC} {' '.join(FLAGS)} -c <each of {', '.join(SOURCES)}>", flush=True)
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(workers) as pool:
        results = list(pool.map(lambda j: (j[0], *_run(j[2])), jobs))
    errs = [f"{s}:\n{m}" for s, rc, m in results if rc != 0]
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose:
        for s, _, m in results:
            if m.strip():
                print(f"{s}: {m}", flush=True)
    tmp = LIB + ".tmp"
    rc, msgs = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[j[1] for j in jobs], "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{msgs}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
