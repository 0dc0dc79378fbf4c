"""Build libsrmoe.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m shared_routed_expert_amd.build

Each source is compiled to its own object in parallel (every translation unit holds
its kernels and their host launchers), then the objects are linked into the library.
The library is stamped with source_hash() of the sources it was built from
(srmoe_source_hash); the binding refuses a library whose stamp differs from the
sources beside it.
"""
from __future__ import annotations

import glob
import hashlib
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


def source_hash() -> str:
    """First 16 hex digits of the sha256 over every csrc/*.hip, csrc/*.hpp and include/*.h
    file (sorted by path relative to the repository root; each path, then its bytes)."""
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp"))
                   + glob.glob(os.path.join(ROOT, "include", "*.h")))
    h = hashlib.sha256()
    for f in sorted(files, key=lambda f: os.path.relpath(f, ROOT)):
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)  # the host pass does not know that feature
    return r.returncode, msgs


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    flags = [*FLAGS, f'-DSRMOE_SOURCE_HASH="{source_hash()}"']
    jobs = []
    for s in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(s)[0] + ".o")
        jobs.append((s, obj, [HIPCC, *flags, "-c", os.path.join(CSRC, s), "-o", obj]))
    if verbose:
        print(f"{HIPCC} {' '.join(flags)} -c <each of {', '.join(SOURCES)}>", flush=True)
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
