"""Build libpkv.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m paged_kv_cache_210_amd.build      # or __graft_entry__.build()

Every call recompiles every source (objects go to _build/, the library next
to this file)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 ops are turned off for every HIP source.
COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
          "-I" + INCLUDE, "-I" + CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for _, err in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
