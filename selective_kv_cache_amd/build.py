"""Build libkvb.so (HIP for gfx950) in-tree with hipcc.

Each source is compiled to an object of its own (in parallel) and the objects
are linked into selective_kv_cache_amd/libkvb.so.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkvb.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-Wno-unused-command-line-argument",
]

# Per-source flag overrides (none needed at present).
PER_FILE_FLAGS = {}


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd[-3:])}")


def build(verbose: bool = False, extra=()) -> str:
    """Compile every HIP source and link selective_kv_cache_amd/libkvb.so; returns its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="kvb_build_") as tmp:
        jobs = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            flags = HIPCC_FLAGS + PER_FILE_FLAGS.get(os.path.basename(src), []) + list(extra)
            jobs.append(([hipcc, *flags, *inc, "-c", src, "-o", obj], obj))
        with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            list(ex.map(lambda j: _run(j[0], verbose), jobs))
        out = LIB + ".tmp"
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o in jobs], "-o", out], verbose)
        os.replace(out, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
