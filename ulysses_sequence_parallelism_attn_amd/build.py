"""Build libulattn.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Usage: ``python -m ulysses_sequence_parallelism_attn_amd.build`` or
``build.build()``.  Every call recompiles.  Objects go to ``_build/`` next to the
package; the library lands in the package directory, where the binding loads it.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
OUT = PKG / "libulattn.so"
BUILD_DIR = ROOT / "_build"
ARCH = "gfx950"

SOURCES = ["api.cpp", "relayout.hip", "attn_fwd.hip", "attn_bwd.hip"]

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # never let the compiler form packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{ROOT / 'include'}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    return "hipcc"


def _compile(src: str, verbose: bool) -> Path:
    obj = BUILD_DIR / (Path(src).stem + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [_hipcc(), *FLAGS, *lang, "-c", str(CSRC / src), "-o", str(obj)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    warn = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if warn and verbose:
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> Path:
    """Compile every HIP source and link libulattn.so; returns its path."""
    BUILD_DIR.mkdir(exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT.with_suffix(".so.tmp")
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp),
           *map(str, objs)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
