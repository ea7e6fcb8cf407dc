"""Build libssd_mi355x.so (gfx950 only) in-tree with hipcc.

    python -m mamba_ssd_scan_02_amd.csrc.build [-v]

Every translation unit is compiled for gfx950 with packed-fp32 instruction
selection switched off, then linked into one shared library next to the
package's __init__.py.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

CSRC = Path(__file__).resolve().parent
PKG = CSRC.parent
ROOT = PKG.parent
INCLUDE = ROOT / "include"
BUILD = PKG / "_build"
LIB = PKG / "libssd_mi355x.so"

SOURCES = [
    "chunk_cumsum.hip",
    "chunk_state.hip",
    "state_passing.hip",
    "chunk_scan.hip",
    "state_scan.hip",
    "layer.hip",
    "ssm_step.hip",
    "ssd_api.cpp",
]

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(str(c) for c in cmd), flush=True)
    res = subprocess.run([str(c) for c in cmd], capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(map(str, cmd))}\n{err}")
    if verbose and err.strip():
        print(err, flush=True)


def build(verbose: bool = False, jobs: int | None = None) -> Path:
    hipcc = _hipcc()
    BUILD.mkdir(exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = BUILD / (src + ".o")
        objs.append(obj)
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        cmds.append([hipcc, *COMMON, *lang, "-c", CSRC / src, "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs or min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB.with_suffix(".so.tmp")
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
