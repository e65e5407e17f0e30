"""Build ``libqlr.so`` (gfx950 kernels + host library) in-tree with hipcc.

Usage: ``python -m quantized_base_fine_amd.build`` or ``build()`` from Python.
Every source compiles to its own object under ``_build/`` (in parallel), then
one shared library is linked next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libqlr.so")

SOURCES = ["qlr_host.cpp", "qlr_quant.hip", "qlr_linear_f32.hip", "qlr_gemv.hip", "qlr_gemm.hip", "qlr_bwd.hip",
           "qlr_dba.hip", "qlr_outliers.hip", "qlr_wha.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed float32 ops stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def source_files():
    """Every file the library is built from (kernels, host code, headers), in a fixed order."""
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith((".hip", ".cpp", ".h"))]
    return files + [os.path.join(ROOT, "include", "qlr.h")]


def source_hash() -> str:
    """sha256 over the library's sources (names and contents); built into the library."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.relpath(path, ROOT).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _stamp() -> str:
    """A translation unit that exports the source hash as a data symbol."""
    path = os.path.join(BUILD, "qlr_stamp.cpp")
    text = f'extern "C" __attribute__((visibility("default"))) const char qlr_source_sha256[65] = "{source_hash()}";\n'
    with open(path, "w") as f:
        f.write(text)
    obj = path + ".o"
    res = subprocess.run([hipcc(), "-O2", "-fPIC", "-c", path, "-o", obj], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for the source stamp:\n{res.stderr}")
    return obj


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    workers = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    objs.append(_stamp())
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
