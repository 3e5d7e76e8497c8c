"""Build libattnres.so in-tree with hipcc for gfx950.

Each source is compiled to an object under ``_build/`` (in parallel), then the
objects are linked into ``depth_wise_attention_attnres_amd/libattnres.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libattnres.so")

SOURCES = ["attnres_api.cpp", "lds_limit.cpp", "full_fwd.hip", "full_batch.hip", "full_batch_mfma.hip", "block_fwd.hip", "block_batch.hip", "block_model.hip", "query_proj.hip", "bwd.hip", "bwd_dhist_mfma.hip", "bwd_dw_mfma.hip", "bwd_group.hip", "bwd_scratch.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU instructions stay off: the compiler would otherwise form
    # them from plain float code, and the kernels are validated without them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    # the host pass does not know the packed-fp32 feature; drop that warning only
    noise = "'-packed-fp32-ops' is not a recognized feature"
    rest = "\n".join(l for l in res.stderr.splitlines() if noise not in l).strip()
    if rest and verbose:
        print(rest, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
