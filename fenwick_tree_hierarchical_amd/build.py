"""Build liblogattn.so in-tree with hipcc for gfx950.

    python -m fenwick_tree_hierarchical_amd.build

Each HIP translation unit is compiled to an object in parallel, then linked
into ``fenwick_tree_hierarchical_amd/liblogattn.so`` next to this file.
Objects go to ``fenwick_tree_hierarchical_amd/_build/``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblogattn.so")
SOURCES = ["la_abi.hip", "la_fwd_bf16.hip", "la_fwd_f32.hip", "la_bwd_bf16.hip", "la_bwd_f32.hip", "la_decode.hip",
           "la_gdn_bf16.hip", "la_gdn_f32.hip", "la_layer_bf16.hip", "la_layer_f32.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build liblogattn")
    return h


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        # packed fp32 arithmetic is kept off: only scalar and MFMA fp32 code is emitted
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose: bool = True, jobs: int | None = None) -> str:
    os.makedirs(OUT, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
