"""Build libgdn.so (hand-written HIP kernels for gfx950 + the C ABI) in-tree.

    python -m gated_deltanet_gdn_amd.build        # or: python gated_deltanet_gdn_amd/build.py

Each source compiles to an object with hipcc (in parallel), then links into
gated_deltanet_gdn_amd/libgdn.so. Packed-fp32 instruction selection is turned
off for every device pass (plain scalar/float2 fp32 code only).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdn.so")

ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["gdn_api.cpp", "k_elementwise.hip", "k_conv.hip", "k_recurrent.hip", "k_chunk.hip"]

COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# The chunk kernels run one workgroup per CU (their LDS needs), so the compiler
# would place MFMA accumulators in AGPRs and copy them out for every VALU use;
# keep MFMA results in VGPRs.
EXTRA = {"k_chunk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx feature flag; that warning is harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
