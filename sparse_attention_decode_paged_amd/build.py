"""Compile the HIP sources of this package into libdsa.so (gfx950), in-tree."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdsa.so")
SOURCES = ["dsa_api.cpp", "indexer.hip", "indexer_rows.hip", "indexer_mxfp4.hip", "topk.hip", "sparse_mla.hip",
           "cache_append.hip", "dcp_merge.hip", "hbm_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar / pointer kernel arguments arrive preloaded in SGPRs (gfx950)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    srcs = []
    for s in SOURCES:
        p = os.path.join(CSRC, s)
        # .cpp files hold host code only but still go through the HIP compiler
        srcs += (["-x", "hip", p, "-x", "none"] if p.endswith(".cpp") else [p])
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libdsa.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
