"""Build libpkv.so in-tree with hipcc for gfx950.

    python paged_kv_attention_attn_amd/build.py

(run it as a file: importing the package loads the library it builds).

Every HIP translation unit is compiled with packed-FP32 instructions switched
off; host-side warnings about that target feature are expected.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libpkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["attn_kernels.hip", "accept_kernels.hip", "kv_kernels.hip", "pool_kernels.hip", "quant_kernels.hip", "host.cpp", "page_pool.cpp"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-inline-asm", "-Wno-unused-command-line-argument",
    # leading scalar kernel arguments arrive in SGPRs at wave launch (gfx950
    # kernarg preloading), so the first loads do not wait on the argument buffer
    "-mllvm", "-amdgpu-kernarg-preload-count=8",
]


def build(verbose=False):
    srcs = []
    for s in SOURCES:
        path = os.path.join(CSRC, s)
        # host.cpp carries HIP runtime calls; compile it as HIP too
        srcs += (["-x", "hip", path] if s.endswith(".cpp") else [path])
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-I", INCLUDE] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
