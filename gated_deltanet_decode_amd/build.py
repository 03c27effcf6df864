"""Build libgdn.so (the HIP library) in-tree for gfx950.

    python gated_deltanet_decode_amd/build.py

Run it as a file (or load it by path): importing the package itself loads the
library this script produces.

Every HIP source compiles with -ffp-contract=off (the per-token arithmetic
spells out each fused multiply-add, so decode, tree verify and commit round
identically) and with packed-fp32 instruction selection turned off.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgdn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument", "-Wno-unknown-pragmas",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
SOURCES = ["gdn_api.hip", "gdn_decode.hip", "gdn_token.hip", "gdn_tree.hip", "gdn_prefill.hip", "gdn_state.hip",
           "gdn_selfcheck.hip", "gdn_noalloc.hip"]
# The prefill kernels keep their MFMA accumulators in ordinary VGPRs: the scan
# scales and converts its state accumulators every chunk, which would otherwise
# cost a copy out of and back into the accumulation registers each time.
EXTRA = {"gdn_prefill.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        # host pass warns that it does not know the gfx950-only feature; keep other warnings visible
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and "not a recognized feature" not in l]
        if any(l.strip() for l in lines):
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
