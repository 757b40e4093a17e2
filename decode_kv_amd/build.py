"""Build libcsa2.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m decode_kv_amd.build

Each source compiles to its own object (in parallel), then one link.  The
library lands next to this file, where the binding looks for it.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsa2.so")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")

SOURCES = ["abi.hip", "kv_append.hip", "index_full.hip", "index_reindex.hip",
           "select_topk.hip", "sparse_attn.hip", "measure.hip", "session.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++20", "-fPIC", "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first 64 bytes of every kernel's arguments arrive in SGPRs with the
    # wave, instead of through a scalar load at its start
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I" + os.path.join(ROOT, "include"),
]


# The scoring kernels read every int8 MFMA result straight into VALU
# arithmetic (ReLU and head weight): keeping the results in VGPRs saves one
# accumulator-register read per head and token.  The attention kernel's P.V
# accumulators likewise start from zero and leave in stores without copies
# between accumulator and vector registers.
EXTRA = {
    "index_full.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "index_reindex.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "sparse_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
