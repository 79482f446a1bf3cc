"""Build libgdn.so (all HIP sources, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(LIB_DIR, "libgdn.so")
SOURCES = ["gdn_window.hip", "gdn_window_mfma.hip", "gdn_kda.hip",
           "gdn_kda_mfma.hip", "gdn_prefill.hip", "gdn_state.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: the per-step state update must be the same
#   multiply-then-FMA in verify and commit (bit-exact replay).
# -packed-fp32-ops off: packed FP32 VALU forms are kept out of the build.
FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC",
         "-ffp-contract=off", "-fno-fast-math",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]
# The prefill state chain scales and splits its MFMA accumulators every
# chunk; keeping them in ordinary VGPRs avoids a copy through AGPRs.
EXTRA = {"gdn_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(LIB_DIR, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
           *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
