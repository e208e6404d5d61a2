"""Build libzgattn.so for gfx950 in-tree (``python -m global_attention_zg_amd.build``).

Each HIP source is compiled to an object under ``_build/`` in parallel, then
linked into ``global_attention_zg_amd/libzgattn.so``.  Packed-fp32 VALU ops
are disabled for all device code, and floating-point contraction is off: the
kernels place every fused multiply-add explicitly, so that their rounding does
not depend on how the compiler schedules a code path.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libzgattn.so")
SOURCES = ["prologue.hip", "flash_fwd.hip", "flash_causal.hip", "decode.hip", "backward.hip", "gemm.hip", "api.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


CFLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source extra flags.  The causal kernel keeps its output accumulators in
# AGPRs through inline asm and wants every other MFMA result (the scores,
# which the softmax reads) written straight to VGPRs.
# The atomic optimizer is off there too: it would turn the work-queue claim
# (one lane's atomic add) into a wave-wide form that reads the result at
# once, where the kernel wants to read it only after the job's epilogue.
SOURCE_FLAGS = {"flash_causal.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true",
                                     "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns about the device-only target feature; drop that line
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "warning: feature flag" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=()) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []

    def one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        out = _run([cc, *CFLAGS, *SOURCE_FLAGS.get(src, []), *extra_flags, "-c",
                    os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
