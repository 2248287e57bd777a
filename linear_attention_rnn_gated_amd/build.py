"""Builds libgdn.so (HIP, gfx950) in-tree with hipcc.

Flags that are part of the arithmetic contract: -ffp-contract=off (the only
fused multiply-adds are the explicit fmaf calls), no fast-math, and packed
FP32 instructions disabled; every kernel is in one translation unit built with
the same flags.
"""

import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["gdn_kernels.hip", "gdn_plan.cpp"]
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the 4-wave chunk scan otherwise
    # splits its accumulators into AGPRs and copies them back every chunk
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall",
    "-Wno-unused-function",
]


def source_digest(extra_flags=()):
    """SHA-256 (first 16 hex digits) over the header, every source and the
    compile flags: part of gdn_contract_id(), so two builds that could differ in
    arithmetic never report the same id."""
    h = hashlib.sha256()
    for path in [os.path.join(ROOT, "include", "gdn.h"), os.path.join(CSRC, "gdn_plan.h"),
                 *[os.path.join(CSRC, s) for s in SOURCES]]:
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(" ".join([*FLAGS, *extra_flags]).encode())
    return h.hexdigest()[:16]


def build(verbose=False, extra_flags=()):
    """Compiles every source into libgdn.so; returns the library path."""
    digest = f'-DGDN_SOURCE_DIGEST="{source_digest(extra_flags)}"'
    cmd = [HIPCC, *FLAGS, *extra_flags, digest, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
