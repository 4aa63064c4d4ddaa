"""Build libdspark.so (HIP, gfx950) in-tree with hipcc.

Each ``csrc/*.hip`` translation unit is compiled to an object in parallel and
the objects are linked into ``libdspark.so`` next to this file.  The ABI unit is
compiled a second time with DSPARK_DEBUG_CHECKS and linked with the same kernel
objects into ``libdspark_debug.so`` (input and output scans around every call).
Both link the roctx library (one range per ABI call).  Packed-FP32 instructions
are disabled for device code (the flag is a device feature; the host pass prints
a harmless "not a recognized feature" warning).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdspark.so")
DEBUG_LIB = os.path.join(HERE, "libdspark_debug.so")
OBJDIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("DSPARK_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_LIB = "/opt/rocm/lib"
LINK_LIBS = [f"-L{ROCM_LIB}", "-lrocprofiler-sdk-roctx", f"-Wl,-rpath,{ROCM_LIB}"]
ABI_SOURCE = "dspark_abi.hip"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Per-source additions.  The persistent draft keeps each wave's Wt fragments in
# the accumulation registers (AGPRs) for the whole cycle; with the MFMA results
# in ordinary registers its epilogue reads them directly (no accumulator copies)
# and nothing spills.
SOURCE_FLAGS = {
    "k_persist.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device feature flag; drop that line only
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source and link libdspark.so and libdspark_debug.so;
    returns the path of the first."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJDIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[HIPCC, *CFLAGS, *SOURCE_FLAGS.get(os.path.basename(s), []), "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    abi = os.path.join(CSRC, ABI_SOURCE)
    debug_obj = os.path.join(OBJDIR, "dspark_abi_debug.o")
    cmds.append([HIPCC, *CFLAGS, "-DDSPARK_DEBUG_CHECKS", "-c", abi, "-o", debug_obj])
    with ThreadPoolExecutor(jobs or min(8, len(cmds))) as ex:
        for cmd, err in zip(cmds, ex.map(_run, cmds)):
            if verbose:
                print(" ".join(cmd[-3:]), file=sys.stderr)
                if err.strip():
                    print(err, file=sys.stderr)
    debug_objs = [debug_obj if os.path.basename(s) == ABI_SOURCE else o for s, o in zip(srcs, objs)]
    for lib, parts in ((LIB, objs), (DEBUG_LIB, debug_objs)):
        tmp = lib + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *parts, *LINK_LIBS])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
