"""Build libca.so (HIP kernels + C ABI) for gfx950 in-tree with hipcc.

    python -m long_context_core_amd.build          # or build() from Python

Every source is compiled on every call (no up-to-date check), objects go to
long_context_core_amd/_build/, the library to long_context_core_amd/libca.so.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libca.so")
ROOT = os.path.dirname(PKG)

SOURCES = ["ca_api.cpp", "ca_sched.cpp", "ca_ring.cpp", "ca_fwd.hip", "ca_merge.hip", "ca_decode.hip", "ca_bwd.hip",
           "ca_noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # no packed fp32 ALU ops (v_pk_{add,mul,fma}_f32) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in the VGPR form: with the AGPR form the register
    # allocator shuttles loop-carried accumulators between AGPRs and VGPRs
    # every iteration (hundreds of v_accvgpr moves per tile in the backward)
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libca.so)")


# Kernel sources only (.hip): inputs are finite by contract and the kernels
# use -inf but never NaN; without this, every fmaxf on an MFMA result is
# preceded by a canonicalising v_max (IEEE mode), tripling the cost of row
# maxima.  Host sources (.cpp) keep IEEE NaN semantics for argument checks.
KERNEL_ONLY_FLAGS = ["-fno-honor-nans"]


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    kflags = KERNEL_ONLY_FLAGS if src.endswith(".hip") else []
    cmd = [hipcc()] + HIPCC_FLAGS + kflags + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("compiling %s failed:\n%s" % (src, msgs))
    return obj, msgs


def build(verbose=False, extra_flags=()):
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra_flags)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    for obj, msgs in results:
        if verbose and msgs.strip():
            print(msgs)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libca.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
