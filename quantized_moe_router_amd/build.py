"""Build the HIP library libqmoe.so in-tree with hipcc for gfx950.

Usage: python -m quantized_moe_router_amd.build   (or build() from Python)
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqmoe.so")
SOURCES = ["qmoe.hip"]
HEADERS = ["common.h", "store.h", "router.h", "router_mf.h", "ffn.h", "mfma.h", "decode.h"]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 instructions are disabled for all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix-core accumulators stay in VGPRs: the prefill kernels scale them with VALU FMAs
        # between products, which would otherwise copy them out of and back into AGPRs
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-I", INCLUDE, "-I", CSRC,
        "-Wno-unused-result",
    ]


def build(verbose=False):
    cmd = [hipcc()] + flags() + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + errs)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
