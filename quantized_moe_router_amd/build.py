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
LIB_TIMELINE = os.path.join(HERE, "libqmoe_timeline.so")   # profiling build (phase timestamps)
SOURCES = ["qmoe.hip"]
HEADERS = ["common.h", "bounds.h", "store.h", "router.h", "router_mf.h", "ffn.h", "mfma.h", "decode.h",
           "cache.h", "diag.h"]
HOST_CHECKS_SRC = os.path.join(ROOT, "tests", "csrc", "host_checks.cpp")
HOST_CHECKS = os.path.join(ROOT, "_build", "host_checks")


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


def build(verbose=False, timeline=False):
    """Compile libqmoe.so (or, with timeline, the profiling build libqmoe_timeline.so: the same
    sources with QMOE_TIMELINE defined)."""
    out = LIB_TIMELINE if timeline else LIB
    extra = ["-DQMOE_TIMELINE"] if timeline else []
    cmd = [hipcc()] + flags() + extra + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + errs)
    os.replace(out + ".tmp", out)
    return out


def build_host_checks(verbose=False):
    """Compile the CPU debug build of the host code: tests/csrc/host_checks.cpp, which includes
    the library source, with QMOE_DEBUG_BOUNDS (bounds assertions) and the address and
    undefined-behaviour sanitizers on the host side.  Returns the executable's path."""
    os.makedirs(os.path.dirname(HOST_CHECKS), exist_ok=True)
    cmd = [hipcc(), "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
           "-DQMOE_DEBUG_BOUNDS",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", INCLUDE, "-I", CSRC, HOST_CHECKS_SRC, "-o", HOST_CHECKS + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(HOST_CHECKS + ".tmp", HOST_CHECKS)
    return HOST_CHECKS


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build(verbose="-v" in sys.argv, timeline=True))
