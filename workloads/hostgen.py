"""The seeded synthetic draw and quantiser of gen.py in C on the host (libqmoe_hostgen.so).

Same values as the numpy functions gen.normal_f32 and gen.quantize_groups, bit for bit
(tests/test_workloads.py), only fast enough to draw the experts of full-size layers on the
CPU.  Built with gcc (no GPU involved); gen.py falls back to numpy when it is not built.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmoe_hostgen.so")
SRC = os.path.join(_HERE, "csrc", "qmoe_hostgen.c")
_lib = None


def build():
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           SRC, "-o", LIB_PATH + ".tmp", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed for the host input generator:\n" + r.stderr)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    """The loaded library, or None if it is not built."""
    global _lib
    if _lib is None and os.path.exists(LIB_PATH):
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.qmoe_host_normal.restype = ctypes.c_int
        L.qmoe_host_normal.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64,
                                       ctypes.c_double, P]
        L.qmoe_host_matrix.restype = ctypes.c_int
        L.qmoe_host_matrix.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_double, ctypes.c_int, P, P, P]
        _lib = L
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def normal_f32(k0, k1, n, std):
    out = np.empty(n, np.float32)
    if lib().qmoe_host_normal(k0 & 0xFFFFFFFF, k1 & 0xFFFFFFFF, n, float(std), _ptr(out)):
        raise ValueError("qmoe_host_normal: bad arguments")
    return out


def matrix(k0, k1, rows, cols, std, bits):
    """(codes, scale bits, bias bits) of a drawn, quantised [rows, cols] matrix; codes packed
    two per byte for 4 bits."""
    q = np.empty((rows, cols // 2 if bits == 4 else cols), np.uint8)
    s = np.empty((rows, cols // 64), np.uint16)
    b = np.empty((rows, cols // 64), np.uint16)
    if lib().qmoe_host_matrix(k0 & 0xFFFFFFFF, k1 & 0xFFFFFFFF, rows, cols, float(std), bits,
                              _ptr(q), _ptr(s), _ptr(b)):
        raise ValueError("qmoe_host_matrix: bad arguments")
    return q, s, b
