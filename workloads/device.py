"""Draw the synthetic expert stacks directly on the GPU (same recipe as gen.py, bit for bit).

Only the routed and shared expert matrices are drawn on the device (they are gigabytes for
the large stacks); router tensors and hidden states come from gen.py on the host.
"""
import ctypes
import os
import subprocess

import numpy as np

from . import gen as G

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmoe_gen.so")
SRC = os.path.join(_HERE, "csrc", "qmoe_gen.hip")
_lib = None


def build():
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           SRC, "-o", LIB_PATH + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the input generator:\n" + r.stderr)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} missing: build it with workloads.device.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        for name in ("qmoe_gen_int4", "qmoe_gen_int8"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
                          ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_float, P, P, P, P]
        _lib = L
    return _lib


def gen_quant(bits, k0, tag0, tag_step, n_mat, rows, cols, std, q, s, b):
    """Draw n_mat quantised matrices into device tensors q (uint8: [n_mat, rows, cols/2] packed
    nibbles for 4 bits, [n_mat, rows, cols] for 8 bits) and s, b [n_mat, rows, cols/64]
    (2-byte elements)."""
    import torch
    assert bits in (4, 8)
    assert q.is_cuda and q.dtype == torch.uint8 and q.numel() == n_mat * rows * cols * bits // 8
    assert s.numel() == b.numel() == n_mat * rows * cols // 64
    c = float(np.float32(std / G.IH_STD))
    inv = float(np.float32(1.0 / ((1 << bits) - 1)))
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    f = lib().qmoe_gen_int8 if bits == 8 else lib().qmoe_gen_int4
    rc = f(k0 & 0xFFFFFFFF, tag0, tag_step, n_mat, rows, cols, c, inv,
           ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(s.data_ptr()),
           ctypes.c_void_p(b.data_ptr()), st)
    if rc != 0:
        raise RuntimeError(f"device generator failed ({rc})")


def gen_int4(k0, tag0, tag_step, n_mat, rows, cols, std, q, s, b):
    gen_quant(4, k0, tag0, tag_step, n_mat, rows, cols, std, q, s, b)


class CanonLayerExperts:
    """Canonical int4 arrays of every routed expert of one layer, on the device."""

    def __init__(self, cfg, layer, experts=None, device="cuda"):
        import torch
        E = cfg.experts if experts is None else experts
        H, I = cfg.hidden, cfg.inter
        k0 = G.layer_key(cfg, layer)
        u8, i16 = torch.uint8, torch.int16
        bits = cfg.expert_bits
        cpb = 8 // bits                         # codes per byte
        self.gate_q = torch.empty(E, I, H // cpb, dtype=u8, device=device)
        self.gate_s = torch.empty(E, I, H // 64, dtype=i16, device=device)
        self.gate_b = torch.empty_like(self.gate_s)
        self.up_q = torch.empty_like(self.gate_q)
        self.up_s = torch.empty_like(self.gate_s)
        self.up_b = torch.empty_like(self.gate_s)
        self.down_q = torch.empty(E, H, I // cpb, dtype=u8, device=device)
        self.down_s = torch.empty(E, H, I // 64, dtype=i16, device=device)
        self.down_b = torch.empty_like(self.down_s)
        for m, (q, s, b, rows, cols) in enumerate([
                (self.gate_q, self.gate_s, self.gate_b, I, H), (self.up_q, self.up_s, self.up_b, I, H),
                (self.down_q, self.down_s, self.down_b, H, I)]):
            gen_quant(bits, k0, G.Tag.expert(0, m), 3, E, rows, cols, cfg.weight_std, q, s, b)

    def expert(self, e):
        return (self.gate_q[e], self.gate_s[e], self.gate_b[e], self.up_q[e], self.up_s[e],
                self.up_b[e], self.down_q[e], self.down_s[e], self.down_b[e])


class CanonShared:
    def __init__(self, cfg, layer, device="cuda"):
        import torch
        H, I = cfg.hidden, cfg.shared_inter
        k0 = G.layer_key(cfg, layer)
        u8, i16 = torch.uint8, torch.int16
        self.arrays = []
        bits = cfg.expert_bits
        for m, (rows, cols) in enumerate([(I, H), (I, H), (H, I)]):
            q = torch.empty(rows, cols * bits // 8, dtype=u8, device=device)
            s = torch.empty(rows, cols // 64, dtype=i16, device=device)
            b = torch.empty_like(s)
            gen_quant(bits, k0, G.Tag.shared(m), 1, 1, rows, cols, cfg.weight_std, q, s, b)
            self.arrays += [q, s, b]

    def expert(self):
        return tuple(self.arrays)
