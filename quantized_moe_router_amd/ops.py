"""Torch-facing wrappers of the qmoe C ABI.

Argument marshalling only: every step of the layer runs in the HIP library.  torch supplies
device memory and the current HIP stream.  bf16 data may be passed as torch.bfloat16 or as
any 2-byte integer tensor holding bf16 bit patterns.
"""
import ctypes

import torch

from ._lib import Dims, Layer, Router, check, lib, make_dims  # noqa: F401


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t, dtype_bytes=None, what="tensor", allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{what} must not be None")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype_bytes is not None and t.element_size() != dtype_bytes:
        raise ValueError(f"{what} must have {dtype_bytes}-byte elements (got {t.dtype})")
    return ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, what):
    if t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype} (got {t.dtype})")


def expert_stride(dims, inter):
    return int(lib().qmoe_expert_stride(ctypes.byref(dims), int(inter)))


def workspace_bytes(dims, max_tokens):
    return int(lib().qmoe_workspace_bytes(ctypes.byref(dims), int(max_tokens)))


def workspace(dims, max_tokens, device="cuda"):
    """A zero-initialised workspace tensor for calls of up to max_tokens tokens."""
    n = workspace_bytes(dims, max_tokens)
    if n == 0:
        check(-2)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    check(lib().qmoe_workspace_init(_ptr(ws), n, _stream()))
    return ws


def pack_expert(dims, inter, gate_q, gate_s, gate_b, up_q, up_s, up_b, down_q, down_s, down_b, dst):
    for t, n in ((gate_q, "gate_q"), (up_q, "up_q"), (down_q, "down_q")):
        _need(t, torch.uint8, n)
    check(lib().qmoe_pack_expert(
        ctypes.byref(dims), int(inter), _ptr(gate_q, 1), _ptr(gate_s, 2), _ptr(gate_b, 2),
        _ptr(up_q, 1), _ptr(up_s, 2), _ptr(up_b, 2), _ptr(down_q, 1), _ptr(down_s, 2),
        _ptr(down_b, 2), _ptr(dst, 1, "dst"), _stream()))


def unpack_expert(dims, inter, src, gate_q, gate_s, gate_b, up_q, up_s, up_b, down_q, down_s, down_b):
    check(lib().qmoe_unpack_expert(
        ctypes.byref(dims), int(inter), _ptr(src, 1, "src"), _ptr(gate_q, 1), _ptr(gate_s, 2),
        _ptr(gate_b, 2), _ptr(up_q, 1), _ptr(up_s, 2), _ptr(up_b, 2), _ptr(down_q, 1),
        _ptr(down_s, 2), _ptr(down_b, 2), _stream()))


class RouterWeights:
    """Device tensors of one layer's router (kept alive with the ctypes struct)."""

    def __init__(self, codes, scales, biases, per_expert_scale, router_scale=None, logit_bias=None):
        _need(codes, torch.uint8, "router codes")
        _need(per_expert_scale, torch.float32, "per_expert_scale")
        self.tensors = (codes, scales, biases, per_expert_scale, router_scale, logit_bias)
        self.struct = Router(
            _ptr(codes, 1).value, _ptr(scales, 2).value, _ptr(biases, 2).value,
            _ptr(router_scale, 4, allow_none=True).value if router_scale is not None else None,
            _ptr(per_expert_scale, 4).value,
            _ptr(logit_bias, 4, allow_none=True).value if logit_bias is not None else None)


class LayerWeights:
    """A layer: router + packed expert store (+ shared block)."""

    def __init__(self, dims, router, experts, stride, shared=None, experts_offset=0,
                 post_norm_gain=None, layer_scalar=None):
        self.dims, self.router, self.experts, self.shared = dims, router, experts, shared
        if post_norm_gain is not None:
            _need(post_norm_gain, torch.float32, "post_norm_gain")
        if layer_scalar is not None:
            _need(layer_scalar, torch.float32, "layer_scalar")
        self.post = (post_norm_gain, layer_scalar)
        base = _ptr(experts, 1, "experts").value + int(experts_offset)
        self.struct = Layer(dims, router.struct, base, int(stride),
                            _ptr(shared, 1, "shared").value if shared is not None else None,
                            _ptr(post_norm_gain, 4).value if post_norm_gain is not None else None,
                            _ptr(layer_scalar, 4).value if layer_scalar is not None else None)


def router_topk(dims, router, x, ws, topk_idx=None, topk_w=None, logits=None):
    T = x.shape[0]
    k = dims.top_k
    if topk_idx is None:
        topk_idx = torch.empty(T, k, dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty(T, k, dtype=torch.float32, device=x.device)
    _need(topk_idx, torch.int32, "topk_idx")
    _need(topk_w, torch.float32, "topk_w")
    check(lib().qmoe_router_topk(
        ctypes.byref(dims), ctypes.byref(router.struct), _ptr(x, 2, "x"), T, _ptr(topk_idx, 4),
        _ptr(topk_w, 4), _ptr(logits, 4, allow_none=True), _ptr(ws, 1, "ws"), ws.numel(), _stream()))
    return topk_idx, topk_w


def bucket(dims, topk_idx, ws=None):
    T = topk_idx.shape[0]
    E = dims.n_experts
    dev = topk_idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    srt = torch.empty(max(T * dims.top_k, 1), dtype=torch.int32, device=dev)
    active = torch.empty(E, dtype=torch.int32, device=dev)
    n_active = torch.empty(1, dtype=torch.int32, device=dev)
    _need(topk_idx, torch.int32, "topk_idx")
    check(lib().qmoe_bucket(
        ctypes.byref(dims), _ptr(topk_idx, 4), T, _ptr(counts), _ptr(offsets), _ptr(srt),
        _ptr(active), _ptr(n_active), _ptr(ws, 1, allow_none=True),
        0 if ws is None else ws.numel(), _stream()))
    return counts, offsets, srt[:T * dims.top_k], active, n_active


def expert_ffn(layer, x, offsets, srt, active, n_active, ws, y=None, y_shared=None, want_shared=True):
    T = x.shape[0]
    d = layer.dims
    if y is None:
        y = torch.empty(T * d.top_k, d.hidden, dtype=torch.float32, device=x.device)
    if y_shared is None and want_shared and layer.shared is not None:
        y_shared = torch.empty(T, d.hidden, dtype=torch.float32, device=x.device)
    check(lib().qmoe_expert_ffn(
        ctypes.byref(layer.struct), _ptr(x, 2, "x"), T, _ptr(offsets, 4), _ptr(srt, 4),
        _ptr(active, 4), _ptr(n_active, 4), _ptr(y, 4, "y"), _ptr(y_shared, 4, allow_none=True),
        _ptr(ws, 1, "ws"), ws.numel(), _stream()))
    return y, y_shared


def combine(dims, x, y, topk_w, y_shared=None, out=None, out_f32=None):
    T = x.shape[0]
    if out is None:
        out = torch.empty(T, dims.hidden, dtype=torch.bfloat16, device=x.device)
    check(lib().qmoe_combine(
        ctypes.byref(dims), _ptr(x, 2, "x"), _ptr(y, 4, "y"), _ptr(topk_w, 4, "topk_w"),
        _ptr(y_shared, 4, allow_none=True), T, _ptr(out, 2, "out"),
        _ptr(out_f32, 4, allow_none=True), _stream()))
    return out


def combine_post(dims, x, y, topk_w, y_shared=None, post_norm_gain=None, layer_scalar=None,
                 out=None, out_f32=None):
    T = x.shape[0]
    if out is None:
        out = torch.empty(T, dims.hidden, dtype=torch.bfloat16, device=x.device)
    check(lib().qmoe_combine_post(
        ctypes.byref(dims), _ptr(x, 2, "x"), _ptr(y, 4, "y"), _ptr(topk_w, 4, "topk_w"),
        _ptr(y_shared, 4, allow_none=True), _ptr(post_norm_gain, 4, allow_none=True),
        _ptr(layer_scalar, 4, allow_none=True), T, _ptr(out, 2, "out"),
        _ptr(out_f32, 4, allow_none=True), _stream()))
    return out


def layer_forward(layer, x, ws, out=None, out_f32=None, topk_idx=None, topk_w=None):
    T = x.shape[0]
    d = layer.dims
    if out is None:
        out = torch.empty(T, d.hidden, dtype=torch.bfloat16, device=x.device)
    check(lib().qmoe_layer_forward(
        ctypes.byref(layer.struct), _ptr(x, 2, "x"), T, _ptr(out, 2, "out"),
        _ptr(out_f32, 4, allow_none=True), _ptr(topk_idx, 4, allow_none=True),
        _ptr(topk_w, 4, allow_none=True), _ptr(ws, 1, "ws"), ws.numel(), _stream()))
    return out


def layer_forward_noalloc(layer, x, out, out_f32=None, topk_idx=None, topk_w=None):
    """The layer on the library's own per-device scratch (qmoe_layer_forward_noalloc): no
    workspace; every output is the caller's, nothing is allocated."""
    T = x.shape[0]
    check(lib().qmoe_layer_forward_noalloc(
        ctypes.byref(layer.struct), _ptr(x, 2, "x"), T, _ptr(out, 2, "out"),
        _ptr(out_f32, 4, allow_none=True), _ptr(topk_idx, 4, allow_none=True),
        _ptr(topk_w, 4, allow_none=True), _stream()))
    return out


def decode_stack(layers, x, ws, out=None, out_f32=None, topk_idx=None, topk_w=None):
    """One token through the chained layers in one launch: x [1, H] (or [H]) bf16; returns
    out [n_layers, H] bf16, every layer's output (the last row is the chain's result)."""
    n = len(layers)
    d = layers[0].dims if n else None
    if out is None:
        out = torch.empty(max(n, 1), d.hidden if d else 1, dtype=torch.bfloat16, device=x.device)
    arr = (Layer * max(n, 1))(*[l.struct for l in layers])
    check(lib().qmoe_decode_stack(
        arr, n, _ptr(x, 2, "x"), _ptr(out, 2, "out"), _ptr(out_f32, 4, allow_none=True),
        _ptr(topk_idx, 4, allow_none=True), _ptr(topk_w, 4, allow_none=True), _ptr(ws, 1, "ws"),
        ws.numel(), _stream()))
    return out


class ExpertCache:
    """Tiered residency: routed expert blocks in host memory (`host_store`, a CPU uint8 tensor,
    pinned for full copy speed), `slots` of them cached in the device tensor `slot_store`."""

    def __init__(self, dims, host_store, host_stride, slot_store, slot_stride, slots):
        if not isinstance(host_store, torch.Tensor) or host_store.device.type != "cpu":
            raise ValueError("host_store must be a CPU tensor")
        if not host_store.is_contiguous():
            raise ValueError("host_store must be contiguous")
        self.keep = (host_store, slot_store)
        self.dims = dims
        h = ctypes.c_void_p()
        check(lib().qmoe_cache_create(ctypes.byref(dims), ctypes.c_void_p(host_store.data_ptr()),
                                      int(host_stride), _ptr(slot_store, 1, "slot_store"),
                                      int(slot_stride), int(slots), ctypes.byref(h)))
        self.h = h

    def plan(self, ids):
        """Host-only slot decision for the expert ids of one call: (slot of every id, list of
        (expert, slot) blocks to copy)."""
        import numpy as np
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        n = ids.size
        slot_of = np.empty(max(n, 1), np.int32)
        fe = np.empty(max(n, 1), np.int32)
        fs = np.empty(max(n, 1), np.int32)
        nf = ctypes.c_int32()
        check(lib().qmoe_cache_plan(self.h, ids.ctypes.data, n, slot_of.ctypes.data, fe.ctypes.data,
                                    fs.ctypes.data, ctypes.byref(nf)))
        return slot_of[:n], list(zip(fe[:nf.value].tolist(), fs[:nf.value].tolist()))

    def stats(self):
        h, m = ctypes.c_int64(), ctypes.c_int64()
        check(lib().qmoe_cache_stats(self.h, ctypes.byref(h), ctypes.byref(m)))
        return h.value, m.value

    def __del__(self):
        try:
            if self.h:
                lib().qmoe_cache_destroy(self.h)
        except Exception:
            pass


def layer_forward_tiered(layer, cache, x, ws, out=None, out_f32=None, topk_idx=None, topk_w=None):
    T = x.shape[0]
    d = layer.dims
    if out is None:
        out = torch.empty(T, d.hidden, dtype=torch.bfloat16, device=x.device)
    check(lib().qmoe_layer_forward_tiered(
        ctypes.byref(layer.struct), cache.h, _ptr(x, 2, "x"), T, _ptr(out, 2, "out"),
        _ptr(out_f32, 4, allow_none=True), _ptr(topk_idx, 4, allow_none=True),
        _ptr(topk_w, 4, allow_none=True), _ptr(ws, 1, "ws"), ws.numel(), _stream()))
    return out


class Event:
    """A HIP event created by the library (for timing kernels on the stream they run on)."""

    def __init__(self):
        h = ctypes.c_void_p()
        check(lib().qmoe_event_create(ctypes.byref(h)))
        self.h = h

    def record(self):
        check(lib().qmoe_event_record(self.h, _stream()))

    def elapsed_ms(self, stop):
        ms = ctypes.c_float()
        check(lib().qmoe_event_elapsed_ms(self.h, stop.h, ctypes.byref(ms)))
        return ms.value

    def __del__(self):
        try:
            if self.h:
                lib().qmoe_event_destroy(self.h)
        except Exception:
            pass


def set_profile_events(start, stop):
    check(lib().qmoe_set_profile_events(start.h if start else None, stop.h if stop else None))


def workspace_status(ws):
    """0 when no one-token layer call on this workspace gave up waiting (synchronises)."""
    v = ctypes.c_int32()
    check(lib().qmoe_workspace_status(_ptr(ws, 1, "ws"), ws.numel(), ctypes.byref(v), _stream()))
    return v.value


def timeline_set(buf):
    """Profiling build only (QMOE_LIBRARY=timeline): device tensor of 8 int64 words per
    workgroup that the next one-token layer calls on this thread write their phase timestamps
    to (None: stop)."""
    L = lib()
    from . import _lib as _L
    if not hasattr(L, "qmoe_timeline_set") or not _L.TIMELINE:
        raise RuntimeError("timeline_set needs the profiling build (QMOE_LIBRARY=timeline)")
    check(L.qmoe_timeline_set(None if buf is None else ctypes.c_void_p(buf.data_ptr())))


def read_blocks(base, stride, ids, nbytes, sink):
    """Plain streaming read of the first nbytes of blocks base + ids[i] * stride (measurement
    reference); sink: int32 device tensor of at least len(ids) * ceil(nbytes / 16384) words."""
    n = len(ids)
    waves = n * ((nbytes + 16383) // 16384)
    if sink.numel() < waves or sink.element_size() != 4:
        raise ValueError("sink too small")
    if n and (max(ids) + 1) * stride - stride + nbytes > base.numel() * base.element_size():
        raise ValueError("a block lies outside the buffer")
    arr = (ctypes.c_int32 * max(n, 1))(*ids)
    check(lib().qmoe_read_blocks(ctypes.c_void_p(base.data_ptr()), stride, arr, n, nbytes,
                                 ctypes.c_void_p(sink.data_ptr()), _stream()))
