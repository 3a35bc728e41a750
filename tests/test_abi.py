"""The C ABI on the CPU: the library loads, exports every declared entry point, answers
host-only queries, and rejects bad arguments with a status and message before touching the
device (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from quantized_moe_router_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libqmoe.so not built")
    return _lib


def declared():
    txt = open(os.path.join(ROOT, "include", "qmoe.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(qmoe_[a-z_0-9]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    L = _lib()
    names = declared()
    assert len(names) >= 17
    for n in names:
        assert hasattr(L.lib(), n), n
    assert sorted(L.EXPORTS) == names


def test_version_and_last_error():
    L = _lib()
    assert L.lib().qmoe_version() == 200
    assert isinstance(L.last_error(), str)


def test_stride_and_workspace_queries():
    L = _lib()
    d = L.make_dims(2816, 128, 8, 704, 2112)
    lib = L.lib()
    assert lib.qmoe_expert_stride(ctypes.byref(d), 704) == 3346432
    assert lib.qmoe_expert_stride(ctypes.byref(d), 2112) == 10039296     # 10,036,224 -> 4 KiB
    d2 = L.make_dims(2048, 512, 10, 512, 512)
    assert lib.qmoe_expert_stride(ctypes.byref(d2), 512) == 1769472     # already a 4 KiB multiple
    assert lib.qmoe_workspace_bytes(ctypes.byref(d), 128) > lib.qmoe_workspace_bytes(ctypes.byref(d), 1) > 0
    # 8-bit experts: two 4-bit k-steps per group, 6,690,816 B -> 4 KiB multiple
    d8 = L.make_dims(2816, 128, 8, 704, 2112, expert_bits=8)
    assert lib.qmoe_expert_stride(ctypes.byref(d8), 704) == 6692864


@pytest.mark.parametrize("field,value", [("group", 32), ("hidden", 100), ("hidden", 16384),
                                         ("inter", 0), ("inter", 8192), ("n_experts", 0),
                                         ("n_experts", 2048), ("top_k", 0), ("top_k", 33),
                                         ("shared_inter", 65), ("expert_bits", 5),
                                         ("expert_bits", 16)])
def test_bad_dims_are_rejected(field, value):
    L = _lib()
    d = L.make_dims(256, 16, 2, 128, 128)
    setattr(d, field, value)
    if field == "top_k" and value == 33:
        d.n_experts = 64
    lib = L.lib()
    assert lib.qmoe_expert_stride(ctypes.byref(d), 128) == 0
    assert lib.qmoe_workspace_bytes(ctypes.byref(d), 4) == 0
    assert L.last_error()
    fake = ctypes.c_void_p(4096)
    r = L.Router(4096, 4096, 4096, None, 4096, None)
    rc = lib.qmoe_router_topk(ctypes.byref(d), ctypes.byref(r), fake, 4, fake, fake, None, fake,
                              1 << 30, None)
    assert rc == -2 and field in L.last_error().replace("top_k", "top_k n_experts") or rc == -2


def test_argument_errors_do_not_touch_the_device():
    L = _lib()
    lib = L.lib()
    d = L.make_dims(256, 16, 2, 128, 128)
    fake = ctypes.c_void_p(4096)
    r = L.Router(4096, 4096, 4096, None, 4096, None)
    # null router field
    rbad = L.Router(4096, None, 4096, None, 4096, None)
    assert lib.qmoe_router_topk(ctypes.byref(d), ctypes.byref(rbad), fake, 4, fake, fake, None,
                                fake, 1 << 30, None) == -1
    # negative token count
    assert lib.qmoe_router_topk(ctypes.byref(d), ctypes.byref(r), fake, -1, fake, fake, None,
                                fake, 1 << 30, None) == -2
    # workspace too small / null / misaligned
    assert lib.qmoe_router_topk(ctypes.byref(d), ctypes.byref(r), fake, 4, fake, fake, None,
                                fake, 16, None) == -3
    assert "workspace" in L.last_error()
    assert lib.qmoe_router_topk(ctypes.byref(d), ctypes.byref(r), fake, 4, fake, fake, None,
                                None, 1 << 30, None) == -3
    assert lib.qmoe_router_topk(ctypes.byref(d), ctypes.byref(r), fake, 4, fake, fake, None,
                                ctypes.c_void_p(4100), 1 << 30, None) == -3
    # T = 0 is a no-op
    assert lib.qmoe_router_topk(ctypes.byref(d), ctypes.byref(r), fake, 0, fake, fake, None,
                                None, 0, None) == 0
    # x and the router codes are read with 16-byte loads
    odd = ctypes.c_void_p(4100)
    assert lib.qmoe_router_topk(ctypes.byref(d), ctypes.byref(r), odd, 4, fake, fake, None,
                                fake, 1 << 30, None) == -1
    assert "aligned" in L.last_error()
    rodd = L.Router(4100, 4096, 4096, None, 4096, None)
    assert lib.qmoe_router_topk(ctypes.byref(d), ctypes.byref(rodd), fake, 4, fake, fake, None,
                                fake, 1 << 30, None) == -1
    assert "codes" in L.last_error()
    # layer checks
    lay = L.Layer(d, r, 4096, 4096, None)
    assert lib.qmoe_layer_forward(ctypes.byref(lay), fake, 4, fake, None, None, None, fake,
                                  1 << 30, None) == -1          # stride smaller than a block
    lay = L.Layer(d, r, 4100, 65536, None)
    assert lib.qmoe_layer_forward(ctypes.byref(lay), fake, 4, fake, None, None, None, fake,
                                  1 << 30, None) == -1          # misaligned store
    lay = L.Layer(d, r, 4096, 65536, None)
    assert lib.qmoe_layer_forward(ctypes.byref(lay), None, 4, fake, None, None, None, fake,
                                  1 << 30, None) == -1          # null x
    assert lib.qmoe_layer_forward(ctypes.byref(lay), odd, 4, fake, None, None, None, fake,
                                  1 << 30, None) == -1          # misaligned x
    assert lib.qmoe_layer_forward(ctypes.byref(lay), None, 0, None, None, None, None, None,
                                  0, None) == 0                 # T = 0: pointers unused
    d0 = L.make_dims(256, 16, 2, 128, 0)
    lay = L.Layer(d0, r, 4096, 65536, 8192)
    assert lib.qmoe_layer_forward(ctypes.byref(lay), fake, 4, fake, None, None, None, fake,
                                  1 << 30, None) == -1          # shared block without width
    # pack: null pointer and bad inter
    assert lib.qmoe_pack_expert(ctypes.byref(d), 128, *([fake] * 8), None, fake, None) == -1
    assert lib.qmoe_pack_expert(ctypes.byref(d), 96, *([fake] * 9), fake, None) == -2
    # combine / bucket nulls
    assert lib.qmoe_combine(ctypes.byref(d), fake, None, fake, None, 4, fake, None, None) == -1
    assert lib.qmoe_combine_post(ctypes.byref(d), fake, None, fake, None, None, None, 4, fake,
                                 None, None) == -1
    assert lib.qmoe_combine_post(ctypes.byref(d), fake, fake, fake, None, ctypes.c_void_p(4100), None, 4, fake,
                                 None, None) == -1              # misaligned gain
    lay = L.Layer(d, r, 4096, 65536, None, 4104, None)
    assert lib.qmoe_layer_forward(ctypes.byref(lay), fake, 4, fake, None, None, None, fake,
                                  1 << 30, None) == -1          # misaligned post-norm gain
    assert lib.qmoe_bucket(ctypes.byref(d), None, 4, fake, fake, fake, fake, fake, None, 0, None) == -1
    # chained one-token layers
    lays = (L.Layer * 2)(L.Layer(d, r, 4096, 65536, None), L.Layer(d, r, 4096, 65536, None))
    assert lib.qmoe_decode_stack(None, 2, fake, fake, None, None, None, fake, 1 << 30, None) == -1
    assert lib.qmoe_decode_stack(lays, 65, fake, fake, None, None, None, fake, 1 << 30, None) == -2
    assert lib.qmoe_decode_stack(lays, -1, fake, fake, None, None, None, fake, 1 << 30, None) == -2
    assert lib.qmoe_decode_stack(lays, 0, None, None, None, None, None, None, 0, None) == 0
    assert lib.qmoe_decode_stack(lays, 2, None, fake, None, None, None, fake, 1 << 30, None) == -1
    assert lib.qmoe_decode_stack(lays, 2, fake, fake, None, fake, None, fake, 1 << 30,
                                 None) == -1                    # one of the two top-k outputs
    assert lib.qmoe_decode_stack(lays, 2, fake, fake, None, None, None, fake, 16, None) == -3
    d2 = L.make_dims(256, 16, 2, 192, 128)
    lays[1] = L.Layer(d2, r, 4096, 1 << 20, None)
    assert lib.qmoe_decode_stack(lays, 2, fake, fake, None, None, None, fake, 1 << 30,
                                 None) == -2                    # dims differ
    assert "differ" in L.last_error()
    lays[1] = L.Layer(d, r, 4096, 65536, 8192)
    assert lib.qmoe_decode_stack(lays, 2, fake, fake, None, None, None, fake, 1 << 30,
                                 None) == -1                    # shared block in one layer only
    assert L.MAX_STACK == 64
    # events
    assert lib.qmoe_set_profile_events(None, None) == 0       # profiling off
    assert lib.qmoe_event_create(None) == -1


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    """The allocation-free entry point refuses, before any device call, a shape whose workspace
    would exceed its fixed scratch (here hidden 8192, 1024 experts, top-32, width 4096)."""
    L = _lib()
    d = L.make_dims(8192, 1024, 32, 4096, 0)
    lay = L.Layer()
    lay.d = d
    fake = ctypes.c_void_p(1 << 20)       # never dereferenced: the call fails first
    lay.r = L.Router(fake, fake, fake, None, fake, None)
    lay.experts = fake
    lay.expert_stride = L.lib().qmoe_expert_stride(ctypes.byref(d), 4096)
    rc = L.lib().qmoe_layer_forward_noalloc(ctypes.byref(lay), fake, 128, fake, None, None, None,
                                            None)
    assert rc == -3, L.last_error()
    assert "scratch" in L.last_error()
