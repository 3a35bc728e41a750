"""ctypes binding of libqmoe.so (the C ABI declared in include/qmoe.h).

Loading fails loudly when the library has not been built: there is no fallback path.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# QMOE_LIBRARY=timeline loads the profiling build (same kernels, plus phase timestamps of the
# one-token layer, see qmoe_timeline_set); the default is the product library.
TIMELINE = os.environ.get("QMOE_LIBRARY", "") == "timeline"
LIB_PATH = os.path.join(_HERE, "libqmoe_timeline.so" if TIMELINE else "libqmoe.so")

QMOE_OK = 0
ERRORS = {-1: "QMOE_ERR_ARG", -2: "QMOE_ERR_SHAPE", -3: "QMOE_ERR_WORKSPACE",
          -4: "QMOE_ERR_ARCH", -5: "QMOE_ERR_HIP"}

EXPORTS = [
    "qmoe_version", "qmoe_last_error", "qmoe_expert_stride", "qmoe_workspace_bytes",
    "qmoe_workspace_init", "qmoe_pack_expert", "qmoe_unpack_expert", "qmoe_router_topk",
    "qmoe_bucket", "qmoe_expert_ffn", "qmoe_combine", "qmoe_combine_post", "qmoe_layer_forward",
    "qmoe_event_create", "qmoe_event_destroy", "qmoe_event_record", "qmoe_event_elapsed_ms",
    "qmoe_set_profile_events", "qmoe_workspace_status", "qmoe_cache_create", "qmoe_cache_destroy",
    "qmoe_cache_plan", "qmoe_cache_stats", "qmoe_layer_forward_tiered", "qmoe_decode_stack",
    "qmoe_read_blocks", "qmoe_layer_forward_noalloc",
]
MAX_STACK = 64


class QmoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("group", ctypes.c_int32),
                ("expert_bits", ctypes.c_int32)]


class Router(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p), ("router_scale", ctypes.c_void_p),
                ("per_expert_scale", ctypes.c_void_p), ("logit_bias", ctypes.c_void_p)]


class Layer(ctypes.Structure):
    _fields_ = [("d", Dims), ("r", Router), ("experts", ctypes.c_void_p),
                ("expert_stride", ctypes.c_size_t), ("shared", ctypes.c_void_p),
                ("post_norm_gain", ctypes.c_void_p), ("layer_scalar", ctypes.c_void_p)]


_lib = None


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m quantized_moe_router_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I32 = ctypes.c_int32
    SZ = ctypes.c_size_t
    pd = ctypes.POINTER(Dims)
    sig = {
        "qmoe_version": (ctypes.c_int, []),
        "qmoe_last_error": (ctypes.c_char_p, []),
        "qmoe_expert_stride": (SZ, [pd, I32]),
        "qmoe_workspace_bytes": (SZ, [pd, I32]),
        "qmoe_workspace_init": (ctypes.c_int, [P, SZ, P]),
        "qmoe_pack_expert": (ctypes.c_int, [pd, I32] + [P] * 9 + [P, P]),
        "qmoe_unpack_expert": (ctypes.c_int, [pd, I32, P] + [P] * 9 + [P]),
        "qmoe_router_topk": (ctypes.c_int, [pd, ctypes.POINTER(Router), P, I32, P, P, P, P, SZ, P]),
        "qmoe_bucket": (ctypes.c_int, [pd, P, I32, P, P, P, P, P, P, SZ, P]),
        "qmoe_expert_ffn": (ctypes.c_int, [ctypes.POINTER(Layer), P, I32, P, P, P, P, P, P, P, SZ, P]),
        "qmoe_combine": (ctypes.c_int, [pd, P, P, P, P, I32, P, P, P]),
        "qmoe_combine_post": (ctypes.c_int, [pd, P, P, P, P, P, P, I32, P, P, P]),
        "qmoe_layer_forward": (ctypes.c_int, [ctypes.POINTER(Layer), P, I32, P, P, P, P, P, SZ, P]),
        "qmoe_event_create": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p)]),
        "qmoe_event_destroy": (ctypes.c_int, [P]),
        "qmoe_event_record": (ctypes.c_int, [P, P]),
        "qmoe_event_elapsed_ms": (ctypes.c_int, [P, P, ctypes.POINTER(ctypes.c_float)]),
        "qmoe_set_profile_events": (ctypes.c_int, [P, P]),
        "qmoe_workspace_status": (ctypes.c_int, [P, SZ, ctypes.POINTER(ctypes.c_int32), P]),
        "qmoe_cache_create": (ctypes.c_int, [pd, P, SZ, P, SZ, I32, ctypes.POINTER(ctypes.c_void_p)]),
        "qmoe_cache_destroy": (ctypes.c_int, [P]),
        "qmoe_cache_plan": (ctypes.c_int, [P, P, I32, P, P, P, ctypes.POINTER(ctypes.c_int32)]),
        "qmoe_cache_stats": (ctypes.c_int, [P, ctypes.POINTER(ctypes.c_int64),
                                            ctypes.POINTER(ctypes.c_int64)]),
        "qmoe_layer_forward_tiered": (ctypes.c_int, [ctypes.POINTER(Layer), P, P, I32, P, P, P, P, P,
                                                     SZ, P]),
        "qmoe_decode_stack": (ctypes.c_int, [ctypes.POINTER(Layer), I32, P, P, P, P, P, P, SZ, P]),
        "qmoe_read_blocks": (ctypes.c_int, [P, SZ, ctypes.POINTER(I32), I32, SZ, P, P]),
        "qmoe_layer_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(Layer), P, I32, P, P, P, P, P]),
    }
    if TIMELINE:
        sig["qmoe_timeline_set"] = (ctypes.c_int, [P])
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def last_error():
    return lib().qmoe_last_error().decode()


def check(rc):
    if rc != QMOE_OK:
        raise QmoeError(rc, last_error())
    return rc


def make_dims(hidden, n_experts, top_k, inter, shared_inter=0, group=64, expert_bits=4):
    return Dims(hidden, n_experts, top_k, inter, shared_inter, group, expert_bits)
