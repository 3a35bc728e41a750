"""Host-side tiered-residency cache policy (LFU with recency, the pages' expert cache) against
a plain Python model of the same rule.  CPU only: the cache keeps the store pointers and
touches no device memory until a forward call."""
import ctypes

import numpy as np
import pytest

from cache_model import Model


def _lib():
    from quantized_moe_router_amd import _lib as L
    try:
        L.lib()
    except RuntimeError as e:
        pytest.skip(str(e))
    return L


def _cache(L, E, k, S):
    d = L.make_dims(256, E, k, 128, 0)
    h = ctypes.c_void_p()
    stride = L.lib().qmoe_expert_stride(ctypes.byref(d), 128)
    rc = L.lib().qmoe_cache_create(ctypes.byref(d), ctypes.c_void_p(4096), stride,
                                   ctypes.c_void_p(1 << 20), stride, S, ctypes.byref(h))
    assert rc == 0
    return h


def _plan(L, h, ids):
    ids = np.ascontiguousarray(ids, np.int32)
    n = ids.size
    so, fe, fs = (np.empty(max(n, 1), np.int32) for _ in range(3))
    nf = ctypes.c_int32()
    rc = L.lib().qmoe_cache_plan(h, ids.ctypes.data, n, so.ctypes.data, fe.ctypes.data,
                                 fs.ctypes.data, ctypes.byref(nf))
    return rc, so[:n].tolist(), list(zip(fe[:nf.value].tolist(), fs[:nf.value].tolist()))


@pytest.mark.parametrize("E,k,S,calls,tokens", [(16, 2, 4, 200, 1), (128, 8, 16, 300, 1),
                                                (64, 4, 32, 60, 6), (16, 2, 16, 20, 3)])
def test_cache_plan_matches_model(E, k, S, calls, tokens):
    L = _lib()
    h = _cache(L, E, k, S)
    m = Model(E, S)
    rng = np.random.default_rng(E * 7 + S)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    for _ in range(calls):
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(tokens)]).ravel()
        if len(set(ids.tolist())) > S:
            continue
        rc, so, fills = _plan(L, h, ids)
        want_so, want_fills = m.plan(ids)
        assert rc == 0 and so == want_so and fills == want_fills
    hits, misses = ctypes.c_int64(), ctypes.c_int64()
    assert L.lib().qmoe_cache_stats(h, ctypes.byref(hits), ctypes.byref(misses)) == 0
    assert (hits.value, misses.value) == (m.hits, m.misses)
    assert m.hits > 0 and m.misses >= S
    L.lib().qmoe_cache_destroy(h)


def test_cache_rejects_bad_calls():
    L = _lib()
    h = _cache(L, 16, 2, 4)
    assert _plan(L, h, [1, 2, 3, 4, 5])[0] == -1          # five distinct ids, four slots
    assert _plan(L, h, [16, 0])[0] == -1                  # id out of range
    assert _plan(L, h, [3, 3, 3])[0] == 0                 # repeats count once
    d = L.make_dims(256, 16, 2, 128, 0)
    out = ctypes.c_void_p()
    stride = L.lib().qmoe_expert_stride(ctypes.byref(d), 128)
    assert L.lib().qmoe_cache_create(ctypes.byref(d), ctypes.c_void_p(4096), stride,
                                     ctypes.c_void_p(1 << 20), stride, 1, ctypes.byref(out)) == -2
    assert L.lib().qmoe_cache_create(ctypes.byref(d), ctypes.c_void_p(4096), stride - 256,
                                     ctypes.c_void_p(1 << 20), stride, 4, ctypes.byref(out)) == -1
    L.lib().qmoe_cache_destroy(h)
