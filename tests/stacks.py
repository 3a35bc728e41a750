"""Synthetic layers on the device for tests and the benchmark.

Router tensors and hidden states are drawn on the host (workloads.gen); expert matrices are
drawn on the device (workloads.device, the same recipe bit for bit) and packed by the
library.  The host LayerInputs returned alongside re-draws any expert on the CPU for the
oracle, so no oracle input ever comes from the device.
"""
import numpy as np
import torch

from workloads import gen as G
from workloads import device as D
from quantized_moe_router_amd import ops
from quantized_moe_router_amd.store import PackedLayer
from quantized_moe_router_amd._lib import make_dims


def dims_of(cfg):
    return make_dims(cfg.hidden, cfg.experts, cfg.top_k, cfg.inter, cfg.shared_inter,
                     expert_bits=cfg.expert_bits)


def t16(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)


def router_weights(li, dev="cuda"):
    return ops.RouterWeights(
        torch.from_numpy(li.router_q).to(dev), t16(li.router_s, dev), t16(li.router_b, dev),
        torch.from_numpy(li.pes).to(dev),
        router_scale=torch.from_numpy(li.router_scale).to(dev),
        logit_bias=None if li.bias is None else torch.from_numpy(li.bias).to(dev))


def host_expert_tensors(ew, dev="cuda"):
    out = []
    for a in ew.arrays():
        out.append(torch.from_numpy(a).to(dev) if a.dtype == np.uint8 else t16(a, dev))
    return tuple(out)


def build_layer(cfg, layer, dev="cuda", gpu_gen=True, li=None):
    """(PackedLayer on the device, host LayerInputs for the oracle)."""
    li = G.make_router(cfg, layer) if li is None else li
    dims = dims_of(cfg)
    router = router_weights(li, dev)
    if gpu_gen:
        canon = D.CanonLayerExperts(cfg, layer, device=dev)
        sh = D.CanonShared(cfg, layer, device=dev) if cfg.shared_inter else None
        packed = PackedLayer.from_canonical(dims, router, canon.expert,
                                            sh.expert() if sh else None, device=dev)
        torch.cuda.synchronize()
        del canon, sh
    else:
        packed = PackedLayer.from_canonical(
            dims, router, lambda e: host_expert_tensors(li.expert(e), dev),
            host_expert_tensors(li.shared(), dev) if cfg.shared_inter else None, device=dev)
    return packed, li


def hidden(cfg, step, tokens=None, dev="cuda"):
    xb = G.make_hidden(cfg, step, tokens)
    return xb, t16(xb, dev)
