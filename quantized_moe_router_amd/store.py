"""Packed expert stores resident in HBM.

A layer's routed experts live in one device buffer of E fixed-stride blocks (the Swiftlet
article, section "같은 모델을 왜 이렇게 적은 메모리로 돌릴 수 있나": one fixed-stride block
per expert, so one read fetches one expert); the shared expert has its own block.  Packing is
done by the library's qmoe_pack_expert (layout change only).
"""
import torch

from . import ops
from ._lib import make_dims


class PackedLayer:
    """Router tensors + packed expert store of one layer, all on the device."""

    def __init__(self, dims, router, store, stride, shared=None):
        self.dims = dims
        self.router = router
        self.store = store
        self.stride = stride
        self.shared = shared
        self.weights = ops.LayerWeights(dims, router, store, stride, shared)

    @staticmethod
    def allocate(dims, device="cuda"):
        stride = ops.expert_stride(dims, dims.inter)
        store = torch.empty(dims.n_experts * stride, dtype=torch.uint8, device=device)
        shared = None
        if dims.shared_inter:
            shared = torch.empty(ops.expert_stride(dims, dims.shared_inter), dtype=torch.uint8,
                                 device=device)
        return store, stride, shared

    @classmethod
    def from_canonical(cls, dims, router, expert_arrays, shared_arrays=None, device="cuda"):
        """expert_arrays(e) -> 9 canonical device tensors of expert e; shared_arrays -> 9 tensors."""
        store, stride, shared = cls.allocate(dims, device)
        for e in range(dims.n_experts):
            ops.pack_expert(dims, dims.inter, *expert_arrays(e), store[e * stride:(e + 1) * stride])
        if shared is not None:
            if shared_arrays is None:
                raise ValueError("the dims have a shared expert but no shared arrays were given")
            ops.pack_expert(dims, dims.shared_inter, *shared_arrays, shared)
        return cls(dims, router, store, stride, shared)


def dims_of(hidden, n_experts, top_k, inter, shared_inter=0, expert_bits=4):
    return make_dims(hidden, n_experts, top_k, inter, shared_inter, expert_bits=expert_bits)
