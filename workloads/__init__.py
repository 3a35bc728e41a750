"""Seeded synthetic inputs for the routed int4 MoE layer.

This package is the one module shared by the CPU oracle and the HIP path. It
only *draws* inputs: counter-based random numbers, the synthetic weight
quantiser that turns drawn floats into MLX-style affine codes, and the
workload configurations. It holds none of the layer's arithmetic (no
dequantisation, routing, FFN or combine).

Sources cited in this package:
  [TF]  "TurboFieldfare" post on discuss.pytorch.kr (Gemma 4 26B-A4B on an
        8 GB Mac, Swift/Metal).  Sections used: "TurboFieldfare의 전문가
        스트리밍 구조" (expert-streaming structure: 30 layers, 128 experts,
        top-8, shared expert, 128-token prefill chunks) and "TurboFieldfare가
        메모리를 아끼는 방식" (4-bit MLX affine, 64-weight groups, bf16 scale
        and bias, 8-bit router projection).
  [SW]  Swiftlet article on tech.utomolab.com.  Section "같은 모델을 왜 이렇게
        적은 메모리로 돌릴 수 있나" (512 experts/top-10 and 256 experts/top-8;
        fixed-stride expert blocks).
"""
from .philox import philox4x32_10, PHILOX_M0, PHILOX_M1, PHILOX_W0, PHILOX_W1  # noqa: F401
from .gen import (  # noqa: F401
    CONFIGS, Config, config, LayerInputs, ExpertWeights, make_router, make_expert,
    make_shared, make_hidden, make_layer_small, normal_f32, quantize_groups,
    bf16_bits_from_f32, expert_bytes, credited_expert_bytes, Tag,
)
