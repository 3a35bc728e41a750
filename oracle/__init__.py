"""CPU oracle of the routed int4 MoE layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation in fp64 of what the
layer computes.  It exists to check the HIP library, and nothing in the
product path may import or call it: only the tests, the smoke check and the
benchmark's CPU-baseline leg do.  It shares no code with the HIP path; its
only dependency besides numpy is the duck-typed layer object it is handed.

Every function is pinned in tests/test_oracle_pins.py against closed forms,
brute force, textbook special cases and hand-built fixtures (tests/golden).
"""
from .qmoe_oracle import (  # noqa: F401
    EPS, bf16_to_f64, bf16_rne_bits, unpack_nibbles, dequant, dequant_int4,
    dequant_int8, rmsnorm_no_scale, router_logits, topk_select, topk_weights,
    router, bucket, expert_ffn, combine, post_combine, combine_post, layer_forward,
    near_tie_mask,
)
