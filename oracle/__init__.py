"""CPU oracle for the weight-only-quantized MoE expert layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow NumPy (fp64 for floating point) implementation of what the layer computes,
written from the pages' description.  Only the tests, the package's smoke() check and the
benchmark's CPU-baseline leg may import it.  It shares no code with the HIP path and
never calls it.

Every function is pinned by CPU tests (tests/test_oracle_*.py) against closed forms,
hand-worked examples (tests/golden/), invariants and a pure-Python brute force.
"""
from .oracle import (  # noqa: F401
    GATE_ALL, GATE_TOPK,
    topk_route, stable_expert_sort, permute_rows, dequant_algorithm1, dense_weights,
    expert_ffn, grouped_gemm, unpermute_combine, shared_ffn, moe_layer, moe_layer_tokens,
    elb_accumulate, elb_top_m, bf16_decompose, bf16_recombine,
)
