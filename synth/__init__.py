"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This package draws random numbers and nothing else: it holds none of the layer's
arithmetic (no routing, sorting, dequantization, GEMM or combine).  Both the HIP
path and the CPU oracle consume exactly the arrays it returns.
"""
from .configs import CONFIGS, LayerConfig, get_config  # noqa: F401
from .gen import LayerInputs, make_inputs  # noqa: F401
