"""GPU parity of the BF16 bit-field recombination ("ZipMoE" note, BF16 bit-field lossless
compression): the fields the oracle splits off are merged back into the original bits."""
import numpy as np
import pytest

import oracle
import quantized_expert_layer_amd as q
from tests.gpu_util import case, dev, host

pytestmark = pytest.mark.gpu


def _round_trip(bits):
    import torch
    e, sm = oracle.bf16_decompose(bits)
    out = q.moe_bf16_recombine(dev(e), dev(sm))
    assert out.dtype == torch.bfloat16
    return host(out.view(torch.int16)).view(np.uint16)


def test_every_bf16_pattern_comes_back():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    case("bf16 all patterns")
    assert np.array_equal(_round_trip(bits), bits)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 31, 33, 4095, (1 << 22) + 13])
def test_ragged_sizes_and_real_values(n):
    """Normal(0, 0.02) expert-like weights in bf16, sizes around the 16-value chunk."""
    import torch
    w = torch.from_numpy(np.random.default_rng(n).standard_normal(n).astype(np.float32) * 0.02)
    bits = w.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    case(f"bf16 n={n}")
    got = _round_trip(bits)
    assert np.array_equal(got, bits)


def test_no_write_past_n():
    """The tail is written value by value: the output's bytes past n stay untouched."""
    import torch
    n = 37
    bits = np.random.default_rng(1).integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    e, sm = oracle.bf16_decompose(bits)
    big = torch.full((64,), 7.0, dtype=torch.bfloat16, device="cuda")
    case("bf16 guard")
    q.moe_bf16_recombine(dev(e), dev(sm), out=big)
    h = host(big.view(torch.int16)).view(np.uint16)
    assert np.array_equal(h[:n], bits)
    assert np.all(h[n:] == np.uint16(0x40E0))                 # 7.0 in bf16
