"""The attainable-peak probes compute what they claim (so their timings measure real work)."""
import numpy as np
import pytest

import quantized_expert_layer_amd as q
from tests.gpu_util import case

pytestmark = pytest.mark.gpu


def test_probe_read_xors_every_word():
    import torch
    n = (1 << 20) + 12                                   # 16-byte words, ragged vs the grid
    data = np.random.default_rng(5).integers(0, 2**32, size=4 * n, dtype=np.uint32)
    src = torch.from_numpy(data.view(np.int32)).cuda()
    case("probe read")
    sink = q.moe_probe_read(src, 37).cpu().numpy().view(np.uint32)
    assert np.bitwise_xor.reduce(sink) == np.bitwise_xor.reduce(data)


def test_probe_mfma_sums_exactly():
    case("probe mfma")
    out = q.moe_probe_mfma(300, 5).cpu().numpy()
    assert out.shape == (5 * 256,) and np.all(out == 512.0 * 300)
