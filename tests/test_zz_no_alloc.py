"""moe_decode_layer_noalloc (the decode step on the library's own scratch array, no allocation)
against moe_decode_layer with a caller workspace: two calls in a row, the second with fewer
tokens, each bit-identical to moe_decode_layer and within the layer tolerance of the oracle.
The file's name makes it the last one collected."""
import numpy as np
import pytest

import oracle
import quantized_expert_layer_amd as q
import synth
from tests.gpu_util import assert_layer_close, case, dev, host

pytestmark = pytest.mark.gpu


def _noalloc():
    # the C entry point itself (the binding declares its argument types)
    return q.lib().moe_decode_layer_noalloc


def _call_noalloc(f, inp, layer):
    import torch
    c = inp.cfg
    T = inp.x.shape[0]
    x, lg = dev(inp.x), dev(inp.logits)
    out = torch.full((T, c.d), float("nan"), dtype=torch.float16, device="cuda")
    ids = torch.full((T, c.k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, c.k), float("nan"), dtype=torch.float32, device="cuda")
    st = f(lg.data_ptr(), None, x.data_ptr(), T, c.E, c.k, q.GATES[c.gate_mode], c.d, c.inter,
           q.ACTS[c.act], layer.w1.data_ptr(), layer.s1.data_ptr(), layer.w2.data_ptr(),
           layer.s2.data_ptr(), q.WTYPES[inp.wtype], c.group, None, None, ids.data_ptr(),
           w.data_ptr(), out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, q.status_str(st)
    torch.cuda.synchronize()
    return host(out).copy(), host(ids).copy(), host(w).copy()


def _call_with_workspace(inp, layer):
    c = inp.cfg
    out, ids, w = q.moe_decode_layer(dev(inp.logits), dev(inp.x), c.k, c.gate_mode, c.inter,
                                     c.act, layer.w1, layer.s1, layer.w2, layer.s2, inp.wtype,
                                     c.group)
    return host(out).copy(), host(ids).copy(), host(w).copy()


def test_noalloc_decode_matches_the_workspace_call_twice_in_a_row():
    f = _noalloc()
    cfg = synth.get_config("qwen15_moe")
    big = synth.make_inputs(cfg, 17)
    small = synth.make_inputs(cfg, 5)
    layer = q.DeviceLayer.from_inputs(big)
    for inp in (big, small):
        T = inp.x.shape[0]
        case(f"noalloc decode qwen15_moe T={T}")
        got, gids, gw = _call_noalloc(f, inp, layer)
        want, wids, ww = _call_with_workspace(inp, layer)
        assert np.array_equal(gids, wids)
        assert np.array_equal(gw.view(np.uint32), ww.view(np.uint32))
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), f"T={T}"
        assert_layer_close(got, oracle.moe_layer(inp), f"noalloc T={T}")
