"""GPU parity of batch pruning ("Who Says Elephants Can't Run", Fig. 1 caption and its list of
optimizations: finished sentences are left out of the computation).  A finished token gets ids
-1 and weights 0, takes no expert, and its output row is the shared experts' output (or 0)."""
import numpy as np
import pytest

import oracle
import quantized_expert_layer_amd as q
import synth
from tests.gpu_util import assert_layer_close, case, dev, host

pytestmark = pytest.mark.gpu


def _mask(T, frac, seed, group=1):
    """Finished tokens in whole groups (sentences) of `group` tokens, about `frac` of them."""
    rng = np.random.default_rng(seed)
    n = (T + group - 1) // group
    fin = rng.random(n) < frac
    return ~np.repeat(fin, group)[:T]


# (config, T, finished fraction, sentence length)
CASES = [
    ("mt_encoder", 3840, 0.5, 40),     # five calls, k = 1 (the combine writes finished rows)
    ("qwen15_moe", 544, 0.3, 17),      # five calls, tile path
    ("dsv2_lite", 288, 0.4, 9),        # five calls + shared experts
    ("qwen15_moe", 17, 0.5, 1),        # decode call
    ("dsv2_lite", 9, 0.5, 1),          # decode call + shared experts
    ("phi35_moe", 17, 0.3, 1),
    ("tiny", 16, 1.0, 1),              # everything finished
    ("phi35_moe", 1, 1.0, 1),
]

_CACHE = {}


def _layer(name, T):
    key = (name, T)
    if key not in _CACHE:
        _CACHE.clear()
        inp = synth.make_inputs(synth.get_config(name), T)
        _CACHE[key] = (inp, q.DeviceLayer.from_inputs(inp))
    return _CACHE[key]


@pytest.mark.parametrize("name,T,frac,group", CASES)
def test_pruned_layer_matches_oracle(name, T, frac, group):
    inp, layer = _layer(name, T)
    active = _mask(T, frac, seed=T, group=group)
    case(f"pruned layer {name} T={T} finished={int((~active).sum())}")
    x, L = dev(inp.x), dev(inp.logits)
    ws = layer.workspace(T)
    out = host(layer.forward(x, L, ws=ws, active=dev(active.astype(np.uint8)))).astype(np.float64)
    toks = np.arange(T) if T <= 600 else np.unique(np.concatenate(
        [np.flatnonzero(active)[:200], np.flatnonzero(~active)[:200]]))
    ref = oracle.moe_layer_tokens(inp, toks, active=active)
    if active[toks].any():
        assert_layer_close(out[toks][active[toks]], ref[active[toks]], f"running rows {name}")
    fin = toks[~active[toks]]
    if not inp.shared:
        assert np.array_equal(out[fin], np.zeros_like(out[fin]))     # exactly zero
    elif fin.size:
        assert_layer_close(out[fin], ref[~active[toks]], f"finished rows {name}")
    # finished tokens route nowhere; running tokens route as without the mask
    ids, w = host(ws.bufs["ids"]), host(ws.bufs["w"])
    assert np.all(ids[~active] == -1) and np.all(w[~active] == 0.0)
    ids0, w0 = q.moe_route_topk(L, inp.cfg.k, inp.cfg.gate_mode)
    assert np.array_equal(ids[active], host(ids0)[active])
    assert np.array_equal(w[active].view(np.uint32), host(w0)[active].view(np.uint32))


@pytest.mark.parametrize("name,T,frac,group", [("mt_encoder", 3840, 0.5, 40),
                                               ("qwen15_moe", 544, 0.3, 17)])
def test_running_rows_are_bit_identical_to_the_unpruned_layer(name, T, frac, group):
    """Rows of a grouped GEMM do not interact, so pruning other tokens leaves a running
    token's output bits unchanged (same GEMM path on both sides at these sizes)."""
    inp, layer = _layer(name, T)
    active = _mask(T, frac, seed=T + 1, group=group)
    x, L = dev(inp.x), dev(inp.logits)
    case(f"pruned rows bit-identical {name} T={T}")
    full = host(layer.forward(x, L)).copy()
    part = host(layer.forward(x, L, active=dev(active.astype(np.uint8))))
    assert np.array_equal(part[active].view(np.uint16), full[active].view(np.uint16))


def test_pruned_plan_replays_from_a_graph():
    import torch

    name, T = "qwen15_moe", 17
    inp, layer = _layer(name, T)
    active = dev(_mask(T, 0.5, seed=9).astype(np.uint8))
    x, L = dev(inp.x), dev(inp.logits)
    ws = layer.workspace(T)
    case(f"pruned graph {name} T={T}")
    want = host(layer.forward(x, L, ws=ws, active=active)).copy()
    s = torch.cuda.Stream()
    plan = layer.plan(ws, x, L, stream=s, active=active)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        plan.run()
    for i in range(3):
        ws.bufs["out"].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(ws.bufs["out"]).view(np.uint16), want.view(np.uint16)), i
        layer.forward(x, L, ws=ws)
        torch.cuda.synchronize()
