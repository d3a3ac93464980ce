"""GPU parity of the whole layer (route -> permute -> GEMM1 -> GEMM2 -> combine) against the
fp64 oracle on every layer shape, plus determinism and token-order equivariance."""
import numpy as np
import pytest

import oracle
import quantized_expert_layer_amd as q
import synth
from tests.gpu_util import assert_layer_close, case, dev, host

pytestmark = pytest.mark.gpu

_CACHE = {}


def _layer(name, T, wtype=None, active=0, path=0):
    key = (name, T, wtype, active)
    if key not in _CACHE:
        _CACHE.clear()
        inp = synth.make_inputs(synth.get_config(name), T, wtype=wtype, active=active)
        _CACHE[key] = (inp, {})
    inp, layers = _CACHE[key]
    if path not in layers:
        layers[path] = q.DeviceLayer.from_inputs(inp, gemm_path=path)
    return inp, layers[path]


# (config, T, weight type, active experts, tokens the oracle checks: None = all)
LAYER_CASES = [
    ("tiny", 16, None, 0, None),
    ("mt_encoder", 3840, "int4", 0, None),
    ("mt_encoder", 3840, "int8", 0, None),
    ("mt_encoder", 3840, "int4", 1, 512),
    ("mt_encoder", 3840, "int8", 8, 512),
    ("mt_encoder", 3840, "fp16", 8, 512),
    ("qwen15_moe", 17, None, 0, None),
    ("qwen15_moe", 544, None, 0, None),
    ("dsv2_lite", 9, None, 0, None),
    ("dsv2_lite", 288, None, 0, None),
    ("phi35_moe", 1, None, 0, None),
    ("phi35_moe", 17, None, 0, None),
    ("phi35_moe", 8192, None, 0, 256),
    # the active-expert sweep of the MT encoder ([W] section 4, tokens spread over A experts)
    ("mt_encoder", 3840, "int4", 4, 512),
    ("mt_encoder", 3840, "int4", 16, 512),
    ("mt_encoder", 3840, "int4", 24, 512),
]


def _edge_rows(inp):
    """Tokens behind the rows at every expert's tile edges in the sorted order: each expert's
    first and last row, and the first row of its last (ragged) tile and the row before it, for
    the 48- and 64-row tiles.  Routing and sort are the oracle's."""
    k = inp.cfg.k
    ids, _ = oracle.topk_route(inp.logits, k, inp.cfg.gate_mode)
    perm, _, off = oracle.stable_expert_sort(ids, inp.cfg.E)
    rows = []
    for e in range(inp.cfg.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        rows += [lo, hi - 1]
        for bm in (48, 64):
            last = lo + (hi - lo - 1) // bm * bm
            rows += [last, max(lo, last - 1)]
    return np.unique(perm[np.array(rows)] // k)


def _tokens(T, n, inp=None):
    """All T tokens (n None), else n of them: token 0 and T - 1, the tile-edge rows' tokens
    (with inp) and seeded random others."""
    if n is None or n >= T:
        return np.arange(T)
    rng = np.random.default_rng(T)
    must = np.unique(np.concatenate([[0, T - 1]] + ([_edge_rows(inp)] if inp is not None else [])))
    rest = np.setdiff1d(np.arange(T), must)
    extra = rng.choice(rest, max(0, n - must.size), replace=False)
    return np.unique(np.concatenate([must, extra]))


@pytest.mark.parametrize("name,T,wtype,active,n_check", LAYER_CASES)
def test_layer_matches_oracle(name, T, wtype, active, n_check):
    inp, layer = _layer(name, T, wtype, active)
    case(f"layer {name} T={T} wtype={inp.wtype} active={active}")
    out = host(layer.forward(dev(inp.x), dev(inp.logits)))
    toks = _tokens(T, n_check, inp)
    ref = oracle.moe_layer_tokens(inp, toks)
    rel, mx = assert_layer_close(out[toks], ref, f"{name} T={T}")
    print(f"[gpu-case] {name} T={T}: rel-L2 {rel:.2e} max/rms {mx:.2e}", flush=True)


@pytest.mark.parametrize("name,T", [("tiny", 16), ("qwen15_moe", 544), ("dsv2_lite", 9)])
def test_layer_paths_and_gate_placement_agree(name, T):
    for path in (q.PATH_STREAM, q.PATH_TILE):
        inp, layer = _layer(name, T, path=path)
        ref = oracle.moe_layer(inp)
        for fuse in (True, False):
            layer.fuse_rows = fuse
            for gate_in_gemm in (True, False):
                case(f"layer {name} T={T} path={path} fuse_rows={fuse} gate_in_gemm={gate_in_gemm}")
                out = host(layer.forward(dev(inp.x), dev(inp.logits), gate_in_gemm=gate_in_gemm))
                assert_layer_close(out, ref, f"path {path} fuse {fuse} gate_in_gemm {gate_in_gemm}")
        layer.fuse_rows = True


@pytest.mark.parametrize("fuse", [True, False])
def test_layer_row_fusion_is_bit_identical_to_the_copies(fuse):
    """Gathering x through perm inside the first GEMM, and (k = 1) writing the output through
    perm from the second, computes exactly what x_perm + combine compute."""
    name, T = "mt_encoder", 3840
    inp, layer = _layer(name, T)
    x, L = dev(inp.x), dev(inp.logits)
    layer.fuse_rows = False
    case(f"row fusion reference {name} T={T}")
    want = host(layer.forward(x, L)).copy()
    layer.fuse_rows = fuse
    case(f"row fusion {fuse} {name} T={T}")
    got = host(layer.forward(x, L))
    layer.fuse_rows = True
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("wtype", ["int4", "int8"])
def test_layer_native_i2f_is_bit_identical(wtype):
    """The MT encoder layer with the tile GEMMs converting codes by the conversion instructions
    ([W] section 3, the baseline of the optimized I2F) gives the default layer's output bit for
    bit."""
    inp, layer = _layer("mt_encoder", 3840, wtype, 0)
    native = q.DeviceLayer.from_inputs(inp, gemm_i2f=q.I2F_NATIVE)
    x, L = dev(inp.x), dev(inp.logits)
    case(f"layer native i2f mt_encoder T=3840 {wtype}")
    want = host(layer.forward(x, L)).copy()
    got = host(native.forward(x, L))
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("name,T", [("qwen15_moe", 544), ("mt_encoder", 3840), ("phi35_moe", 17)])
def test_layer_is_deterministic_and_token_order_equivariant(name, T):
    inp, layer = _layer(name, T)
    case(f"determinism {name} T={T}")
    x, L = dev(inp.x), dev(inp.logits)
    a = host(layer.forward(x, L)).copy()
    b = host(layer.forward(x, L)).copy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    p = np.random.default_rng(1).permutation(T)
    c = host(layer.forward(dev(inp.x[p]), dev(inp.logits[p])))
    assert np.array_equal(c.view(np.uint16), a[p].view(np.uint16))


@pytest.mark.parametrize("name,T", [("qwen15_moe", 544), ("dsv2_lite", 9)])
def test_plan_outlives_its_layer(name, T):
    """A pre-marshalled plan holds raw device pointers (weights, scales, shared-expert weights,
    workspace); it must keep them alive after the caller drops the layer and the workspace."""
    import gc

    import torch

    inp = synth.make_inputs(synth.get_config(name), T)
    x, logits = dev(inp.x), dev(inp.logits)
    layer = q.DeviceLayer.from_inputs(inp)
    want = host(layer.forward(x, logits))
    plan = layer.plan(layer.workspace(T), x, logits)
    del layer
    gc.collect()
    # churn the caching allocator so freed blocks would be handed out again and overwritten
    junk = [torch.full((1 << 20,), float("nan"), dtype=torch.float16, device="cuda")
            for _ in range(64)]
    case(f"plan without its layer {name} T={T}")
    plan.run()
    got = host(plan.out)
    del junk
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("name,T,n_check,overlap", [("mt_encoder", 3840, 64, False),
                                                    ("qwen15_moe", 544, 64, False),
                                                    ("dsv2_lite", 288, 64, False),
                                                    ("dsv2_lite", 288, 64, True),
                                                    ("phi35_moe", 8192, 256, False)])
def test_layer_replays_from_a_graph(name, T, n_check, overlap):
    """The step the bench times: the layer plan captured once in a HIP graph and replayed with
    eager work in between (with overlap, the shared experts on a forked stream inside the
    graph).  Every replay gives the eager output bit for bit, and sampled tokens of the
    replayed output match the fp64 oracle."""
    import torch

    inp, layer = _layer(name, T, None, 0)
    x, L = dev(inp.x), dev(inp.logits)
    ws = layer.workspace(T)
    case(f"layer graph {name} T={T} overlap={overlap}")
    want = host(layer.forward(x, L, ws=ws)).copy()
    s = torch.cuda.Stream()
    plan = layer.plan(ws, x, L, stream=s, overlap_shared=overlap)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        plan.run()
    for i in range(3):
        ws.bufs["out"].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = host(ws.bufs["out"])
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), i
        # eager work on other inputs between the replays
        layer.forward(dev(inp.x[::-1].copy()), dev(inp.logits[::-1].copy()), ws=ws)
        torch.cuda.synchronize()
    toks = _tokens(T, n_check, inp)
    assert_layer_close(got[toks], oracle.moe_layer_tokens(inp, toks), f"graph {name} T={T}")
