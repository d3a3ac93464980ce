"""GPU parity of moe_decode_layer (gating + sort, GEMM 1, GEMM 2 with the combine in its
epilogue) against the fp64 oracle, its routing outputs against moe_route_topk, and its
agreement with the five-call sequence, determinism, token-order equivariance, graph replay
and workspace reuse."""
import dataclasses

import numpy as np
import pytest

import oracle
import quantized_expert_layer_amd as q
import synth
from tests.gpu_util import assert_layer_close, case, dev, host

pytestmark = pytest.mark.gpu

TINY = synth.get_config("tiny")
# edge shapes: the most rows a call takes (T * k = 512), and the most experts (E = 256)
MAX_ROWS = dataclasses.replace(TINY, name="tiny_k8", cfg_id=101, k=8, T_list=(64,))
MAX_EXPERTS = dataclasses.replace(TINY, name="wide_e256", cfg_id=102, E=256, k=8, inter=128,
                                  T_list=(64,))
# shared experts inside the decode launches: 2 x 64 intermediate columns (the second GEMM's
# K = 128 leaves most of its eight K slices empty), and with more routed rows (T * k = 512) than
# the first launch takes beside them
TINY_SHARED = dataclasses.replace(TINY, name="tiny_shared", cfg_id=103, n_shared=2,
                                  shared_inter=64)
TINY_SHARED_K8 = dataclasses.replace(TINY_SHARED, name="tiny_shared_k8", cfg_id=104, k=8,
                                     T_list=(64,))
CONFIGS = {c.name: c for c in (MAX_ROWS, MAX_EXPERTS, TINY_SHARED, TINY_SHARED_K8)}


def _cfg(name):
    return CONFIGS.get(name) or synth.get_config(name)


_CACHE = {}


def _layer(name, T, wtype=None, decode=None):
    key = (name, T, wtype, decode)
    if key not in _CACHE:
        if len(_CACHE) > 4:
            _CACHE.clear()
        inp = synth.make_inputs(_cfg(name), T, wtype=wtype)
        _CACHE[key] = (inp, q.DeviceLayer.from_inputs(inp, decode=decode))
    return _CACHE[key]


# (config, T, weight type)
DECODE_CASES = [
    ("tiny", 16, None),            # ReLU, int4 per channel, k = 2
    ("tiny", 1, None),
    ("mt_encoder", 1, "int4"),     # top-1, softmax over all experts, per-channel scales
    ("mt_encoder", 8, "int4"),
    ("mt_encoder", 8, "int8"),
    ("mt_encoder", 8, "fp16"),
    ("qwen15_moe", 17, None),      # SwiGLU, group 128, k = 4
    ("dsv2_lite", 9, None),        # + shared experts in the same launches, k = 6
    ("dsv2_lite", 9, "int8"),
    ("dsv2_lite", 32, None),       # 192 routed rows: the shared GEMM 1 as a launch of its own
    ("dsv2_lite", 1, None),        # one token: the first GEMM split over waves, shared beside it
    ("tiny_shared", 16, None),
    ("tiny_shared", 16, "int8"),
    ("tiny_shared", 16, "fp16"),   # fp16 routed weights: shared experts on a side stream
    ("tiny_shared_k8", 64, None),
    ("phi35_moe", 1, None),
    ("phi35_moe", 17, None),
    ("tiny_k8", 64, None),         # 512 routed rows: every expert takes every token
    ("wide_e256", 64, None),       # 256 experts, 4 logits per lane in the gating
]


@pytest.mark.parametrize("name,T,wtype", DECODE_CASES)
def test_decode_layer_matches_oracle(name, T, wtype):
    inp, layer = _layer(name, T, wtype)
    assert layer.uses_decode(T)
    case(f"decode {name} T={T} wtype={inp.wtype}")
    x, L = dev(inp.x), dev(inp.logits)
    ws = layer.workspace(T)
    out = host(layer.forward(x, L, ws=ws))
    ref = oracle.moe_layer(inp)
    rel, mx = assert_layer_close(out, ref, f"decode {name} T={T}")
    print(f"[gpu-case] decode {name} T={T}: rel-L2 {rel:.2e} max/rms {mx:.2e}", flush=True)
    # the routing it returns is moe_route_topk's, bit for bit
    ids, w = q.moe_route_topk(L, inp.cfg.k, inp.cfg.gate_mode)
    assert np.array_equal(host(ws.bufs["ids"]), host(ids))
    assert np.array_equal(host(ws.bufs["w"]).view(np.uint32), host(w).view(np.uint32))


@pytest.mark.parametrize("name,T", [("qwen15_moe", 17), ("dsv2_lite", 9), ("phi35_moe", 1),
                                    ("mt_encoder", 8), ("tiny_shared_k8", 64)])
def test_decode_layer_agrees_with_the_five_calls(name, T):
    """Only the fp16 rounding of each expert's output row differs from the five-call path."""
    inp, fused = _layer(name, T)
    _, plain = _layer(name, T, decode=False)
    assert fused.uses_decode(T) and not plain.uses_decode(T)
    x, L = dev(inp.x), dev(inp.logits)
    case(f"decode vs five calls {name} T={T}")
    a = host(fused.forward(x, L)).astype(np.float64)
    b = host(plain.forward(x, L)).astype(np.float64)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel <= 1e-3, rel


@pytest.mark.parametrize("name,T", [("tiny", 16), ("dsv2_lite", 9), ("mt_encoder", 8),
                                    ("phi35_moe", 1), ("tiny_shared", 16)])
def test_decode_layer_is_deterministic_and_token_order_equivariant(name, T):
    """Bit-identical on repeat, and (every expert holding at most 16 rows here, so a row's
    contributions land in the same place whatever its position) under a token permutation."""
    inp, layer = _layer(name, T)
    x, L = dev(inp.x), dev(inp.logits)
    case(f"decode determinism {name} T={T}")
    a = host(layer.forward(x, L)).copy()
    b = host(layer.forward(x, L)).copy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    p = np.random.default_rng(3).permutation(T)
    c = host(layer.forward(dev(inp.x[p]), dev(inp.logits[p])))
    assert np.array_equal(c.view(np.uint16), a[p].view(np.uint16))


def test_decode_workspace_is_reusable_across_token_counts():
    """One workspace (sized for the larger step) serves a smaller step and back: nothing in it
    carries over from one call to the next."""
    import torch

    name = "qwen15_moe"
    inp17, layer = _layer(name, 17)
    inp5 = synth.make_inputs(_cfg(name), 5)
    ws = layer.workspace(17)
    outs = []
    for inp in (inp17, inp5, inp17):
        T = inp.x.shape[0]
        case(f"decode workspace reuse {name} T={T}")
        out = torch.empty((T, inp.cfg.d), dtype=torch.float16, device="cuda")
        ids = torch.empty((T, inp.cfg.k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, inp.cfg.k), dtype=torch.float32, device="cuda")
        q.moe_decode_layer(dev(inp.logits), dev(inp.x), inp.cfg.k, inp.cfg.gate_mode,
                           inp.cfg.inter, inp.cfg.act, layer.w1, layer.s1, layer.w2, layer.s2,
                           inp.wtype, inp.cfg.group, topk_ids=ids, topk_w=w, out=out,
                           ws=ws.bufs["dws"])
        outs.append(host(out).copy())
    assert np.array_equal(outs[0].view(np.uint16), outs[2].view(np.uint16))
    assert_layer_close(outs[1], oracle.moe_layer(inp5), "T=5 in the T=17 workspace")


@pytest.mark.parametrize("name,T,wtype", [("dsv2_lite", 9, None), ("tiny_shared", 16, "fp16"),
                                          ("tiny_shared_k8", 64, None)])
def test_decode_layer_replays_from_a_graph(name, T, wtype):
    """Captured once, replayed several times with eager work in between: every replay gives
    the eager output (shared experts in the decode launches; on a side stream that the graph
    forks and joins, for fp16 routed weights; the shared GEMM 1 as a launch of its own)."""
    import torch

    inp, layer = _layer(name, T, wtype)
    x, L = dev(inp.x), dev(inp.logits)
    ws = layer.workspace(T)
    case(f"decode graph {name} T={T} wtype={inp.wtype}")
    want = host(layer.forward(x, L, ws=ws)).copy()
    s = torch.cuda.Stream()
    plan = layer.plan(ws, x, L, stream=s)
    assert "decode" in plan.names
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        plan.run()
    for i in range(3):
        ws.bufs["out"].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(ws.bufs["out"]).view(np.uint16), want.view(np.uint16)), i
        layer.forward(dev(inp.x[::-1].copy()), dev(inp.logits[::-1].copy()), ws=ws)
        torch.cuda.synchronize()


def _a256(v):
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("name,T", [("qwen15_moe", 17), ("tiny_k8", 64), ("wide_e256", 64),
                                    ("phi35_moe", 1), ("dsv2_lite", 9)])
def test_decode_sort_matches_moe_permute(name, T):
    """The decode step's one-wave sort leaves perm, inv_perm, offsets, w_perm and the tile table
    at the head of its workspace (256-byte aligned parts, in that order): the first four equal
    moe_permute's, bit for bit, on the same routing, and the table lists the 16-row tiles of
    the offsets."""
    inp, layer = _layer(name, T)
    x, L = dev(inp.x), dev(inp.logits)
    ws = layer.workspace(T)
    case(f"decode sort {name} T={T}")
    layer.forward(x, L, ws=ws)
    E, k = inp.cfg.E, inp.cfg.k
    R = T * k
    raw = ws.bufs["dws"]
    o_inv = _a256(4 * R)
    o_off = _a256(o_inv + 4 * R)
    o_wp = _a256(o_off + 4 * (E + 1))
    i32 = lambda o, n: host(raw[o:o + 4 * n].view(dtype=__import__("torch").int32))
    perm, inv, off = i32(0, R), i32(o_inv, R), i32(o_off, E + 1)
    wp = host(raw[o_wp:o_wp + 4 * R].view(dtype=__import__("torch").float32))
    p2, i2, off2, _, w2 = q.moe_permute(ws.bufs["ids"], ws.bufs["w"], x, E, want_x_perm=False)
    assert np.array_equal(perm, host(p2))
    assert np.array_equal(inv, host(i2))
    assert np.array_equal(off, host(off2))
    assert np.array_equal(wp.view(np.uint32), host(w2).view(np.uint32))
    # then the tile table: the count, then every expert's 16-row tiles in expert order, each
    # packed as e | first_row << 9 | (rows - 1) << 19
    o_tiles = _a256(o_wp + 4 * R)
    n_max = R // 16 + 256
    tab = i32(o_tiles, 1 + n_max)
    want = []
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        for r0 in range(lo, hi, 16):
            want.append(e | (r0 << 9) | ((min(16, hi - r0) - 1) << 19))
    assert tab[0] == len(want)
    assert np.array_equal(tab[1:1 + len(want)], np.array(want, dtype=np.int32))


def test_decode_waits_for_an_addend_made_on_another_stream():
    """addend_ready: the addend is produced on a second stream (behind a slow fill, so it is
    late); the decode call waits for the event before its last launch and adds it exactly as
    an addend ready beforehand."""
    import torch

    name, T = "qwen15_moe", 17
    inp, layer = _layer(name, T)
    x, L = dev(inp.x), dev(inp.logits)
    add_h = np.random.default_rng(2).standard_normal((T, inp.cfg.d)).astype(np.float16)
    want_addend = dev(add_h)
    kw = dict(k=inp.cfg.k, gate_mode=inp.cfg.gate_mode, inter=inp.cfg.inter, act=inp.cfg.act,
              w1=layer.w1, s1=layer.s1, w2=layer.w2, s2=layer.s2, wtype=inp.wtype,
              group_size=inp.cfg.group)
    case("decode addend_ready")
    want = host(q.moe_decode_layer(L, x, addend=want_addend, **kw)[0]).copy()
    side = torch.cuda.Stream()
    late = torch.zeros_like(want_addend)
    big = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
    main = torch.cuda.current_stream()
    ready = torch.cuda.Event()
    with torch.cuda.stream(side):
        side.wait_stream(main)
        for _ in range(20):
            big.fill_(1.0)                          # delay the side stream
        late.copy_(want_addend)
        ready.record(side)
    got = host(q.moe_decode_layer(L, x, addend=late, addend_ready=ready, **kw)[0])
    torch.cuda.synchronize()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("name,T,finished", [("tiny_shared", 16, "all"), ("tiny_shared", 16, "half"),
                                             ("tiny_shared_k8", 64, "all")])
def test_decode_shared_with_finished_tokens(name, T, finished):
    """Batch pruning with the shared experts inside the decode launches: a finished token takes
    no routed expert but still gets the shared experts' output; with every token finished the
    routed blocks find no tile and the output is the shared experts' alone."""
    inp, layer = _layer(name, T)
    active = np.zeros(T, dtype=bool) if finished == "all" else (np.arange(T) % 2 == 0)
    case(f"decode shared pruned {name} T={T} finished={finished}")
    x, L = dev(inp.x), dev(inp.logits)
    ws = layer.workspace(T)
    out = host(layer.forward(x, L, ws=ws, active=dev(active.astype(np.uint8))))
    ref = oracle.moe_layer(inp, active=active)
    assert_layer_close(out, ref, f"decode shared pruned {name} T={T}")
    ids = host(ws.bufs["ids"])
    assert np.all(ids[~active] == -1)
