"""Pins of the CPU oracle against what the pages and mathematics fix (CPU only).

Each test names the passage or fact it checks.  Pages:
  [W] "Who Says Elephants Can't Run" review, section 3 (Algorithm 1, optimized I2F, workflow)
  [S] "Specter" summary (Background / MoE; Method steps, step 5)
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth
from tests import brute

RNG = np.random.default_rng(12345)


def _golden(golden_dir, name):
    rows = []
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- fp16 rounding helper
def test_brute_fp16_round_is_ieee_binary16():
    vals = np.concatenate([RNG.standard_normal(20000) * 10.0 ** RNG.integers(-9, 5, 20000),
                           np.array([0.5 * 2.0 ** -24, 1.5 * 2.0 ** -24, 65504.0, 65519.9,
                                     65520.0, 2.0 ** -14, 1e-9])])
    for v in vals:
        assert brute.fp16_round(float(v)) == float(np.float16(v)), v


# ---------------------------------------------------------------- Algorithm 1  [W] sec. 3
def test_algorithm1_hand_worked_products(golden_dir):
    for sbits, code, ebits in _golden(golden_dir, "algorithm1_products.txt"):
        s = np.array([int(sbits, 16)], dtype=np.uint16).view(np.float16).reshape(1, 1, 1)
        c = np.array([int(code)], dtype=np.int8).reshape(1, 1, 1)
        got = oracle.dequant_algorithm1(c, s, 0).view(np.uint16)[0, 0, 0]
        assert got == int(ebits, 16), (sbits, code, hex(got), ebits)


def test_algorithm1_unit_and_power_of_two_scales():
    codes = RNG.integers(-128, 128, size=(3, 256, 16)).astype(np.int8)
    one = np.ones((3, 1, 16), np.float16)
    assert np.array_equal(oracle.dequant_algorithm1(codes, one, 0).astype(np.float64), codes)
    for j in (-12, -3, 0, 4, 7):
        s = np.full((3, 2, 16), 2.0 ** j, np.float16)
        got = oracle.dequant_algorithm1(codes, s, 128).astype(np.float64)
        assert np.array_equal(got, codes.astype(np.float64) * 2.0 ** j)


def test_algorithm1_scale_indexing():
    # Distinct power-of-two scales per (e, group, n) and unit codes: W_dq[e,m,n] must equal
    # S[e, m // 128, n] (a transposed or off-by-group index gives other values).
    E, K, N = 2, 384, 8
    expo = np.arange(E * (K // 128) * N).reshape(E, K // 128, N) % 20 - 10
    s = (2.0 ** expo).astype(np.float16)
    codes = np.ones((E, K, N), np.int8)
    got = oracle.dequant_algorithm1(codes, s, 128)
    for e in range(E):
        for m in range(K):
            assert np.array_equal(got[e, m], s[e, m // 128])
    # per-channel: (E, 1, N)
    got = oracle.dequant_algorithm1(codes, s[:, :1], 0)
    assert np.array_equal(got, np.broadcast_to(s[:, :1], (E, K, N)))


def test_algorithm1_vs_brute_force():
    for group, K in ((0, 64), (128, 256)):
        G = 1 if group == 0 else K // group
        codes = RNG.integers(-128, 128, size=(2, K, 12)).astype(np.int8)
        s = RNG.uniform(2.0 ** -20, 8.0, size=(2, G, 12)).astype(np.float16)
        got = oracle.dequant_algorithm1(codes, s, group)
        for e in range(2):
            ref = brute.brute_dequant(codes[e].tolist(), s[e].astype(float).tolist(), group)
            assert np.array_equal(got[e].astype(np.float64), np.array(ref)), (group, e)


# ---------------------------------------------------------------- optimized I2F  [W] sec. 3
def _f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def test_i2f_exponent_of_1024_reading(golden_dir):
    g = {r[0]: r[1:] for r in _golden(golden_dir, "i2f_constants.txt")}
    base = int(g["fp16_bits_of_1024"][0], 16)
    assert _f16(base) == 1024.0
    Y = np.arange(1024, dtype=np.uint16)
    assert np.array_equal(_f16(base | Y), 1024.0 + Y)       # Y + 1024 for every Y < 1024


def test_i2f_int8_all_codes(golden_dir):
    # 8-bit variant: the byte written into the mantissa is the offset-binary code q + 128,
    # so subtracting 1152 = 1024 + 128 gives q, exactly, for all 256 codes.
    g = {r[0]: r[1:] for r in _golden(golden_dir, "i2f_constants.txt")}
    sub = float(g["int8_subtrahend"][0])
    q = np.arange(-128, 128)
    u = (q.astype(np.int16).astype(np.uint16) ^ 0x80) & 0xFF      # two's complement xor 0x80
    assert np.array_equal(u, q + 128)
    assert np.array_equal(_f16(0x6400 | u) - sub, q)


def test_i2f_int4_all_codes_both_nibble_positions():
    q = np.arange(-8, 8)
    u = (q + 8).astype(np.uint16)
    assert np.array_equal(_f16(0x6400 | u) - 1032.0, q)          # low nibble: 1024 + 8
    # a nibble four bits higher lands as 16 * u in the mantissa: scale by 1/16, subtract 72
    assert np.array_equal(_f16(0x6400 | (u << 4)) * (1.0 / 16.0) - 72.0, q)


def test_i2f_int4_nibble_order_gives_adjacent_pairs(golden_dir):
    # 4-bit variant: nibbles stored as [e0,e2,e4,e6,e1,e3,e5,e7]; masking 0x000F000F (or
    # 0x00F000F0) of the word, or of the word shifted right by 8, yields the fp16 pairs
    # [e0,e1], [e2,e3], [e4,e5], [e6,e7] in the (low, high) halves.
    g = {r[0]: r[1:] for r in _golden(golden_dir, "i2f_constants.txt")}
    order = [int(v) for v in g["int4_stored_order"]]
    for _ in range(200):
        e = RNG.integers(-8, 8, size=8)
        w = 0
        for p, src in enumerate(order):
            w |= int(e[src] + 8) << (4 * p)
        pairs = []
        for src_word, mask, mul, sub in ((w, 0x000F000F, 1.0, 1032.0),
                                         (w, 0x00F000F0, 1.0 / 16.0, 72.0),
                                         (w >> 8, 0x000F000F, 1.0, 1032.0),
                                         (w >> 8, 0x00F000F0, 1.0 / 16.0, 72.0)):
            v = (src_word & mask) | 0x64006400
            lo, hi = v & 0xFFFF, v >> 16
            pairs += [_f16(lo) * mul - sub, _f16(hi) * mul - sub]
        assert np.array_equal(np.array(pairs, dtype=np.float64).ravel(), e)


# ---------------------------------------------------------------- top-k  [S] Background/MoE
def test_topk_hand_cases():
    L = np.array([[1.0, 3.0, 3.0, 2.0]], np.float32)
    ids, _ = oracle.topk_route(L, 2, "topk")
    assert ids.tolist() == [[1, 2]]                    # tie -> smaller index first
    ids, _ = oracle.topk_route(np.array([[-0.0, 0.0]], np.float32), 1, "topk")
    assert ids.tolist() == [[0]]                       # -0 == +0
    ids, _ = oracle.topk_route(np.array([[0.0, -0.0]], np.float32), 1, "topk")
    assert ids.tolist() == [[0]]
    ids, w = oracle.topk_route(np.array([[-1e30, -5.0, -1e30]], np.float32), 3, "all")
    assert ids.tolist() == [[1, 0, 2]]
    assert w[0, 0] == 1.0 and w[0, 1] == 0.0


def test_topk_vs_all_subsets_brute_force():
    for E in range(1, 9):
        L = synth.gen.tie_heavy_logits(12, E, seed=E)
        for k in range(1, E + 1):
            ids, w = oracle.topk_route(L, k, "topk")
            ids_a, w_a = oracle.topk_route(L, k, "all")
            for t in range(L.shape[0]):
                row = [float(v) for v in L[t]]
                ref = brute.brute_topk(row, k)
                assert ids[t].tolist() == ref and ids_a[t].tolist() == ref
                np.testing.assert_allclose(w[t], brute.brute_gate_weights(row, ref, "topk"),
                                           rtol=1e-12, atol=1e-300)
                np.testing.assert_allclose(w_a[t], brute.brute_gate_weights(row, ref, "all"),
                                           rtol=1e-12, atol=1e-300)


def test_gate_weight_closed_forms():
    ln3 = np.float32(math.log(3.0))
    _, w = oracle.topk_route(np.array([[ln3, 0.0]], np.float32), 2, "topk")
    np.testing.assert_allclose(w[0], [0.75, 0.25], rtol=1e-7)
    _, w = oracle.topk_route(np.array([[ln3, 0.0, -1e30, 0.0]], np.float32), 2, "all")
    np.testing.assert_allclose(w[0], [0.6, 0.2], rtol=1e-7)   # 3/5 and 1/5
    _, w = oracle.topk_route(np.array([[2.0, 2.0, 2.0, 2.0]], np.float32), 3, "topk")
    np.testing.assert_allclose(w[0], [1 / 3] * 3, rtol=1e-15)
    _, w = oracle.topk_route(np.array([[7.0, 1.0]], np.float32), 1, "topk")
    assert w[0, 0] == 1.0


# ---------------------------------------------------------------- sort  [W] sec. 3 workflow
def _textbook_counting_sort(keys, E):
    count = [0] * E
    for key in keys:
        count[key] += 1
    start, acc = [0] * E, 0
    for e in range(E):
        start[e], acc = acc, acc + count[e]
    perm = [0] * len(keys)
    for f, key in enumerate(keys):          # ascending f -> stable
        perm[start[key]] = f
        start[key] += 1
    return perm


@pytest.mark.parametrize("T,k,E,skew", [(1, 1, 1, False), (16, 2, 8, False), (97, 4, 60, True),
                                        (300, 6, 64, True), (50, 1, 32, True), (0, 2, 8, False)])
def test_sort_invariants_and_textbook(T, k, E, skew):
    ids = synth.gen.random_ids(T, k, E, seed=T, skew=skew) if T else np.zeros((0, k), np.int32)
    perm, inv, off = oracle.stable_expert_sort(ids, E)
    key = ids.ravel()
    R = T * k
    assert sorted(perm.tolist()) == list(range(R))                    # a permutation
    assert np.array_equal(inv[perm], np.arange(R))                    # inverse restores order
    assert np.all(np.diff(key[perm]) >= 0)                            # grouped by expert
    for e in range(E):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)                               # stable within a key
        assert np.all(key[seg] == e)
    assert off[0] == 0 and off[E] == R
    assert perm.tolist() == _textbook_counting_sort(key.tolist(), E)


def test_permute_rows_definition():
    ids = synth.gen.random_ids(40, 3, 10, seed=3)
    perm, _, _ = oracle.stable_expert_sort(ids, 10)
    x = RNG.standard_normal((40, 16)).astype(np.float16)
    xp = oracle.permute_rows(x, perm, 3)
    for p in range(120):
        assert np.array_equal(xp[p].view(np.uint16), x[perm[p] // 3].view(np.uint16))


# ---------------------------------------------------------------- layer: hand-worked examples
def _inputs(x, logits, c1, s1, c2, s2, k, gate_mode, act, group=0):
    cfg = synth.LayerConfig("hand", 0, d=len(x[0]), inter=np.asarray(c2).shape[1],
                            E=np.asarray(c1).shape[0], k=k, act=act, wtypes=("int4",),
                            group=group, gate_mode=gate_mode, zipf_bias=False,
                            T_list=(len(x),))
    return synth.LayerInputs(cfg=cfg, T=len(x), wtype="int4", active=0, coverage=False,
                             seed=(0,), x=np.array(x, np.float16),
                             logits=np.array(logits, np.float32),
                             codes1=np.array(c1, np.int8), scales1=np.array(s1, np.float16),
                             codes2=np.array(c2, np.int8), scales2=np.array(s2, np.float16))


def test_layer_hand_worked_examples(golden_dir):
    g = {r[0]: [float(v) for v in r[1:]] for r in _golden(golden_dir, "layer_worked_examples.txt")}
    c1 = [[[1, -2], [3, 0]], [[-1, 2], [1, 1]]]
    s1 = [[[0.5, 1]], [[2, 0.5]]]
    c2 = [[[2, 1], [-1, 4]], [[1, 0], [2, -3]]]
    s2 = [[[1, 0.25]], [[0.5, 2]]]
    A = _inputs([[1, 2], [3, 1]], [[0.5, 1.0], [2.0, -1.0]], c1, s1, c2, s2, 1, "topk", "relu")
    assert np.array_equal(oracle.moe_layer(A).ravel(), g["A.out"])
    B = _inputs([[1, 2]], [[math.log(3.0), 0.0]], c1, s1, c2, s2, 2, "topk", "relu")
    np.testing.assert_allclose(oracle.moe_layer(B).ravel(), g["B.out"], rtol=1e-6)
    C = _inputs([[1]], [[0.0]], [[[1, 3]]], [[[2, 1]]], [[[1]]], [[[1]]], 1, "topk", "swiglu")
    np.testing.assert_allclose(oracle.moe_layer(C).ravel(), g["C.out"], rtol=1e-14)


def _lists(a):
    return np.asarray(a, dtype=np.float64).tolist()


@pytest.mark.parametrize("gate_mode", ["topk", "all"])
@pytest.mark.parametrize("coverage", [False, True])
def test_layer_vs_brute_force_tiny(gate_mode, coverage):
    inp = synth.make_inputs(synth.get_config("tiny"), 16, coverage=coverage)
    got = oracle.moe_layer(inp, gate_mode=gate_mode)
    ref = brute.brute_layer(_lists(inp.x), _lists(inp.logits), inp.codes1.tolist(),
                            _lists(inp.scales1), inp.codes2.tolist(), _lists(inp.scales2),
                            0, inp.cfg.k, gate_mode, "relu")
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-11, atol=1e-12 * np.abs(ref).max())


def test_swiglu_layer_vs_brute_force_with_shared():
    cfg = synth.LayerConfig("tiny_swiglu", 9, d=128, inter=128, E=6, k=3, act="swiglu",
                            wtypes=("int4",), group=128, gate_mode="all", zipf_bias=True,
                            T_list=(5,), n_shared=2, shared_inter=64)
    inp = synth.make_inputs(cfg, 5)
    got = oracle.moe_layer(inp)
    shared = [(_lists(w1), _lists(w2)) for w1, w2 in inp.shared]
    ref = brute.brute_layer(_lists(inp.x), _lists(inp.logits), inp.codes1.tolist(),
                            _lists(inp.scales1), inp.codes2.tolist(), _lists(inp.scales2),
                            128, 3, "all", "swiglu", shared)
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-11, atol=1e-12 * np.abs(ref).max())


# ---------------------------------------------------------------- batch pruning pins
# [W] Fig. 1 caption and the list of optimizations: a finished sentence is left out of the
# computation.  A finished token takes no routed expert; the shared experts still apply.
def test_pruned_layer_vs_brute_force():
    cfg = synth.LayerConfig("tiny_swiglu", 9, d=128, inter=128, E=6, k=3, act="swiglu",
                            wtypes=("int4",), group=128, gate_mode="all", zipf_bias=True,
                            T_list=(6,), n_shared=2, shared_inter=64)
    inp = synth.make_inputs(cfg, 6)
    active = [1, 0, 1, 1, 0, 0]
    got = oracle.moe_layer(inp, active=np.array(active, dtype=bool))
    shared = [(_lists(w1), _lists(w2)) for w1, w2 in inp.shared]
    ref = brute.brute_layer(_lists(inp.x), _lists(inp.logits), inp.codes1.tolist(),
                            _lists(inp.scales1), inp.codes2.tolist(), _lists(inp.scales2),
                            128, 3, "all", "swiglu", shared, active=active)
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-11, atol=1e-12 * np.abs(ref).max())


def test_pruning_special_cases():
    inp = synth.make_inputs(synth.get_config("tiny"), 16)
    full = oracle.moe_layer(inp)
    # nothing pruned: the plain layer
    assert np.array_equal(oracle.moe_layer(inp, active=np.ones(16, bool)), full)
    # everything pruned, no shared experts: zeros
    assert np.array_equal(oracle.moe_layer(inp, active=np.zeros(16, bool)), np.zeros_like(full))
    # tokens are independent: running rows equal the unpruned rows, finished rows are 0
    active = np.random.default_rng(4).random(16) < 0.5
    part = oracle.moe_layer(inp, active=active)
    np.testing.assert_allclose(part[active], full[active], rtol=1e-13, atol=1e-15)
    assert np.array_equal(part[~active], np.zeros_like(part[~active]))


def test_pruned_rows_keep_the_shared_experts():
    cfg = synth.LayerConfig("tiny_swiglu", 9, d=128, inter=128, E=6, k=3, act="swiglu",
                            wtypes=("int4",), group=128, gate_mode="all", zipf_bias=True,
                            T_list=(5,), n_shared=2, shared_inter=64)
    inp = synth.make_inputs(cfg, 5)
    out = oracle.moe_layer(inp, active=np.zeros(5, bool))
    assert np.array_equal(out, oracle.shared_ffn(inp.x, inp.shared))


# ---------------------------------------------------------------- grouped GEMM / FFN pins
def test_grouped_gemm_one_hot_rows_reproduce_weight_rows():
    inp = synth.make_inputs(synth.get_config("tiny"), 16, coverage=True)
    wdq = oracle.dequant_algorithm1(inp.codes1, inp.scales1, 0)
    E, K, N = wdq.shape
    offsets = np.arange(0, (E + 1) * K, K)           # expert e gets K one-hot rows
    a = np.tile(np.eye(K), (E, 1))
    for act in ("none", "relu"):
        out = oracle.grouped_gemm(a, offsets, wdq, act)
        ref = wdq.astype(np.float64).reshape(E * K, N)
        if act == "relu":
            ref = np.maximum(ref, 0)
        assert np.array_equal(out, ref)
    # swiglu: one-hot row i gives silu(Wg[i]) * Wu[i]
    out = oracle.grouped_gemm(a, offsets, wdq, "swiglu").reshape(E, K, N // 2)
    g, u = wdq[..., :N // 2].astype(np.float64), wdq[..., N // 2:].astype(np.float64)
    np.testing.assert_allclose(out, g / (1 + np.exp(-g)) * u, rtol=1e-15, atol=0)


def test_swiglu_odd_part_identity():
    # silu(z) - silu(-z) = z, so FFN(x) + FFN(-x) = ((x Wg) * (x Wu)) W2 for SwiGLU experts.
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 32))
    w1 = rng.standard_normal((32, 2 * 24)) * 0.2
    w2 = rng.standard_normal((24, 32)) * 0.2
    lhs = oracle.expert_ffn(x, w1, w2, "swiglu") + oracle.expert_ffn(-x, w1, w2, "swiglu")
    rhs = ((x @ w1[:, :24]) * (x @ w1[:, 24:])) @ w2
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_down_scale_power_of_two_scales_output_exactly():
    inp = synth.make_inputs(synth.get_config("tiny"), 16)
    base = oracle.moe_layer(inp)
    inp.scales2 = (inp.scales2.astype(np.float32) * 8.0).astype(np.float16)
    assert np.array_equal(oracle.moe_layer(inp), base * 8.0)


@pytest.mark.parametrize("name,T", [("tiny", 16)])
@pytest.mark.parametrize("gate_mode", ["topk", "all"])
def test_sorted_pipeline_equals_plain_definition(name, T, gate_mode):
    # [S] step 5: grouping by expert, computing, then scattering back is equivalent.
    inp = synth.make_inputs(synth.get_config(name), T)
    cfg = inp.cfg
    ids, w = oracle.topk_route(inp.logits, cfg.k, gate_mode)
    perm, inv, off = oracle.stable_expert_sort(ids, cfg.E)
    xp = oracle.permute_rows(inp.x, perm, cfg.k)
    w1 = oracle.dequant_algorithm1(inp.codes1, inp.scales1, cfg.group)
    w2 = oracle.dequant_algorithm1(inp.codes2, inp.scales2, cfg.group)
    h = oracle.grouped_gemm(xp, off, w1, cfg.act)
    y = oracle.grouped_gemm(h, off, w2, "none", row_scale=w.ravel()[perm])
    out_a = oracle.unpermute_combine(y, inv, cfg.k)                 # gate weight in GEMM 2
    y2 = oracle.grouped_gemm(h, off, w2, "none")
    out_b = oracle.unpermute_combine(y2, inv, cfg.k, w=w)           # gate weight at combine
    ref = oracle.moe_layer(inp, gate_mode=gate_mode)
    np.testing.assert_allclose(out_a, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out_b, ref, rtol=1e-12, atol=1e-13)


def test_unpermute_combine_hand_case():
    # T=2, k=2: slot order f = [t0j0, t0j1, t1j0, t1j1]; perm puts them at positions 2,0,3,1.
    inv = np.array([2, 0, 3, 1], np.int32)
    y = np.array([[10.0], [20.0], [1.0], [2.0]])     # y_perm rows by sorted position
    w = np.array([[0.5, 0.25], [1.0, 2.0]])
    out = oracle.unpermute_combine(y, inv, 2, w=w, addend=np.array([[100.0], [0.0]]))
    # t0 = 0.5*y[2] + 0.25*y[0] + 100 = 0.5 + 2.5 + 100 ; t1 = 1*y[3] + 2*y[1] = 2 + 40
    assert out.ravel().tolist() == [103.0, 42.0]


def test_shared_experts_equal_one_concatenated_expert():
    # Two always-on SwiGLU experts summed equal one expert with concatenated intermediate
    # columns [gate_a | gate_b | up_a | up_b] and stacked down rows [W2_a ; W2_b].
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, 16)).astype(np.float16)
    sh = [((rng.standard_normal((16, 2 * 8)) * 0.1).astype(np.float16),
           (rng.standard_normal((8, 16)) * 0.1).astype(np.float16)) for _ in range(2)]
    ref = oracle.shared_ffn(x, sh)
    (a1, a2), (b1, b2) = sh
    w1 = np.concatenate([a1[:, :8], b1[:, :8], a1[:, 8:], b1[:, 8:]], axis=1)
    w2 = np.concatenate([a2, b2], axis=0)
    got = oracle.expert_ffn(x, oracle.dense_weights(w1), oracle.dense_weights(w2), "swiglu")
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_token_subset_equals_full_layer_rows():
    inp = synth.make_inputs(synth.get_config("tiny"), 16)
    full = oracle.moe_layer(inp)
    sub = np.array([3, 0, 15, 7])
    assert np.array_equal(oracle.moe_layer_tokens(inp, sub), full[sub])


def test_fp16_experts_equal_their_dequantized_codes():
    """The FP16-expert baseline ([W] section 4's comparison) run on Algorithm 1's dequantized
    weights gives exactly the quantized layer."""
    import dataclasses
    inp = synth.make_inputs(synth.get_config("tiny"), 16)
    w1 = oracle.dequant_algorithm1(inp.codes1, inp.scales1, inp.cfg.group)
    w2 = oracle.dequant_algorithm1(inp.codes2, inp.scales2, inp.cfg.group)
    as_fp16 = dataclasses.replace(inp, wtype="fp16", codes1=w1, codes2=w2, scales1=None,
                                  scales2=None)
    assert np.array_equal(oracle.moe_layer(as_fp16), oracle.moe_layer(inp))


def test_fp16_expert_inputs_are_seeded_normals():
    inp = synth.make_inputs(synth.get_config("mt_encoder"), 8, wtype="fp16", active=2)
    assert inp.scales1 is None and inp.scales2 is None
    assert inp.codes1.dtype == np.float16 and inp.codes1.shape == (32, 1024, 4096)
    sd = float(inp.codes1[:2].astype(np.float64).std())
    assert abs(sd - 0.02) < 1e-3
    again = synth.make_inputs(synth.get_config("mt_encoder"), 8, wtype="fp16", active=2)
    assert np.array_equal(again.codes2[5], inp.codes2[5])


# ---------------------------------------------------------------- expert lookahead buffer pins
def _elb_golden(golden_dir):
    g = {}
    for line in open(os.path.join(golden_dir, "elb_worked_example.txt")):
        line = line.split("#")[0].split()
        if line:
            g[line[0]] = np.array([int(v) for v in line[1:]])
    return g


def test_elb_worked_example(golden_dir):
    g = _elb_golden(golden_dir)
    counts = np.zeros((2, 5), dtype=np.int64)
    counts = oracle.elb_accumulate(counts, g["step1"].reshape(2, 2, 2), 5)
    counts = oracle.elb_accumulate(counts, g["step2"].reshape(2, 2, 2), 5)
    assert np.array_equal(counts.ravel(), g["counts"])
    ex, cn = oracle.elb_top_m(counts, 3)
    assert np.array_equal(ex.ravel(), g["top3_experts"])
    assert np.array_equal(cn.ravel(), g["top3_counts"])


def test_elb_matches_the_counting_rule_brute_force():
    """The definition written out with Python sets and loops, on random small inputs."""
    rng = np.random.default_rng(11)
    for trial in range(20):
        L, T, k, E, steps = (int(rng.integers(1, 4)), int(rng.integers(1, 4)),
                             int(rng.integers(1, 4)), int(rng.integers(1, 7)),
                             int(rng.integers(1, 5)))
        all_ids = rng.integers(-1, E, size=(steps, L, T, k))
        counts = np.zeros((L, E), dtype=np.int64)
        for i in range(steps):
            counts = oracle.elb_accumulate(counts, all_ids[i], E)
        for j in range(L):
            for e in range(E):
                want = sum(1 for i in range(steps)
                           if e in {int(v) for v in all_ids[i, j].ravel()})
                assert counts[j, e] == want
        M = int(rng.integers(1, E + 1))
        ex, cn = oracle.elb_top_m(counts, M)
        for j in range(L):
            ranked = sorted(range(E), key=lambda e: (-counts[j, e], e))[:M]
            assert list(ex[j]) == ranked and list(cn[j]) == [counts[j, e] for e in ranked]


# ---------------------------------------------------------------- BF16 bit-field pins
def test_bf16_fields_hand_worked(golden_dir):
    import torch
    for line in open(os.path.join(golden_dir, "bf16_fields.txt")):
        line = line.split("#")[0].split()
        if not line:
            continue
        name, bits, e, sm = line[0], int(line[1], 16), int(line[2], 16), int(line[3], 16)
        ge, gsm = oracle.bf16_decompose(np.array([bits], np.uint16))
        assert (int(ge[0]), int(gsm[0])) == (e, sm), name
        assert int(oracle.bf16_recombine(ge, gsm)[0]) == bits, name
        # the bit pattern is the value the row names (torch's own bf16 encoding)
        if name not in ("nan", "2^-133"):
            want = torch.tensor([float(name)], dtype=torch.bfloat16).view(torch.int16).item() & 0xFFFF
            assert want == bits, name
    assert torch.tensor([2.0 ** -133], dtype=torch.bfloat16).view(torch.int16).item() == 1


def test_bf16_round_trip_is_lossless_for_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    e, sm = oracle.bf16_decompose(bits)
    assert np.array_equal(oracle.bf16_recombine(e, sm), bits)
    # each field takes every value: 256 exponents, 256 sign-mantissa bytes
    assert np.unique(e).size == 256 and np.unique(sm).size == 256
