"""GPU parity: Algorithm 1 dequantization (bit-exact) and the grouped GEMM (tolerance; exact
special cases) on both GEMM paths, every weight type and activation."""
import numpy as np
import pytest

import oracle
import quantized_expert_layer_amd as q
import synth
from tests.gpu_util import assert_layer_close, case, dev, host

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- dequant (Algorithm 1)
@pytest.mark.parametrize("wtype,group,coverage", [("int4", 0, True), ("int4", 128, True),
                                                  ("int8", 0, True), ("int8", 128, True),
                                                  ("int4", 0, False), ("int8", 0, False)])
def test_dequant_bit_exact(wtype, group, coverage):
    case(f"dequant {wtype} g={group} coverage={coverage}")
    cfg = synth.LayerConfig("dq", 11, d=384, inter=256, E=3, k=1, act="relu", wtypes=(wtype,),
                            group=group, gate_mode="topk", zipf_bias=False, T_list=(1,))
    inp = synth.make_inputs(cfg, 1, wtype=wtype, coverage=coverage)
    for codes, scales in ((inp.codes1, inp.scales1), (inp.codes2, inp.scales2)):
        E, K, N = codes.shape
        out = q.moe_dequant(dev(q.moe_pack_wq(codes, wtype)), dev(scales), wtype, group, E, K, N)
        ref = oracle.dequant_algorithm1(codes, scales, group)
        assert np.array_equal(host(out).view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("wtype", ["int4", "int8"])
def test_dequant_unit_scale_reproduces_every_code(wtype):
    # s = 1: W_dq == code for every code value at every position in the word
    case(f"dequant unit scale {wtype}")
    lo, hi = (-8, 8) if wtype == "int4" else (-128, 128)
    K, N = 256, 32
    codes = ((np.arange(K * N).reshape(1, K, N) % (hi - lo)) + lo).astype(np.int8)
    scales = np.ones((1, 1, N), np.float16)
    out = q.moe_dequant(dev(q.moe_pack_wq(codes, wtype)), dev(scales), wtype, 0, 1, K, N)
    assert np.array_equal(host(out).astype(np.float64), codes.astype(np.float64))


def test_dequant_hand_worked_products(golden_dir):
    # the golden products (ties to even, subnormal scales) through the GPU's fp16 multiply
    rows = []
    for line in open(f"{golden_dir}/algorithm1_products.txt"):
        line = line.split("#", 1)[0].split()
        if line:
            rows.append((int(line[0], 16), int(line[1]), int(line[2], 16)))
    N = 16
    codes = np.zeros((1, 128, N), np.int8)
    scales = np.ones((1, 1, N), np.float16)
    for n, (sb, c, _) in enumerate(rows):
        codes[0, 0, n] = c
        scales[0, 0, n] = np.array([sb], np.uint16).view(np.float16)[0]
    case("dequant golden products")
    out = host(q.moe_dequant(dev(q.moe_pack_wq(codes, "int8")), dev(scales), "int8", 0, 1, 128, N))
    got = out.view(np.uint16)[0, 0]
    for n, (_, _, eb) in enumerate(rows):
        assert got[n] == eb, (n, hex(got[n]), hex(eb))


# ---------------------------------------------------------------- grouped GEMM
def _gemm_case(E, K, N, wtype, group, T, k, seed, skew=True):
    rng = np.random.default_rng(seed)
    codes, scales = synth.gen.make_expert_weights(E, K, N, wtype, group, seed)
    ids = synth.gen.random_ids(T, k, E, seed=seed, skew=skew)
    _, _, off = oracle.stable_expert_sort(ids, E)
    a = rng.standard_normal((T * k, K)).astype(np.float16)
    return codes, scales, off, a


GEMM_CASES = [
    # E, K, N, wtype, group, T, k
    (8, 128, 256, "int4", 0, 16, 2),
    (32, 1024, 512, "int4", 0, 300, 1),
    (32, 1024, 512, "int8", 0, 300, 1),
    (60, 256, 352, "int4", 128, 17, 4),
    (60, 256, 352, "int4", 128, 200, 4),
    (16, 512, 160, "int8", 128, 70, 2),
    (5, 384, 96, "int4", 128, 1, 2),
    (3, 256, 48, "int4", 0, 333, 1),
]


PATHS = [(q.PATH_STREAM, q.TILE_AUTO), (q.PATH_TILE, q.TILE_64x256),
         (q.PATH_TILE, q.TILE_64x128), (q.PATH_TILE, q.TILE_128x128),
         (q.PATH_TILE, q.TILE_48x256), (q.PATH_TILE, q.TILE_48x128)]

# expert row counts hitting every specialised body of the tile kernel (1, 2, 3, 4, 6 and all
# 16-row subtiles, as whole tiles and as the ragged last tile of a larger expert), an empty
# expert and a full 128-row tile
SUBTILE_COUNTS = [1, 16, 17, 32, 33, 40, 47, 48, 49, 64, 0, 65, 97, 110, 128, 150, 176, 129]


@pytest.mark.parametrize("path,tile", PATHS[1:])
@pytest.mark.parametrize("wtype,group,act", [("int4", 128, "swiglu"), ("int8", 0, "relu"),
                                             ("fp16", 0, "none"), ("fp16", 0, "swiglu")])
def test_tile_bodies_for_every_subtile_count(wtype, group, act, path, tile):
    # (the grid here is small, so fp16 weights run with the K stages split over 2 or 4 wave
    # groups of the block)
    E, K, N = len(SUBTILE_COUNTS), 256, 128
    counts = np.array(SUBTILE_COUNTS)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(off[-1])
    rng = np.random.default_rng(5)
    a = rng.standard_normal((R, K)).astype(np.float16)
    if wtype == "fp16":
        codes = (rng.standard_normal((E, K, N)) * 0.05).astype(np.float16)
        scales, wdq = None, codes
    else:
        codes, scales = synth.gen.make_expert_weights(E, K, N, wtype, group, seed=9)
        wdq = oracle.dequant_algorithm1(codes, scales, group)
    case(f"gemm subtile counts {wtype} g={group} {act} tile={tile}")
    out = q.moe_grouped_gemm_wq(dev(a), dev(off), E, K, N, dev(q.moe_pack_wq(codes, wtype)),
                                None if scales is None else dev(scales), wtype, group, act,
                                path=path, tile=tile)
    ref = oracle.grouped_gemm(a, off, wdq if wtype != "fp16" else wdq.astype(np.float64), act)
    assert_layer_close(host(out), ref, "subtile counts")


@pytest.mark.parametrize("path,tile", PATHS)
@pytest.mark.parametrize("act", ["none", "relu", "swiglu"])
@pytest.mark.parametrize("E,K,N,wtype,group,T,k", GEMM_CASES)
def test_grouped_gemm_matches_oracle(E, K, N, wtype, group, T, k, act, path, tile):
    if act == "swiglu" and N % 32:
        pytest.skip("SwiGLU needs an even number of 16-column blocks")
    codes, scales, off, a = _gemm_case(E, K, N, wtype, group, T, k, seed=E * K + N)
    R = a.shape[0]
    rs = np.random.default_rng(3).random(R, dtype=np.float32)
    case(f"gemm E={E} K={K} N={N} {wtype} g={group} T={T} k={k} act={act} path={path} tile={tile}")
    out = q.moe_grouped_gemm_wq(dev(a), dev(off), E, K, N, dev(q.moe_pack_wq(codes, wtype)),
                                dev(scales), wtype, group, act, row_scale=dev(rs), path=path,
                                tile=tile)
    wdq = oracle.dequant_algorithm1(codes, scales, group)
    ref = oracle.grouped_gemm(a, off, wdq, act, row_scale=rs)
    assert_layer_close(host(out), ref, "grouped gemm")


NATIVE_TILES = [q.TILE_48x256, q.TILE_48x128, q.TILE_64x128, q.TILE_64x256]


@pytest.mark.parametrize("tile", NATIVE_TILES)
@pytest.mark.parametrize("wtype", ["int4", "int8"])
def test_native_i2f_equals_exponent_construction(wtype, tile):
    # [W] section 3 (optimized I2F): the exponent-of-1024 construction and the conversion
    # instructions give the same fp16 code values, so the GEMMs agree bit for bit; both against
    # the oracle.  Expert row counts: SUBTILE_COUNTS (every subtile body, ragged tails, an empty
    # expert); per-channel scales, the MT encoder's ReLU GEMM and its gate-weighted second GEMM.
    E, K, N = len(SUBTILE_COUNTS), 512, 256
    counts = np.array(SUBTILE_COUNTS)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(off[-1])
    rng = np.random.default_rng(21)
    a = rng.standard_normal((R, K)).astype(np.float16)
    rs = rng.random(R, dtype=np.float32)
    codes, scales = synth.gen.make_expert_weights(E, K, N, wtype, 0, seed=23, coverage=True)
    wdq = oracle.dequant_algorithm1(codes, scales, 0)
    w = dev(q.moe_pack_wq(codes, wtype))
    for act, row_scale in (("relu", None), ("none", rs)):
        case(f"native i2f {wtype} tile={tile} act={act}")
        outs = [host(q.moe_grouped_gemm_wq(dev(a), dev(off), E, K, N, w, dev(scales), wtype, 0,
                                           act, row_scale=None if row_scale is None else
                                           dev(row_scale), path=q.PATH_TILE, tile=tile, i2f=i2f))
                for i2f in ("trick", "native")]
        assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16))
        ref = oracle.grouped_gemm(a, off, wdq, act, row_scale=row_scale)
        assert_layer_close(outs[1], ref, "native i2f gemm")


@pytest.mark.parametrize("split", [2, 3, 4, 5, 8])
def test_stream_split_k_matches_oracle_and_unsplit(split):
    # K = 2048 is 16 int4 super-blocks: splits 3 and 5 leave a short last slice, 8 gives
    # slices of 2 (shorter than the 8-deep load ring)
    E, K, N = 4, 2048, 256
    codes, scales, off, a = _gemm_case(E, K, N, "int4", 128, 3, 2, seed=split)
    w = dev(q.moe_pack_wq(codes, "int4"))
    wdq = oracle.dequant_algorithm1(codes, scales, 128)
    for act in ("relu", "swiglu"):
        case(f"split-k S={split} act={act}")
        o1 = host(q.moe_grouped_gemm_wq(dev(a), dev(off), E, K, N, w, dev(scales), "int4", 128,
                                        act, path=q.PATH_STREAM, split_k=1))
        oS = host(q.moe_grouped_gemm_wq(dev(a), dev(off), E, K, N, w, dev(scales), "int4", 128,
                                        act, path=q.PATH_STREAM, split_k=split))
        ref = oracle.grouped_gemm(a, off, wdq, act)
        assert_layer_close(oS, ref, "split")
        assert_layer_close(o1, ref, "unsplit")


@pytest.mark.parametrize("path,tile", PATHS)
@pytest.mark.parametrize("wtype,group", [("int4", 0), ("int4", 128), ("int8", 0), ("int8", 128)])
def test_one_hot_rows_reproduce_dequantized_weight_rows(wtype, group, path, tile):
    # a one-hot row i of expert e gives exactly W_dq[e, i, :] (pins packing, nibble order,
    # scale indexing and the fragment layout inside the fused kernel)
    E, K, N = 3, 256, 64
    codes, scales = synth.gen.make_expert_weights(E, K, N, wtype, group, seed=77, coverage=True)
    rows = [np.arange(0, K, 3), np.arange(1, K, 5), np.arange(2, K, 2)]   # ragged row counts
    a = np.concatenate([np.eye(K, dtype=np.float16)[r] for r in rows])
    off = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    case(f"one-hot {wtype} g={group} path={path} tile={tile}")
    out = host(q.moe_grouped_gemm_wq(dev(a), dev(off), E, K, N, dev(q.moe_pack_wq(codes, wtype)),
                                     dev(scales), wtype, group, "none", path=path, tile=tile))
    wdq = oracle.dequant_algorithm1(codes, scales, group)
    ref = np.concatenate([wdq[e][r] for e, r in enumerate(rows)])
    assert np.array_equal(out.view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("K", [256, 128, 384])
@pytest.mark.parametrize("path,tile", PATHS)
def test_fp16_weights_and_zero_row_experts(path, tile, K):
    # fp16 stages are 64 rows of K: 256 gives 4 stages, which the small grid splits over 4 wave
    # groups (2 for the larger tiles); 128 (2 stages) and 384 (6) do not divide by 4 and fall
    # back to 2 groups
    E, N, T = 6, 128, 40
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((E, K, N)) * 0.05).astype(np.float16)
    off = np.array([0, 0, 17, 17, 17, 40, 40], np.int32)      # experts 0, 2, 3, 5 have no rows
    a = rng.standard_normal((T, K)).astype(np.float16)
    for act in ("none", "swiglu"):
        case(f"fp16 weights act={act} path={path} tile={tile} K={K}")
        out = q.moe_grouped_gemm_wq(dev(a), dev(off), E, K, N, dev(q.moe_pack_wq(w, "fp16")), None,
                                    "fp16", 0, act, path=path, tile=tile)
        ref = oracle.grouped_gemm(a, off, w.astype(np.float64), act)
        assert_layer_close(host(out), ref, "fp16 gemm")


@pytest.mark.parametrize("R", [288, 100, 1])
@pytest.mark.parametrize("act", ["none", "relu", "swiglu"])
def test_dense_fp16_expert_small_grid(R, act):
    # one dense fp16 expert (E = 1, the shared experts' form) on a grid of a few tiles: without
    # SwiGLU it runs 64x64 tiles, with SwiGLU 64x128; both column-group major, K split over
    # wave groups; ragged last m-tile at R = 100, a single row at R = 1
    K, N = 512, 512
    rng = np.random.default_rng(R)
    w = (rng.standard_normal((1, K, N)) * 0.05).astype(np.float16)
    a = rng.standard_normal((R, K)).astype(np.float16)
    off = np.array([0, R], np.int32)
    case(f"dense fp16 E=1 R={R} act={act}")
    out = q.moe_grouped_gemm_wq(dev(a), dev(off), 1, K, N, dev(q.moe_pack_wq(w, "fp16")), None,
                                "fp16", 0, act, path=2)
    ref = oracle.grouped_gemm(a, off, w.astype(np.float64), act)
    assert_layer_close(host(out), ref, "dense fp16 gemm")


def test_gemm_rows_beyond_offsets_are_untouched():
    E, K, N = 2, 128, 32
    codes, scales, _, a = _gemm_case(E, K, N, "int4", 0, 20, 1, seed=4)
    off = np.array([0, 5, 12], np.int32)                       # rows 12..19 belong to no expert
    import torch
    out = torch.full((20, N), 7.0, dtype=torch.float16, device="cuda")
    case("gemm rows beyond offsets")
    q.moe_grouped_gemm_wq(dev(a), dev(off), E, K, N, dev(q.moe_pack_wq(codes, "int4")),
                          dev(scales), "int4", 0, "relu", out=out)
    assert (host(out)[12:] == 7.0).all()


@pytest.mark.parametrize("path,tile", PATHS)
@pytest.mark.parametrize("act", ["relu", "swiglu"])
def test_row_mapped_gemm_gathers_and_scatters(path, tile, act):
    """moe_grouped_gemm_wq_rows: row p reads a[a_rows[p] // div] and writes out[out_rows[p]]
    ([W] section 3 workflow's permute and unpermute folded into the GEMM's loads and stores)."""
    import torch
    E, K, N, T, k = 12, 512, 256, 150, 3
    codes, scales, off, _ = _gemm_case(E, K, N, "int4", 128, T, k, seed=77)
    R = T * k
    rng = np.random.default_rng(78)
    x = rng.standard_normal((T, K)).astype(np.float16)
    ids = synth.gen.random_ids(T, k, E, seed=77, skew=True)
    perm, _, off = oracle.stable_expert_sort(ids, E)
    rs = rng.random(R, dtype=np.float32)
    wdq = oracle.dequant_algorithm1(codes, scales, 128)
    ref = oracle.grouped_gemm(oracle.permute_rows(x, perm, k), off, wdq, act, row_scale=rs)
    w = dev(q.moe_pack_wq(codes, "int4"))
    case(f"row-mapped gemm gather path={path} tile={tile} act={act}")
    got = host(q.moe_grouped_gemm_wq_rows(dev(x), dev(perm.astype(np.int32)), k, dev(off), R, E,
                                          K, N, w, dev(scales), "int4", 128, act,
                                          row_scale=dev(rs), path=path, tile=tile))
    assert_layer_close(got, ref, "gathered rows")
    # scatter: a is already permuted, the destinations are a permutation of R rows
    dst = rng.permutation(R).astype(np.int32)
    n_out = N // 2 if act == "swiglu" else N
    out = torch.full((R, n_out), float("nan"), dtype=torch.float16, device="cuda")
    case(f"row-mapped gemm scatter path={path} tile={tile} act={act}")
    q.moe_grouped_gemm_wq_rows(dev(oracle.permute_rows(x, perm, k)), None, 1, dev(off), R, E, K,
                               N, w, dev(scales), "int4", 128, act, row_scale=dev(rs), out=out,
                               out_rows=dev(dst), path=path, tile=tile)
    got = host(out)
    assert_layer_close(got[dst], ref, "scattered rows")
    # destinations outside out are skipped, the rest still land
    dst2 = dst.copy()
    dst2[::7] = -1
    dst2[1::7] = R + 5
    out2 = torch.full((R, n_out), float("nan"), dtype=torch.float16, device="cuda")
    q.moe_grouped_gemm_wq_rows(dev(oracle.permute_rows(x, perm, k)), None, 1, dev(off), R, E, K,
                               N, w, dev(scales), "int4", 128, act, row_scale=dev(rs), out=out2,
                               out_rows=dev(dst2), path=path, tile=tile)
    got2 = host(out2)
    keep = (dst2 >= 0) & (dst2 < R)
    assert_layer_close(got2[dst2[keep]], ref[keep], "scattered rows with skips")
    untouched = np.setdiff1d(np.arange(R), dst2[keep])
    assert np.isnan(got2[untouched].astype(np.float64)).all()
