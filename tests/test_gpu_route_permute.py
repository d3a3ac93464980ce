"""GPU parity: top-k gating, stable sort/permute, combine (bit-exact or 1 fp16 ulp)."""
import numpy as np
import pytest

import oracle
import quantized_expert_layer_amd as q
import synth
from tests.gpu_util import assert_within_one_fp16_ulp, case, dev, host

pytestmark = pytest.mark.gpu


def _gate_tol(E):
    # fp32 gate weights: each exp is within a few ulp, a sum of up to E terms adds E * 2^-24
    # relative, the division half an ulp; weights are <= 1, so |diff| <= (E + 8) * 2^-24.
    return (E + 8) * 2.0 ** -24


ROUTE_CASES = [("tiny", 16, None), ("mt_encoder", 3840, None), ("mt_encoder", 3840, 4),
               ("qwen15_moe", 17, None), ("qwen15_moe", 544, None), ("dsv2_lite", 288, None),
               ("phi35_moe", 8192, None)]


@pytest.mark.parametrize("name,T,active", ROUTE_CASES)
def test_route_topk_matches_oracle(name, T, active):
    cfg = synth.get_config(name)
    inp = synth.make_inputs(cfg, T, active=active or 0, with_weights=False)
    for mode in ("topk", "all"):
        case(f"route_topk {name} T={T} active={active} mode={mode}")
        ids, w = q.moe_route_topk(dev(inp.logits), cfg.k, mode)
        ref_ids, ref_w = oracle.topk_route(inp.logits, cfg.k, mode)
        assert np.array_equal(host(ids), ref_ids)
        assert np.abs(host(w) - ref_w).max() <= _gate_tol(cfg.E)


@pytest.mark.parametrize("E,k", [(1, 1), (8, 8), (64, 6), (100, 3), (200, 8), (256, 2)])
def test_route_topk_tie_heavy(E, k):
    L = synth.gen.tie_heavy_logits(333, E, seed=E * 10 + k)
    for mode in ("topk", "all"):
        case(f"route_topk ties E={E} k={k} mode={mode}")
        ids, w = q.moe_route_topk(dev(L), k, mode)
        ref_ids, ref_w = oracle.topk_route(L, k, mode)
        assert np.array_equal(host(ids), ref_ids)
        assert np.abs(host(w) - ref_w).max() <= _gate_tol(E)


PERMUTE_CASES = [(16, 2, 8, 128, False), (17, 4, 60, 2048, True), (544, 4, 60, 64, True),
                 (288, 6, 64, 64, True), (1, 2, 16, 4096, False), (3840, 1, 32, 1024, True),
                 (8192, 2, 16, 64, False), (97, 8, 256, 24, True), (5, 1, 1, 8, False),
                 (2049, 3, 7, 16, True), (5000, 4, 64, 16, True)]


@pytest.mark.parametrize("T,k,E,d,skew", PERMUTE_CASES)
def test_permute_matches_oracle(T, k, E, d, skew):
    case(f"permute T={T} k={k} E={E} d={d}")
    ids = synth.gen.random_ids(T, k, E, seed=T + E, skew=skew)
    rng = np.random.default_rng(T)
    w = rng.random((T, k), dtype=np.float32)
    x = rng.standard_normal((T, d)).astype(np.float16)
    perm, inv, off, xp, wp = q.moe_permute(dev(ids), dev(w), dev(x), E)
    r_perm, r_inv, r_off = oracle.stable_expert_sort(ids, E)
    assert np.array_equal(host(perm), r_perm)
    assert np.array_equal(host(inv), r_inv)
    assert np.array_equal(host(off), r_off)
    assert np.array_equal(host(xp).view(np.uint16),
                          oracle.permute_rows(x, r_perm, k).view(np.uint16))
    assert np.array_equal(host(wp), w.ravel()[r_perm])


@pytest.mark.parametrize("T,k,E", [(600, 2, 8), (3000, 2, 40), (4096, 2, 16), (4097, 2, 16),
                                   (9000, 2, 256), (5000, 7, 8)])
def test_permute_multi_block_with_dropped_slots(T, k, E):
    """Above 1024 slots the sort runs over several blocks: ids -1 (finished tokens) and out of
    range, a skewed key mix, and block boundaries inside runs of equal keys.  Up to 8 blocks
    (8192 slots) each block counts all keys itself; 8194 slots and more take the two-launch
    form."""
    rng = np.random.default_rng(T)
    ids = synth.gen.random_ids(T, k, E, seed=T, skew=True)
    drop = rng.random((T, k)) < 0.1
    ids[drop] = -1
    ids[rng.random((T, k)) < 0.01] = E + 3
    w = rng.random((T, k), dtype=np.float32)
    x = rng.standard_normal((T, 8)).astype(np.float16)
    case(f"permute multi-block T={T} k={k} E={E}")
    _check_sort_with_drops(ids, w, x, E)


def _check_sort_with_drops(ids, w, x, E):
    """moe_permute against a stable argsort in which slots outside [0, E) sort last and are
    dropped."""
    T, k = ids.shape
    perm, inv, off, xp, wp = q.moe_permute(dev(ids), dev(w), dev(x), E)
    valid = (ids >= 0) & (ids < E)
    keys = np.where(valid, ids, E).ravel()               # dropped slots sort after every expert
    order = np.argsort(keys, kind="stable")
    n_valid = int(valid.sum())
    r_perm = np.full(T * k, -1, np.int64)
    r_perm[:n_valid] = order[:n_valid]
    r_inv = np.full(T * k, -1, np.int64)
    r_inv[order[:n_valid]] = np.arange(n_valid)
    r_off = np.concatenate([[0], np.cumsum(np.bincount(ids[valid], minlength=E))])
    assert np.array_equal(host(perm), r_perm)
    assert np.array_equal(host(inv), r_inv)
    assert np.array_equal(host(off), r_off)
    r_wp = np.zeros(T * k, np.float32)
    r_wp[:n_valid] = w.ravel()[order[:n_valid]]
    assert np.array_equal(host(wp), r_wp)
    r_xp = np.zeros((T * k, x.shape[1]), np.float16)     # rows routed nowhere are zero-filled
    r_xp[:n_valid] = x[order[:n_valid] // k]
    assert np.array_equal(host(xp).view(np.uint16), r_xp.view(np.uint16))


@pytest.mark.parametrize("T,k,E,fill", [(3000, 1, 1, None), (1000, 8, 256, None),
                                        (1024, 8, 256, None), (2000, 2, 16, -1),
                                        (3000, 2, 40, 40)])
def test_permute_multi_block_edge_cases(T, k, E, fill):
    """The multi-block sort at its corners: one expert (no key bits to match), 256 experts at
    and just below the 8192-slot edge of the one-launch form, and every slot dropped (-1, or
    ids equal to E)."""
    case(f"permute multi-block edge T={T} k={k} E={E} fill={fill}")
    if fill is None:
        ids = synth.gen.random_ids(T, k, E, seed=T + 7, skew=True)
    else:
        ids = np.full((T, k), fill, np.int32)
    rng = np.random.default_rng(T + k)
    w = rng.random((T, k), dtype=np.float32)
    x = rng.standard_normal((T, 8)).astype(np.float16)
    _check_sort_with_drops(ids, w, x, E)


def test_permute_drops_ids_out_of_range():
    case("permute out-of-range ids")
    ids = np.array([[0, 3], [7, 1], [2, -1]], np.int32)       # 7 and -1 are outside [0, 4)
    x = np.arange(3 * 8, dtype=np.float16).reshape(3, 8)
    w = np.ones((3, 2), np.float32)
    perm, inv, off, xp, wp = q.moe_permute(dev(ids), dev(w), dev(x), 4)
    assert host(off).tolist() == [0, 1, 2, 3, 4]
    assert host(perm).tolist() == [0, 3, 4, 1, -1, -1]
    assert host(inv).tolist() == [0, 3, -1, 1, 2, -1]
    assert not host(xp)[4:].any()


@pytest.mark.parametrize("T,k,d,with_w,with_add", [(16, 2, 128, True, False),
                                                   (288, 6, 2048, False, True),
                                                   (3840, 1, 1024, True, False),
                                                   (17, 4, 2048, True, True), (1, 8, 8, True, True)])
def test_combine_within_one_ulp(T, k, d, with_w, with_add):
    case(f"combine T={T} k={k} d={d}")
    rng = np.random.default_rng(T * k)
    ids = synth.gen.random_ids(T, k, max(k, 8), seed=d)
    _, inv, _ = oracle.stable_expert_sort(ids, max(k, 8))
    y = rng.standard_normal((T * k, d)).astype(np.float16)
    w = rng.random((T, k), dtype=np.float32) if with_w else None
    add = rng.standard_normal((T, d)).astype(np.float16) if with_add else None
    out = q.moe_unpermute_combine(dev(y), dev(inv), None if w is None else dev(w),
                                  None if add is None else dev(add), T, k)
    ref = oracle.unpermute_combine(y, inv, k, w=w, addend=add)
    assert_within_one_fp16_ulp(host(out), ref, "combine")
