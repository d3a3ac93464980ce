"""GPU parity of the expert lookahead buffer ("Specter" summary, Method steps, steps 2 and 3):
per-layer counts of the draft steps that used each expert, and each layer's top-M experts,
bit-exact against the oracle."""
import numpy as np
import pytest

import oracle
import quantized_expert_layer_amd as q
import synth
from tests.gpu_util import case, dev, host

pytestmark = pytest.mark.gpu


def _draft_ids(cfg_name, L, K, T):
    """Seeded draft routing of K steps, L layers and T tokens: ids int32 [K, L, T, k] from the
    shape's router logits (its Zipf skew), routed on the device by moe_route_topk."""
    cfg = synth.get_config(cfg_name)
    inp = synth.make_inputs(cfg, K * L * T, with_weights=False)
    ids, _ = q.moe_route_topk(dev(inp.logits), cfg.k, cfg.gate_mode)
    return ids.reshape(K, L, T, cfg.k).contiguous(), cfg.E


# (routing shape, MoE layers, draft steps K, tokens per step, finished fraction)
CASES = [
    ("qwen15_moe", 24, 16, 1, 0.0),     # one request, K* = 16, 24 MoE layers
    ("dsv2_lite", 26, 8, 32, 0.2),      # a batch of 32 requests, some finished (ids -1)
    ("phi35_moe", 32, 16, 1, 0.0),
]


@pytest.mark.parametrize("name,L,K,T,finished", CASES)
def test_elb_counts_and_top_m_match_oracle(name, L, K, T, finished):
    import torch

    ids, E = _draft_ids(name, L, K, T)
    if finished:
        fin = np.random.default_rng(L).random(T) < finished
        ids[:, :, torch.from_numpy(fin).cuda()] = -1
    case(f"elb {name} L={L} K={K} T={T}")
    counts = torch.zeros((L, E), dtype=torch.int32, device="cuda")
    want = np.zeros((L, E), dtype=np.int64)
    ids_h = host(ids)
    for i in range(K):
        q.moe_elb_accumulate(ids[i].contiguous(), E, counts)
        want = oracle.elb_accumulate(want, ids_h[i], E)
        assert np.array_equal(host(counts), want), i
    for M in sorted({1, 4, 8, E // 2, E}):
        ex, cn = q.moe_elb_top_m(counts, M)
        wex, wcn = oracle.elb_top_m(want, M)
        assert np.array_equal(host(ex), wex) and np.array_equal(host(cn), wcn), M
    work = (want > 0).sum(axis=1).mean()
    print(f"[gpu-case] elb {name}: {work:.1f} experts per layer after {K} draft steps", flush=True)


def test_elb_edges_many_experts_ties_and_null_outputs():
    """E = 256 with k = 8 and heavy count ties; M = E; top_counts NULL; a step with T = 0."""
    import ctypes

    import torch

    rng = np.random.default_rng(3)
    L, E, k, T = 3, 256, 8, 64
    counts = torch.zeros((L, E), dtype=torch.int32, device="cuda")
    want = np.zeros((L, E), dtype=np.int64)
    for i in range(5):
        ids_h = rng.integers(-1, E, size=(L, T, k)).astype(np.int32)
        q.moe_elb_accumulate(dev(ids_h), E, counts)
        want = oracle.elb_accumulate(want, ids_h, E)
    empty = torch.empty((L, 0, k), dtype=torch.int32, device="cuda")
    q.moe_elb_accumulate(empty, E, counts)                      # adds nothing
    case("elb edges")
    assert np.array_equal(host(counts), want)
    ex, cn = q.moe_elb_top_m(counts, E)
    wex, wcn = oracle.elb_top_m(want, E)
    assert np.array_equal(host(ex), wex) and np.array_equal(host(cn), wcn)
    assert all(sorted(row) == list(range(E)) for row in host(ex))   # a permutation per layer
    ex1 = torch.full((L, 7), -5, dtype=torch.int32, device="cuda")
    st = q.lib().moe_elb_top_m(ctypes.c_void_p(counts.data_ptr()), L, E, 7,
                               ctypes.c_void_p(ex1.data_ptr()), None, None)
    assert st == 0
    torch.cuda.synchronize()
    assert np.array_equal(host(ex1), oracle.elb_top_m(want, 7)[0])
