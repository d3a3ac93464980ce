"""Seeded input generator for the MoE expert layer.

Every array is a pure function of (config, T, weight type, active-expert count,
coverage flag), drawn from numpy PCG64 streams spawned from two seed sequences: the
routing inputs (logits, Zipf permutation, x) from SeedSequence([cfg_id, 10 * A, T,
20261202]), the layer weights from SeedSequence([cfg_id, 10000 * coverage + 1, 20261202])
with one child stream per weight matrix and expert.  So the weights are the same layer for
every T, and int4, int8 and fp16 experts are one normal draw quantized (or kept) three
ways under the same routing.  Value distributions follow the layer shapes being modelled:

  * x ~ fp16(N(0, 1)), gate logits ~ fp32(N(0, 1));
  * optional skew: logit bias b_e = ln p_{pi(e)}, p_r proportional to r^-1.1
    (Zipf exponent 1.1, r = 1..E, pi a seeded permutation of the experts);
  * optional active-expert restriction A: logits of experts >= A are set to -1e30;
  * expert weights ~ N(0, 0.02^2) in fp32, stored as symmetric integer codes with fp16
    scales.  The codes come from round-to-nearest, a stand-in for the GPTQ solver named
    on the Specter page (GPTQ needs calibration data and trained weights); the format is
    the pages' one: symmetric codes, one fp16 scale per output channel, shape (E,1,N),
    as in "Who Says Elephants Can't Run" section 3, or per 128-row group along K, shape
    (E,K/128,N), the GPTQ group size the Specter page uses.  Turning codes back into
    weights is the layer's job and does not happen here;
  * weight type "fp16": the unquantized baseline, fp16 of the same draw, no scales;
  * shared experts (always on, fp16): fp16(N(0, 0.02^2)).

A "coverage" variant replaces the weight draw by codes uniform over the full code
range and scales uniform in [2^-8, 2^-4], so that every code value occurs.
"""
import concurrent.futures
import os
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

from .configs import LayerConfig

SEED_TAG = 20261202
QMAX = {"int4": 7, "int8": 127}
WTYPE_ID = {"int4": 0, "int8": 1, "fp16": 2}


@dataclass
class LayerInputs:
    cfg: LayerConfig
    T: int
    wtype: str
    active: int
    coverage: bool
    seed: Tuple[int, ...]
    x: np.ndarray            # fp16 [T, d]
    logits: np.ndarray       # fp32 [T, E]
    codes1: np.ndarray       # int8 [E, d, N1]   N1 = F (ReLU) or 2I, columns [gate | up]
    scales1: Optional[np.ndarray]  # fp16 [E, G1, N1]  G1 = 1 (per channel) or d/128
    codes2: np.ndarray       # int8 [E, F or I, d]
    scales2: Optional[np.ndarray]  # fp16 [E, G2, d]
    # wtype "fp16": codes1 / codes2 are the fp16 weights themselves and the scales are None
    # per shared expert: (w1 fp16 [d, 2*Is] with columns [gate | up], w2 fp16 [Is, d])
    shared: List[Tuple[np.ndarray, np.ndarray]] = field(default_factory=list)

    @property
    def group(self) -> int:
        return self.cfg.group


def _zipf_bias(rng: np.random.Generator, E: int) -> np.ndarray:
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** -1.1
    p /= p.sum()
    pi = rng.permutation(E)
    return np.log(p[pi]).astype(np.float32)


def _rtn_codes(w: np.ndarray, qmax: int, group: int) -> Tuple[np.ndarray, np.ndarray]:
    """Round-to-nearest symmetric codes and fp16 scales for one expert matrix w [K, N]."""
    K, N = w.shape
    if group == 0:
        amax = np.abs(w).max(axis=0, keepdims=True)                     # [1, N]
    else:
        amax = np.abs(w.reshape(K // group, group, N)).max(axis=1)      # [G, N]
    s16 = (amax / np.float32(qmax)).astype(np.float16)
    s16 = np.maximum(s16, np.float16(2.0 ** -14))
    s32 = s16.astype(np.float32)
    if group == 0:
        sfull = s32
    else:
        sfull = np.repeat(s32, group, axis=0)
    q = np.clip(np.rint(w / sfull), -qmax - 1, qmax).astype(np.int8)
    return q, s16


def _expert_mats(rngs, E, K, N, qmax, group, coverage):
    """Codes int8 [E, K, N] and fp16 scales [E, G, N]; qmax None: the fp16 weights themselves
    (same draw, unquantized) and scales None."""
    G = 1 if group == 0 else K // group
    fp16 = qmax is None
    codes = np.empty((E, K, N), dtype=np.float16 if fp16 else np.int8)
    scales = None if fp16 else np.empty((E, G, N), dtype=np.float16)

    def one(e):
        rng = rngs[e]
        if fp16:
            codes[e] = (rng.standard_normal((K, N), dtype=np.float32) * np.float32(0.02)).astype(np.float16)
        elif coverage:
            codes[e] = rng.integers(-qmax - 1, qmax + 1, size=(K, N), dtype=np.int8)
            scales[e] = rng.uniform(2.0 ** -8, 2.0 ** -4, size=(G, N)).astype(np.float16)
        else:
            w = rng.standard_normal((K, N), dtype=np.float32) * np.float32(0.02)
            codes[e], scales[e] = _rtn_codes(w, qmax, group)

    # Each expert has its own stream, so the result does not depend on the thread count.
    workers = max(1, min(E, 16, os.cpu_count() or 1))
    if workers == 1 or E * K * N < (1 << 22):
        for e in range(E):
            one(e)
    else:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(E)))
    return codes, scales


def make_inputs(cfg: LayerConfig, T: int, wtype: Optional[str] = None, active: int = 0,
                coverage: bool = False, with_weights: bool = True) -> LayerInputs:
    """Build the seeded inputs of one layer call.

    active > 0 restricts routing to experts [0, active) (the active-expert sweep).
    with_weights=False skips the weight draw (routing-only tests).
    """
    wtype = wtype or cfg.wtypes[0]
    if wtype == "fp16" and (cfg.group or coverage):
        raise ValueError("fp16 experts have no scale groups and no code coverage variant")
    # Two seed sequences: the routing inputs (logits, Zipf permutation, x) depend on the token
    # count and the active-expert restriction; the layer's weights depend on neither, nor on
    # the weight type -- int4, int8 and fp16 experts are the same normal draw, quantized (or
    # not) differently, and see the same routing.
    routing_id = 10 * active
    seed = (cfg.cfg_id, routing_id, T, SEED_TAG)
    c_logits, c_perm, c_x = np.random.SeedSequence(list(seed)).spawn(3)
    c_w1, c_w2, c_sh = np.random.SeedSequence(
        [cfg.cfg_id, 10000 * int(coverage) + 1, SEED_TAG]).spawn(3)

    rl = np.random.Generator(np.random.PCG64(c_logits))
    logits = rl.standard_normal((T, cfg.E), dtype=np.float32)
    if cfg.zipf_bias:
        logits += _zipf_bias(np.random.Generator(np.random.PCG64(c_perm)), cfg.E)[None, :]
    if active:
        logits[:, active:] = np.float32(-1e30)

    rx = np.random.Generator(np.random.PCG64(c_x))
    x = rx.standard_normal((T, cfg.d), dtype=np.float32).astype(np.float16)

    G1 = 1 if cfg.group == 0 else cfg.d // cfg.group
    G2 = 1 if cfg.group == 0 else cfg.inter // cfg.group
    if with_weights:
        qmax = None if wtype == "fp16" else QMAX[wtype]
        r1 = [np.random.Generator(np.random.PCG64(s)) for s in c_w1.spawn(cfg.E)]
        r2 = [np.random.Generator(np.random.PCG64(s)) for s in c_w2.spawn(cfg.E)]
        codes1, scales1 = _expert_mats(r1, cfg.E, cfg.d, cfg.n1, qmax, cfg.group, coverage)
        codes2, scales2 = _expert_mats(r2, cfg.E, cfg.inter, cfg.d, qmax, cfg.group, coverage)
    else:
        codes1 = np.zeros((cfg.E, 0, cfg.n1), np.int8)
        scales1 = np.zeros((cfg.E, G1, cfg.n1), np.float16)
        codes2 = np.zeros((cfg.E, 0, cfg.d), np.int8)
        scales2 = np.zeros((cfg.E, G2, cfg.d), np.float16)

    shared = []
    if cfg.n_shared and with_weights:
        for s in c_sh.spawn(cfg.n_shared):
            rs = np.random.Generator(np.random.PCG64(s))
            w1 = (rs.standard_normal((cfg.d, 2 * cfg.shared_inter), dtype=np.float32)
                  * np.float32(0.02)).astype(np.float16)
            w2 = (rs.standard_normal((cfg.shared_inter, cfg.d), dtype=np.float32)
                  * np.float32(0.02)).astype(np.float16)
            shared.append((w1, w2))

    return LayerInputs(cfg=cfg, T=T, wtype=wtype, active=active, coverage=coverage,
                       seed=seed, x=x, logits=logits, codes1=codes1, scales1=scales1,
                       codes2=codes2, scales2=scales2, shared=shared)


def make_expert_weights(E: int, K: int, N: int, wtype: str, group: int, seed: int,
                        coverage: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Codes int8 [E, K, N] and fp16 scales [E, G, N] of one weight matrix per expert (for
    single-GEMM tests), drawn like a layer's weights."""
    ss = np.random.SeedSequence([seed, E, K, N, WTYPE_ID[wtype], group, int(coverage), SEED_TAG])
    rngs = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(E)]
    return _expert_mats(rngs, E, K, N, QMAX[wtype], group, coverage)


def random_ids(T: int, k: int, E: int, seed: int = 0, skew: bool = False) -> np.ndarray:
    """Routing ids [T, k] with k distinct experts per token (for sort/permute tests)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, T, k, E, SEED_TAG])))
    p = None
    if skew:
        r = np.arange(1, E + 1, dtype=np.float64) ** -1.1
        p = r / r.sum()
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        ids[t] = rng.choice(E, size=k, replace=False, p=p)
    return ids


def tie_heavy_logits(T: int, E: int, seed: int = 0) -> np.ndarray:
    """Logits drawn from {-1, -0.0, +0.0, 1, -1e30}: many exact ties, signed zeros, masks."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, T, E, 7, SEED_TAG])))
    vals = np.array([-1.0, -0.0, 0.0, 1.0, -1e30], dtype=np.float32)
    return vals[rng.integers(0, len(vals), size=(T, E))]
