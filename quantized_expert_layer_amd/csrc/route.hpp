// Top-k gating of one token by one wave ("Specter" summary, Background / MoE: the router
// scores every expert and only the k best run).  Shared by the gating kernel and the fused
// decode-step kernel, so both select and weight bit for bit alike.
#pragma once

#include "common.hpp"

namespace moe {

// (value, index) order: larger value first, smaller index on equal values.
__device__ __forceinline__ bool route_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// One wave, row = the token's E logits.  Lane j < k receives choice j: its expert (out_e) and
// gate weight (out_w).  Softmax over the k chosen logits, or over all E (gate_all) keeping the
// k chosen entries; fp32, exp(l - m) / sum with m the largest logit.  NaN orders as -inf.
template <int PER_LANE>
__device__ __forceinline__ void topk_token(const float* row, int E, int k, int gate_all,
                                           int lane, int& out_e, float& out_w) {
    float v[PER_LANE];
    bool taken[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int e = lane + i * kWave;
        float x = (e < E) ? row[e] : -__builtin_inff();
        if (x != x) x = -__builtin_inff();
        v[i] = x;
        taken[i] = (e >= E);
    }

    float sel_v[MOE_MAX_TOPK];
    int sel_e[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        if (j >= k) break;
        // best untaken candidate of this lane
        float bv = -__builtin_inff();
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const int e = lane + i * kWave;
            if (!taken[i] && route_before(v[i], e, bv, be)) { bv = v[i]; be = e; }
        }
        // wave arg-best (butterfly: every lane ends with the same winner)
#pragma unroll
        for (int s = 1; s < kWave; s <<= 1) {
            const float ov = __shfl_xor(bv, s, kWave);
            const int oe = __shfl_xor(be, s, kWave);
            if (route_before(ov, oe, bv, be)) { bv = ov; be = oe; }
        }
        sel_v[j] = bv;
        sel_e[j] = be;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i)
            if (lane + i * kWave == be) taken[i] = true;
    }

    const float m = sel_v[0];
    float denom = 0.0f;
    if (gate_all) {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i)
            if (lane + i * kWave < E) part += expf(v[i] - m);
#pragma unroll
        for (int s = 1; s < kWave; s <<= 1) part += __shfl_xor(part, s, kWave);
        denom = part;
    } else {
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK; ++j)
            if (j < k) denom += expf(sel_v[j] - m);
    }
    float my_v = sel_v[0];
    int my_e = sel_e[0];
#pragma unroll
    for (int j = 1; j < MOE_MAX_TOPK; ++j)
        if (j < k && lane == j) { my_v = sel_v[j]; my_e = sel_e[j]; }
    out_e = my_e;
    out_w = expf(my_v - m) / denom;
}

}  // namespace moe
