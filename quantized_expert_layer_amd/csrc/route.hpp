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

// Wave-wide reductions by DPP: row shifts by 1, 2, 4 and 8 lanes, then broadcasts of lanes 15
// and 31 into the rows after them, leave the reduction of all 64 lanes in lane 63, which every
// lane then reads.  Lanes a shift or broadcast does not reach combine with `ident`.  Max and min
// are exact in any order; the sum has this one fixed order, the same on every lane.
template <typename Op>
__device__ __forceinline__ int wave_reduce_bits(int v, int ident, Op op) {
    v = op(v, __builtin_amdgcn_update_dpp(ident, v, 0x111, 0xF, 0xF, false));   // row_shr:1
    v = op(v, __builtin_amdgcn_update_dpp(ident, v, 0x112, 0xF, 0xF, false));   // row_shr:2
    v = op(v, __builtin_amdgcn_update_dpp(ident, v, 0x114, 0xF, 0xF, false));   // row_shr:4
    v = op(v, __builtin_amdgcn_update_dpp(ident, v, 0x118, 0xF, 0xF, false));   // row_shr:8
    v = op(v, __builtin_amdgcn_update_dpp(ident, v, 0x142, 0xA, 0xF, false));   // row_bcast:15
    v = op(v, __builtin_amdgcn_update_dpp(ident, v, 0x143, 0xC, 0xF, false));   // row_bcast:31
    return __builtin_amdgcn_readlane(v, kWave - 1);
}
__device__ __forceinline__ float wave_max_f32(float v) {
    return __builtin_bit_cast(float, wave_reduce_bits(
        __builtin_bit_cast(int, v), __builtin_bit_cast(int, -__builtin_inff()), [](int a, int b) {
            return __builtin_bit_cast(int, fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
        }));
}
__device__ __forceinline__ int wave_min_i32(int v) {
    return wave_reduce_bits(v, 0x7fffffff, [](int a, int b) { return a < b ? a : b; });
}
__device__ __forceinline__ float wave_sum_f32(float v) {
    return __builtin_bit_cast(float, wave_reduce_bits(
        __builtin_bit_cast(int, v), 0, [](int a, int b) {
            return __builtin_bit_cast(int, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
        }));
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
        // wave arg-best: the largest value, then the smallest index holding it (every lane
        // ends with the same winner)
        const float wm = wave_max_f32(bv);
        be = wave_min_i32(bv == wm ? be : 0x7fffffff);
        bv = wm;
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
        denom = wave_sum_f32(part);
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
