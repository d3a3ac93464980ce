// Top-k gating ("Specter" summary, Background / MoE: the router scores every expert and only
// the k best run): one token per 16-lane row (topk_row), the routine of both the gating kernel
// and the decode step, so both select and weight bit for bit alike.
#pragma once

#include "common.hpp"

namespace moe {

// (value, index) order: larger value first, smaller index on equal values.
__device__ __forceinline__ bool route_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// ------------------------------------------------------------------------------------
// Four tokens per wave: the 16-lane row r of a wave routes one token.  Lane j of the row holds
// experts j, j + 16, j + 32, ... (PER_LANE of them).  The arg-best of each of the k rounds is an
// all-reduce inside the row by DPP row rotations by 1, 2, 4 and 8 lanes, after which every
// lane of the row holds the row's result: no cross-row traffic and no lane reads, and the four
// tokens' reductions run in the same instructions.  Max and min are exact in any order.
// ------------------------------------------------------------------------------------
template <typename Op>
__device__ __forceinline__ int row_allreduce_bits(int v, Op op) {
    v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x121, 0xF, 0xF, false));   // row_ror:1
    v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x122, 0xF, 0xF, false));   // row_ror:2
    v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x124, 0xF, 0xF, false));   // row_ror:4
    v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x128, 0xF, 0xF, false));   // row_ror:8
    return v;
}
__device__ __forceinline__ float row_max_f32(float v) {
    return __builtin_bit_cast(float, row_allreduce_bits(__builtin_bit_cast(int, v), [](int a, int b) {
        return __builtin_bit_cast(int, fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
    }));
}
__device__ __forceinline__ int row_min_i32(int v) {
    return row_allreduce_bits(v, [](int a, int b) { return a < b ? a : b; });
}
// Sum over the 16 lanes of each row in one fixed order (shifts by 1, 2, 4, 8 leave the row's
// total in its lane 15), then that lane's value for every lane of the row.
__device__ __forceinline__ float row_sum_f32(float v, int lane) {
    int b = __builtin_bit_cast(int, v);
    auto add = [](int a, int c) {
        return __builtin_bit_cast(int, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, c));
    };
    b = add(b, __builtin_amdgcn_update_dpp(0, b, 0x111, 0xF, 0xF, false));   // row_shr:1
    b = add(b, __builtin_amdgcn_update_dpp(0, b, 0x112, 0xF, 0xF, false));   // row_shr:2
    b = add(b, __builtin_amdgcn_update_dpp(0, b, 0x114, 0xF, 0xF, false));   // row_shr:4
    b = add(b, __builtin_amdgcn_update_dpp(0, b, 0x118, 0xF, 0xF, false));   // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(b, 15), r1 = __builtin_amdgcn_readlane(b, 31);
    const int r2 = __builtin_amdgcn_readlane(b, 47), r3 = __builtin_amdgcn_readlane(b, 63);
    const int row = lane >> 4;
    return __builtin_bit_cast(float, row == 0 ? r0 : row == 1 ? r1 : row == 2 ? r2 : r3);
}

// Row r of the wave routes the token whose E logits start at `row` (may be NULL for a row with
// no token: it routes nothing and returns e = -1).  Lane j < k of the row receives choice j:
// its expert (out_e) and gate weight (out_w).  Selection in the order (value desc, index asc),
// NaN as -inf (+0 and -0 compare equal); softmax over the k chosen logits, or over all E
// (gate_all) keeping the k chosen entries; fp32, exp(l - m) / sum with m the largest logit.
template <int PER_LANE>
__device__ __forceinline__ void topk_row(const float* row, int E, int k, int gate_all, int lane,
                                         int& out_e, float& out_w) {
    const int j16 = lane & 15;
    float v[PER_LANE];
    bool taken[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int e = j16 + 16 * i;
        float x = (row && e < E) ? row[e] : -__builtin_inff();
        if (x != x) x = -__builtin_inff();
        v[i] = x;
        taken[i] = (e >= E);
    }
    float sel_v[MOE_MAX_TOPK];
    int sel_e[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        if (j >= k) break;
        float bv = -__builtin_inff();
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const int e = j16 + 16 * i;
            if (!taken[i] && route_before(v[i], e, bv, be)) { bv = v[i]; be = e; }
        }
        const float rm = row_max_f32(bv);
        be = row_min_i32(bv == rm ? be : 0x7fffffff);
        sel_v[j] = rm;
        sel_e[j] = be;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i)
            if (j16 + 16 * i == be) taken[i] = true;
    }
    const float m = sel_v[0];
    float denom = 0.0f;
    if (gate_all) {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i)
            if (j16 + 16 * i < E) part += expf(v[i] - m);
        denom = row_sum_f32(part, lane);
    } else {
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK; ++j)
            if (j < k) denom += expf(sel_v[j] - m);
    }
    float my_v = sel_v[0];
    int my_e = sel_e[0];
#pragma unroll
    for (int j = 1; j < MOE_MAX_TOPK; ++j)
        if (j < k && j16 == j) { my_v = sel_v[j]; my_e = sel_e[j]; }
    out_e = row ? my_e : -1;
    out_w = row ? expf(my_v - m) / denom : 0.0f;
}

}  // namespace moe
