// Top-k gating over fp32 router logits ("Specter" summary, Background / MoE: the router
// scores every expert and only the k best run).  One wave per token.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// (value, index) order: larger value first, smaller index on equal values.
__device__ __forceinline__ bool before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

template <int PER_LANE>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int T, int E, int k, int gate_all,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ wts) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (t >= T) return;
    const float* row = logits + (size_t)t * E;

    float v[PER_LANE];
    bool taken[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int e = lane + i * kWave;
        float x = (e < E) ? row[e] : -__builtin_inff();
        if (x != x) x = -__builtin_inff();      // NaN is ordered as -inf
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
            if (!taken[i] && before(v[i], e, bv, be)) { bv = v[i]; be = e; }
        }
        // wave arg-best (butterfly: every lane ends with the same winner)
#pragma unroll
        for (int s = 1; s < kWave; s <<= 1) {
            const float ov = __shfl_xor(bv, s, kWave);
            const int oe = __shfl_xor(be, s, kWave);
            if (before(ov, oe, bv, be)) { bv = ov; be = oe; }
        }
        sel_v[j] = bv;
        sel_e[j] = be;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i)
            if (lane + i * kWave == be) taken[i] = true;
    }

    // gate weights, fp32: exp(l - m) / sum, m = the largest logit (= sel_v[0])
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
    if (lane < k) {
        float my_v = sel_v[0];
        int my_e = sel_e[0];
#pragma unroll
        for (int j = 1; j < MOE_MAX_TOPK; ++j)
            if (j < k && lane == j) { my_v = sel_v[j]; my_e = sel_e[j]; }
        ids[(size_t)t * k + lane] = my_e;
        wts[(size_t)t * k + lane] = expf(my_v - m) / denom;
    }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int gate_all,
                             int32_t* ids, float* wts, hipStream_t stream) {
    const int tokens_per_block = 4;
    const dim3 grid((T + tokens_per_block - 1) / tokens_per_block), block(256);
    if (E <= 64)
        route_topk_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, k, gate_all, ids, wts);
    else if (E <= 128)
        route_topk_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, k, gate_all, ids, wts);
    else
        route_topk_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, k, gate_all, ids, wts);
    return hipGetLastError();
}

}  // namespace moe
