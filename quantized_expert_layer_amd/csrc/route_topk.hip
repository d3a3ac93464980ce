// Top-k gating over fp32 router logits ("Specter" summary, Background / MoE: the router
// scores every expert and only the k best run).  One wave per token.
#include "common.hpp"
#include "launch.hpp"
#include "route.hpp"

namespace moe {

// active (nullable): a token with active[t] == 0 is finished ("Who Says Elephants Can't Run",
// Fig. 1 and the optimizations table: batch pruning drops finished sentences from the
// computation); it gets ids -1 and weights 0, which the sort drops, so it takes no expert.
template <int PER_LANE>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         const uint8_t* __restrict__ active,
                                                         int T, int E, int k, int gate_all,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ wts) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (t >= T) return;
    if (active && !active[t]) {
        if (lane < k) {
            ids[(size_t)t * k + lane] = -1;
            wts[(size_t)t * k + lane] = 0.0f;
        }
        return;
    }
    int e;
    float w;
    topk_token<PER_LANE>(logits + (size_t)t * E, E, k, gate_all, lane, e, w);
    if (lane < k) {
        ids[(size_t)t * k + lane] = e;
        wts[(size_t)t * k + lane] = w;
    }
}

hipError_t launch_route_topk(const float* logits, const uint8_t* active, int T, int E, int k,
                             int gate_all, int32_t* ids, float* wts, hipStream_t stream) {
    const int tokens_per_block = 4;
    const dim3 grid((T + tokens_per_block - 1) / tokens_per_block), block(256);
    if (E <= 64)
        route_topk_kernel<1><<<grid, block, 0, stream>>>(logits, active, T, E, k, gate_all, ids,
                                                           wts);
    else if (E <= 128)
        route_topk_kernel<2><<<grid, block, 0, stream>>>(logits, active, T, E, k, gate_all, ids,
                                                           wts);
    else
        route_topk_kernel<4><<<grid, block, 0, stream>>>(logits, active, T, E, k, gate_all, ids,
                                                           wts);
    return hipGetLastError();
}

}  // namespace moe
