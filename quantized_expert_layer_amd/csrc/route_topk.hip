// Top-k gating over fp32 router logits ("Specter" summary, Background / MoE: the router
// scores every expert and only the k best run).  One token per 16-lane row.
#include "common.hpp"
#include "launch.hpp"
#include "route.hpp"

namespace moe {

// Four tokens per wave (topk_row).  active (nullable): a token with active[t] == 0 is finished ("Who Says Elephants Can't Run",
// Fig. 1 and the optimizations table: batch pruning drops finished sentences from the
// computation); it gets ids -1 and weights 0, which the sort drops, so it takes no expert.
template <int PER_LANE>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         const uint8_t* __restrict__ active,
                                                         int T, int E, int k, int gate_all,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ wts) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t0 = (blockIdx.x * (blockDim.x / kWave) + (int)(threadIdx.x / kWave)) * 4;
    if (t0 >= T) return;                                   // wave-uniform
    const int t = t0 + (lane >> 4);
    const bool live = t < T && (!active || active[t]);
    int e;
    float w;
    topk_row<PER_LANE>(live ? logits + (size_t)t * E : nullptr, E, k, gate_all, lane, e, w);
    if (t < T && (lane & 15) < k) {
        ids[(size_t)t * k + (lane & 15)] = e;
        wts[(size_t)t * k + (lane & 15)] = w;
    }
}

hipError_t launch_route_topk(const float* logits, const uint8_t* active, int T, int E, int k,
                             int gate_all, int32_t* ids, float* wts, hipStream_t stream) {
    const int tokens_per_block = 16;                       // 4 waves x 4 rows
    const dim3 grid((T + tokens_per_block - 1) / tokens_per_block), block(256);
    if (E <= 16)
        route_topk_kernel<1><<<grid, block, 0, stream>>>(logits, active, T, E, k, gate_all, ids,
                                                           wts);
    else if (E <= 64)
        route_topk_kernel<4><<<grid, block, 0, stream>>>(logits, active, T, E, k, gate_all, ids,
                                                           wts);
    else if (E <= 128)
        route_topk_kernel<8><<<grid, block, 0, stream>>>(logits, active, T, E, k, gate_all, ids,
                                                           wts);
    else
        route_topk_kernel<16><<<grid, block, 0, stream>>>(logits, active, T, E, k, gate_all, ids,
                                                            wts);
    return hipGetLastError();
}

}  // namespace moe
