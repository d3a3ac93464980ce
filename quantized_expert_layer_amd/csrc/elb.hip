// Expert lookahead buffer ("Specter" summary, Method steps, steps 2 and 3).  While the draft
// model advances, the analyzer keeps per MoE layer j and expert e the number of draft steps
// whose routing used e in layer j: ELB_cnt[j, e] = sum over steps i of [e in ELB_route[i, j]].
// At a chunk boundary the planner takes each layer's M most-counted experts as the prefetch
// plan.  Both run on the device next to the draft's routing, one block per layer.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// One draft step: counts[j][e] += 1 for every expert e that appears among layer j's T*k ids.
// Membership is marked in LDS (several tokens choosing e mark it once), then added.
__global__ __launch_bounds__(256) void elb_accumulate_kernel(const int32_t* __restrict__ ids,
                                                             int n, int E,
                                                             int32_t* __restrict__ counts) {
    __shared__ int used[MOE_MAX_EXPERTS];
    const int j = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x) used[e] = 0;
    __syncthreads();
    const int32_t* lid = ids + (size_t)j * n;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int e = lid[i];
        if ((unsigned)e < (unsigned)E) used[e] = 1;      // ids outside [0, E) route nowhere
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        if (used[e]) counts[(size_t)j * E + e] += 1;
}

// Top-M per layer: expert e's rank is the number of experts ahead of it in the order (count
// descending, index ascending); ranks are distinct, so the experts with rank < M fill the M
// output slots exactly once.  All threads read the same count at a time (an LDS broadcast).
__global__ __launch_bounds__(256) void elb_top_m_kernel(const int32_t* __restrict__ counts, int E,
                                                        int M, int32_t* __restrict__ experts,
                                                        int32_t* __restrict__ top_counts) {
    __shared__ int c[MOE_MAX_EXPERTS];
    const int j = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x) c[e] = counts[(size_t)j * E + e];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int ce = c[e];
        int rank = 0;
        for (int f = 0; f < E; ++f) {
            const int cf = c[f];
            rank += (cf > ce || (cf == ce && f < e)) ? 1 : 0;
        }
        if (rank < M) {
            experts[(size_t)j * M + rank] = e;
            if (top_counts) top_counts[(size_t)j * M + rank] = ce;
        }
    }
}

hipError_t launch_elb_accumulate(const int32_t* ids, int L, int n, int E, int32_t* counts,
                                 hipStream_t stream) {
    elb_accumulate_kernel<<<L, 256, 0, stream>>>(ids, n, E, counts);
    return hipGetLastError();
}

hipError_t launch_elb_top_m(const int32_t* counts, int L, int E, int M, int32_t* experts,
                            int32_t* top_counts, hipStream_t stream) {
    elb_top_m_kernel<<<L, 256, 0, stream>>>(counts, E, M, experts, top_counts);
    return hipGetLastError();
}

}  // namespace moe
