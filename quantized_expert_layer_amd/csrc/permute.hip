// Token routing by a stable sort keyed on expert index, then the activation permute
// ("Who Says Elephants Can't Run", section 3 workflow: the row index is attached to the
// gating output, the tuples are sorted by expert_idx, the activations are permuted).
//
// The sort itself is sort_block (one workgroup of 16 waves, ballot-matched counting sort).
#include "common.hpp"
#include "launch.hpp"
#include "sort.hpp"

namespace moe {

constexpr int kSortLdsKeys = 16384;     // keys staged in LDS when R fits (64 KB)

// KEYS_IN_LDS: all R keys are first copied to LDS with one coalesced pass, so the two walks
// of the sort read LDS instead of issuing one dependent global load per 64-key chunk.
template <bool KEYS_IN_LDS>
__global__ __launch_bounds__(1024) void sort_kernel(const int32_t* __restrict__ ids,
                                                    const float* __restrict__ wts, int R, int E,
                                                    int32_t* __restrict__ perm,
                                                    int32_t* __restrict__ inv_perm,
                                                    int32_t* __restrict__ offsets,
                                                    float* __restrict__ w_perm) {
    __shared__ int keys[KEYS_IN_LDS ? kSortLdsKeys : 1];
    if constexpr (KEYS_IN_LDS) {
        for (int i = threadIdx.x; i < R; i += blockDim.x) keys[i] = ids[i];
    }
    auto key_of = [&](int f) -> int {
        if constexpr (KEYS_IN_LDS) return keys[f];
        else return ids[f];
    };
    sort_block(R, E, key_of, [&](int f) { return wts[f]; }, perm, inv_perm, offsets, w_perm);
}

// x_perm[p] = x[perm[p] / k], 16 bytes per thread; rows with perm < 0 are zero-filled.
// The caller guarantees R * d/8 < 2^32 so that 32-bit index math is exact.
__global__ __launch_bounds__(256) void gather_kernel(const u32x4* __restrict__ x,
                                                     const int32_t* __restrict__ perm,
                                                     uint32_t total, int k, uint32_t d16,
                                                     u32x4* __restrict__ xp) {
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += gridDim.x * blockDim.x) {
        const uint32_t p = i / d16;
        const uint32_t c = i - p * d16;
        const int f = perm[p];
        u32x4 v = {0u, 0u, 0u, 0u};
        if (f >= 0) v = x[(size_t)(f / k) * d16 + c];
        xp[i] = v;
    }
}

hipError_t launch_sort(const int32_t* ids, const float* wts, int R, int E, int32_t* perm,
                       int32_t* inv_perm, int32_t* offsets, float* w_perm, hipStream_t stream) {
    if (R <= kSortLdsKeys)
        sort_kernel<true><<<1, kSortWaves * kWave, 0, stream>>>(ids, wts, R, E, perm, inv_perm,
                                                                offsets, w_perm);
    else
        sort_kernel<false><<<1, kSortWaves * kWave, 0, stream>>>(ids, wts, R, E, perm, inv_perm,
                                                                 offsets, w_perm);
    return hipGetLastError();
}

hipError_t launch_gather(const uint16_t* x, const int32_t* perm, int R, int k, int d,
                         uint16_t* x_perm, hipStream_t stream) {
    const uint32_t d16 = (uint32_t)d / 8u;
    const uint32_t total = (uint32_t)R * d16;
    const uint32_t want = (total + 255u) / 256u;
    const int grid = (int)(want < 8192u ? want : 8192u);
    gather_kernel<<<grid, 256, 0, stream>>>((const u32x4*)x, perm, total, k, d16,
                                            (u32x4*)x_perm);
    return hipGetLastError();
}

}  // namespace moe
