// Token routing by a stable sort keyed on expert index, then the activation permute
// ("Who Says Elephants Can't Run", section 3 workflow: the row index is attached to the
// gating output, the tuples are sorted by expert_idx, the activations are permuted).
//
// The sort is a counting sort done by one workgroup of 16 waves.  Each wave owns a
// contiguous range of flat slots and walks it 64 slots at a time.  Lanes holding the same
// key find each other with one ballot per key bit (a wave-wide "match"), which gives every
// slot its rank among equal keys in the chunk and lets one lane per key update the wave's
// running count in LDS.  A scan over (expert, wave) turns counts into bases; a second walk
// writes perm / inv_perm.  Order inside a key is ascending slot index: stable.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kSortWaves = 16;

struct Match {
    unsigned long long peers;   // lanes holding the same valid key
    int rank;                   // number of peers below this lane
    int total;                  // number of peers
};

__device__ __forceinline__ Match wave_match(int key, bool valid, int nbits, int lane) {
    unsigned long long peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const unsigned long long ones = __ballot(bit);
        peers &= bit ? ones : ~ones;
    }
    Match m;
    m.peers = peers;
    m.rank = __popcll(peers & ((1ull << lane) - 1ull));
    m.total = __popcll(peers);
    return m;
}

constexpr int kSortLdsKeys = 16384;     // keys staged in LDS when R fits (64 KB)

// KEYS_IN_LDS: all R keys are first copied to LDS with one coalesced pass, so the two walks
// below read LDS instead of issuing one dependent global load per 64-key chunk.
template <bool KEYS_IN_LDS>
__global__ __launch_bounds__(1024) void sort_kernel(const int32_t* __restrict__ ids,
                                                    const float* __restrict__ wts, int R, int E,
                                                    int32_t* __restrict__ perm,
                                                    int32_t* __restrict__ inv_perm,
                                                    int32_t* __restrict__ offsets,
                                                    float* __restrict__ w_perm) {
    __shared__ int cnt[kSortWaves][MOE_MAX_EXPERTS];
    __shared__ int keys[KEYS_IN_LDS ? kSortLdsKeys : 1];
    __shared__ int wave_sum[4];
    __shared__ int n_valid;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    for (int i = threadIdx.x; i < kSortWaves * MOE_MAX_EXPERTS; i += blockDim.x)
        (&cnt[0][0])[i] = 0;
    if constexpr (KEYS_IN_LDS) {
        for (int i = threadIdx.x; i < R; i += blockDim.x) keys[i] = ids[i];
    }
    __syncthreads();
    auto key_of = [&](int f) -> int {
        if (f >= R) return -1;
        if constexpr (KEYS_IN_LDS) return keys[f];
        else return ids[f];
    };

    const int nbits = (E <= 1) ? 0 : 32 - __clz(E - 1);
    const int chunks = (R + kWave - 1) / kWave;
    const int per_wave = (chunks + kSortWaves - 1) / kSortWaves;
    const int c0 = wave * per_wave, c1 = min(chunks, c0 + per_wave);

    // pass 1: per-wave key counts
    for (int c = c0; c < c1; ++c) {
        const int f = c * kWave + lane;
        const int key = key_of(f);
        const bool valid = (unsigned)key < (unsigned)E;
        const Match m = wave_match(key, valid, nbits, lane);
        if (valid && m.rank == m.total - 1) cnt[wave][key] += m.total;
    }
    __syncthreads();

    // scan: bases in (expert-major, wave-minor) order.  Threads 0..255 are waves 0..3, one
    // expert per thread; the branch is uniform per wave and the barriers are block-wide.
    int tot = 0, incl = 0;
    if (threadIdx.x < 256) {
        const int e = threadIdx.x;
        if (e < E)
            for (int w = 0; w < kSortWaves; ++w) tot += cnt[w][e];
        incl = tot;
        for (int s = 1; s < kWave; s <<= 1) {
            const int v = __shfl_up(incl, s, kWave);
            if (lane >= s) incl += v;
        }
        if (lane == kWave - 1) wave_sum[wave] = incl;
    }
    __syncthreads();
    if (threadIdx.x < 256) {
        const int e = threadIdx.x;
        int before = 0;
        for (int w = 0; w < wave; ++w) before += wave_sum[w];
        const int start = before + incl - tot;
        if (e < E) {
            int run = start;
            for (int w = 0; w < kSortWaves; ++w) {
                const int c = cnt[w][e];
                cnt[w][e] = run;
                run += c;
            }
            offsets[e] = start;
            if (e == E - 1) {
                offsets[E] = run;
                n_valid = run;
            }
        }
    }
    __syncthreads();

    // pass 2: scatter
    for (int c = c0; c < c1; ++c) {
        const int f = c * kWave + lane;
        const int key = key_of(f);
        const bool valid = (unsigned)key < (unsigned)E;
        const Match m = wave_match(key, valid, nbits, lane);
        if (valid) {
            const int pos = cnt[wave][key] + m.rank;
            perm[pos] = f;
            inv_perm[f] = pos;
            if (w_perm) w_perm[pos] = wts[f];
            if (m.rank == m.total - 1) cnt[wave][key] += m.total;
        } else if (f < R) {
            inv_perm[f] = -1;
        }
    }
    // positions left empty by ids outside [0, E)
    for (int p = n_valid + threadIdx.x; p < R; p += blockDim.x) {
        perm[p] = -1;
        if (w_perm) w_perm[p] = 0.0f;
    }
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
