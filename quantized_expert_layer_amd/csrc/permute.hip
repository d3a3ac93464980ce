// Token routing by a stable sort keyed on expert index, then the activation permute
// ("Who Says Elephants Can't Run", section 3 workflow: the row index is attached to the
// gating output, the tuples are sorted by expert_idx, the activations are permuted).
//
// Up to 1024 slots the sort is sort_block (one workgroup of 16 waves, ballot-matched counting
// sort).  Beyond that one workgroup is bound by its CU's VALU (the per-bit ballot matching of
// every 64-slot chunk), so the slots are split into 1024-slot blocks, each of which turns the
// per-expert counts of all slots into its own per-expert bases and places its slots.  Up to
// kSortCountBlocks blocks every block counts all R keys itself (one launch; the keys are at
// most 32 KiB and sit in L2; counting costs about 0.3 us per 1000 keys, less than a second
// launch up to about 12000); beyond that a first launch counts each block's keys into a small
// workspace and the second reads those counts.  Same result either way, stable.
#include "common.hpp"
#include "launch.hpp"
#include "sort.hpp"

namespace moe {

constexpr int kSortBlockSlots = kSortWaves * kWave;   // slots per block of the multi-block sort
constexpr int kSortCountBlocks = 8;   // up to this many blocks each block counts all keys itself

// One workgroup sorts up to kSortBlockSlots slots.  The keys are first copied to LDS with one
// coalesced pass, so the two walks of the sort read LDS instead of issuing one dependent global
// load per 64-key chunk.
__global__ __launch_bounds__(1024) void sort_kernel(const int32_t* __restrict__ ids,
                                                    const float* __restrict__ wts, int R, int E,
                                                    int32_t* __restrict__ perm,
                                                    int32_t* __restrict__ inv_perm,
                                                    int32_t* __restrict__ offsets,
                                                    float* __restrict__ w_perm) {
    __shared__ int keys[kSortBlockSlots];
    for (int i = threadIdx.x; i < R; i += blockDim.x) keys[i] = ids[i];
    sort_block(R, E, [&](int f) { return keys[f]; }, [&](int f) { return wts[f]; }, perm,
               inv_perm, offsets, w_perm);
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

// Multi-block sort, launch 1: block b counts the keys of slots [1024 b, 1024 (b + 1)) per
// expert (one 64-slot chunk per wave; one LDS add per distinct key per wave).
__global__ __launch_bounds__(1024) void sort_hist_kernel(const int32_t* __restrict__ ids, int R,
                                                         int E, int32_t* __restrict__ hist) {
    __shared__ int cnt[MOE_MAX_EXPERTS];
    const int lane = threadIdx.x & (kWave - 1);
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int nbits = (E <= 1) ? 0 : 32 - __clz(E - 1);
    const int f = blockIdx.x * kSortBlockSlots + threadIdx.x;
    const int kf = f < R ? ids[f] : -1;
    const bool valid = (unsigned)kf < (unsigned)E;
    const Match m = wave_match(kf, valid, nbits, lane);
    if (valid && m.rank == m.total - 1) atomicAdd(&cnt[kf], m.total);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Multi-block sort, scatter: block b takes the per-expert counts of all slots (COUNT: by
// counting every key itself; else from the counts launch 1 left in hist), the global offsets
// of the experts (exclusive scan of the totals) plus the counts of the slots before its own as
// its bases, ranks its own slots as sort_block does (wave order, then rank among equal keys of
// a chunk) and writes perm / inv_perm / w_perm.  Block 0 also writes offsets and fills the
// positions left empty by slots routed nowhere.
template <bool COUNT>
__global__ __launch_bounds__(1024) void sort_scatter_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int R, int E,
    const int32_t* __restrict__ hist, int nblk, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv_perm, int32_t* __restrict__ offsets, float* __restrict__ w_perm) {
    __shared__ int cnt[kSortWaves][MOE_MAX_EXPERTS];
    __shared__ int base[MOE_MAX_EXPERTS];
    __shared__ int all_cnt[COUNT ? MOE_MAX_EXPERTS : 1];    // keys of all slots, per expert
    __shared__ int pre_cnt[COUNT ? MOE_MAX_EXPERTS : 1];    // keys of the slots before block b
    __shared__ int wave_sum[4];
    __shared__ int n_valid;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int f = blockIdx.x * kSortBlockSlots + threadIdx.x;
    const int kf = f < R ? ids[f] : -1;
    const float wf = (w_perm && f < R) ? wts[f] : 0.0f;
    const int nbits = (E <= 1) ? 0 : 32 - __clz(E - 1);
    for (int i = threadIdx.x; i < kSortWaves * MOE_MAX_EXPERTS; i += blockDim.x)
        (&cnt[0][0])[i] = 0;

    if constexpr (COUNT) {
        // every block counts all R keys: wave w takes 64-slot chunks w, w + 16, ...; four
        // chunks' loads are issued before the first is matched.  The chunks before this
        // block's first (16 b) are its predecessors' slots.
        for (int e = threadIdx.x; e < MOE_MAX_EXPERTS; e += blockDim.x) {
            all_cnt[e] = 0;
            pre_cnt[e] = 0;
        }
        __syncthreads();
        const int nchunks = (R + kWave - 1) / kWave;
        const int first_own = blockIdx.x * kSortWaves;
        constexpr int U = 4;
        for (int c0 = wave; c0 < nchunks; c0 += U * kSortWaves) {
            int key[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int g = (c0 + u * kSortWaves) * kWave + lane;
                key[u] = g < R ? ids[g] : -1;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool ok = (unsigned)key[u] < (unsigned)E;
                const Match mu = wave_match(key[u], ok, nbits, lane);
                if (ok && mu.rank == mu.total - 1) {
                    atomicAdd(&all_cnt[key[u]], mu.total);
                    if (c0 + u * kSortWaves < first_own) atomicAdd(&pre_cnt[key[u]], mu.total);
                }
            }
        }
        __syncthreads();
    }

    int tot = 0, pre = 0, incl = 0;
    if (threadIdx.x < 256) {                   // waves 0..3, one expert per thread
        const int e = threadIdx.x;
        if (e < E) {
            if constexpr (COUNT) {
                tot = all_cnt[e];
                pre = pre_cnt[e];
            } else {
                for (int b = 0; b < nblk; ++b) {
                    const int h = hist[(size_t)b * E + e];
                    tot += h;
                    if (b < (int)blockIdx.x) pre += h;
                }
            }
        }
        incl = wave_incl_scan(tot);
        if (lane == kWave - 1) wave_sum[wave] = incl;
    }
    __syncthreads();
    if (threadIdx.x < 256) {
        const int e = threadIdx.x;
        int before = 0;
        for (int w = 0; w < wave; ++w) before += wave_sum[w];
        const int start = before + incl - tot;
        if (e < E) {
            base[e] = start + pre;
            if (blockIdx.x == 0) offsets[e] = start;
            if (e == E - 1) {
                if (blockIdx.x == 0) offsets[E] = start + tot;
                n_valid = start + tot;
            }
        }
    }
    // pass 1: per-wave counts of this block's slots (one chunk per wave)
    const bool valid = (unsigned)kf < (unsigned)E;
    const Match m = wave_match(kf, valid, nbits, lane);
    if (valid && m.rank == m.total - 1) cnt[wave][kf] = m.total;
    __syncthreads();
    // per-(wave, expert) bases in wave order
    if (threadIdx.x < E) {
        const int e = threadIdx.x;
        int run = base[e];
        for (int w = 0; w < kSortWaves; ++w) {
            const int c = cnt[w][e];
            cnt[w][e] = run;
            run += c;
        }
    }
    __syncthreads();
    // pass 2: scatter
    if (valid) {
        const int pos = cnt[wave][kf] + m.rank;
        perm[pos] = f;
        inv_perm[f] = pos;
        if (w_perm) w_perm[pos] = wf;
    } else if (f < R) {
        inv_perm[f] = -1;
    }
    if (blockIdx.x == 0) {
        for (int p = n_valid + threadIdx.x; p < R; p += blockDim.x) {
            perm[p] = -1;
            if (w_perm) w_perm[p] = 0.0f;
        }
    }
}

size_t sort_workspace_bytes(int R, int E) {
    const size_t nblk = ((size_t)R + kSortBlockSlots - 1) / kSortBlockSlots;
    if (nblk <= (size_t)kSortCountBlocks) return 0;
    return nblk * (size_t)E * sizeof(int32_t);
}

hipError_t launch_sort(const int32_t* ids, const float* wts, int R, int E, int32_t* perm,
                       int32_t* inv_perm, int32_t* offsets, float* w_perm, void* ws,
                       hipStream_t stream) {
    if (R > kSortBlockSlots) {
        const int nblk = (R + kSortBlockSlots - 1) / kSortBlockSlots;
        if (nblk <= kSortCountBlocks) {
            sort_scatter_kernel<true><<<nblk, kSortBlockSlots, 0, stream>>>(
                ids, wts, R, E, nullptr, nblk, perm, inv_perm, offsets, w_perm);
            return hipGetLastError();
        }
        int32_t* hist = (int32_t*)ws;
        sort_hist_kernel<<<nblk, kSortBlockSlots, 0, stream>>>(ids, R, E, hist);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        sort_scatter_kernel<false><<<nblk, kSortBlockSlots, 0, stream>>>(
            ids, wts, R, E, hist, nblk, perm, inv_perm, offsets, w_perm);
        return hipGetLastError();
    }
    sort_kernel<<<1, kSortWaves * kWave, 0, stream>>>(ids, wts, R, E, perm, inv_perm, offsets,
                                                     w_perm);
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
