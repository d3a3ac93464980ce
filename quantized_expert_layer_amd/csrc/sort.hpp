// Stable counting sort of routed slots by expert, done by one workgroup of 16 waves
// ("Who Says Elephants Can't Run", section 3 workflow: the row index is attached to the
// gating output and the tuples are sorted by expert_idx).  Shared by the permute kernel and
// the fused decode-step kernel.
//
// Each wave owns a contiguous range of flat slots and walks it 64 slots at a time.  Lanes
// holding the same key find each other with one ballot per key bit (a wave-wide "match"),
// which gives every slot its rank among equal keys in the chunk and lets one lane per key
// update the wave's running count in LDS.  A scan over (expert, wave) turns counts into
// bases; a second walk writes perm / inv_perm.  Order inside a key is ascending slot index.
#pragma once

#include "common.hpp"

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

// Called by all kSortWaves * 64 threads of the block.  key_of(f) is the expert of slot f
// (f < R; keys outside [0, E) are dropped), w_of(f) its gate weight (read only when w_perm is
// given).  Writes perm [R], inv_perm [R] (-1 for a dropped slot), offsets [E+1] and w_perm [R];
// sorted positions left empty by dropped slots get perm -1, w_perm 0.  Begins with a block
// barrier, so LDS the caller filled just before is visible to key_of.
template <typename KeyOf, typename WOf>
__device__ __forceinline__ void sort_block(int R, int E, KeyOf key_of, WOf w_of,
                                           int32_t* __restrict__ perm,
                                           int32_t* __restrict__ inv_perm,
                                           int32_t* __restrict__ offsets,
                                           float* __restrict__ w_perm) {
    __shared__ int cnt[kSortWaves][MOE_MAX_EXPERTS];
    __shared__ int wave_sum[4];
    __shared__ int n_valid;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    for (int i = threadIdx.x; i < kSortWaves * MOE_MAX_EXPERTS; i += blockDim.x)
        (&cnt[0][0])[i] = 0;
    __syncthreads();
    auto key = [&](int f) -> int { return f < R ? key_of(f) : -1; };

    const int nbits = (E <= 1) ? 0 : 32 - __clz(E - 1);
    const int chunks = (R + kWave - 1) / kWave;
    const int per_wave = (chunks + kSortWaves - 1) / kSortWaves;
    const int c0 = wave * per_wave, c1 = min(chunks, c0 + per_wave);

    // pass 1: per-wave key counts
    for (int c = c0; c < c1; ++c) {
        const int f = c * kWave + lane;
        const int kf = key(f);
        const bool valid = (unsigned)kf < (unsigned)E;
        const Match m = wave_match(kf, valid, nbits, lane);
        if (valid && m.rank == m.total - 1) cnt[wave][kf] += m.total;
    }
    __syncthreads();

    // scan: bases in (expert-major, wave-minor) order.  Threads 0..255 are waves 0..3, one
    // expert per thread; the branch is uniform per wave and the barriers are block-wide.
    int tot = 0, incl = 0;
    if (threadIdx.x < 256) {
        const int e = threadIdx.x;
        if (e < E)
            for (int w = 0; w < kSortWaves; ++w) tot += cnt[w][e];
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
        const int kf = key(f);
        const bool valid = (unsigned)kf < (unsigned)E;
        const Match m = wave_match(kf, valid, nbits, lane);
        if (valid) {
            const int pos = cnt[wave][kf] + m.rank;
            perm[pos] = f;
            inv_perm[f] = pos;
            if (w_perm) w_perm[pos] = w_of(f);
            if (m.rank == m.total - 1) cnt[wave][kf] += m.total;
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

// The same sort done by a single wave, for the few slots of a decode step: one running count
// per expert in LDS (cnt [E], the caller's), no per-wave tables and no block barriers.  LDS
// accesses of one wave take effect in program order; the wave-scope LDS fences keep the
// compiler from moving them across the phases.  Same outputs as sort_block.
// off_lds (LDS, [E + 1]) receives a copy of the offsets.
template <typename KeyOf, typename WOf>
__device__ __forceinline__ void sort_wave(int R, int E, KeyOf key_of, WOf w_of, int* cnt,
                                          int* off_lds, int32_t* __restrict__ perm,
                                          int32_t* __restrict__ inv_perm,
                                          int32_t* __restrict__ offsets,
                                          float* __restrict__ w_perm) {
    const int lane = threadIdx.x & (kWave - 1);
    // LDS ordering only: the global stores of perm / inv_perm / w_perm need not complete
    // before the next phase
    auto phase = [] { lds_wave_fence(); };
    for (int e = lane; e < E; e += kWave) cnt[e] = 0;
    phase();
    const int nbits = (E <= 1) ? 0 : 32 - __clz(E - 1);
    const int chunks = (R + kWave - 1) / kWave;
    for (int c = 0; c < chunks; ++c) {
        const int f = c * kWave + lane;
        const int kf = f < R ? key_of(f) : -1;
        const bool valid = (unsigned)kf < (unsigned)E;
        const Match m = wave_match(kf, valid, nbits, lane);
        if (valid && m.rank == m.total - 1) cnt[kf] += m.total;
        phase();
    }
    // exclusive prefix over the experts: offsets, and the running base of each expert
    int run = 0;
    for (int c0 = 0; c0 < E; c0 += kWave) {
        const int e = c0 + lane;
        const int v = e < E ? cnt[e] : 0;
        const int incl = wave_incl_scan(v);
        if (e < E) {
            offsets[e] = run + incl - v;
            off_lds[e] = run + incl - v;
            cnt[e] = run + incl - v;
        }
        run += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    if (lane == 0) {
        offsets[E] = run;
        off_lds[E] = run;
    }
    phase();
    for (int c = 0; c < chunks; ++c) {
        const int f = c * kWave + lane;
        const int kf = f < R ? key_of(f) : -1;
        const bool valid = (unsigned)kf < (unsigned)E;
        const Match m = wave_match(kf, valid, nbits, lane);
        if (valid) {
            const int base = cnt[kf];
            const int pos = base + m.rank;
            perm[pos] = f;
            inv_perm[f] = pos;
            if (w_perm) w_perm[pos] = w_of(f);
            if (m.rank == m.total - 1) cnt[kf] = base + m.total;
        } else if (f < R) {
            inv_perm[f] = -1;
        }
        phase();
    }
    // positions left empty by keys outside [0, E)
    for (int p = run + lane; p < R; p += kWave) {
        perm[p] = -1;
        if (w_perm) w_perm[p] = 0.0f;
    }
}

}  // namespace moe
