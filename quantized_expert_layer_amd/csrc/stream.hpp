// Stream path of the grouped GEMM: the block body, shared by the grouped GEMM's stream kernel
// and the decode step's launches.  "Who Says Elephants Can't Run", section 3 (grouped GEMM over
// all experts), section 4 (dequantization fused into the GEMM), section 3 optimized I2F.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace moe {

// Row maps of a GEMM call: the A row read for GEMM row p (a gather fused into the load) and
// the output row written for it (a scatter fused into the store).  Source rows are clamped
// into a; a destination outside out is skipped (-1).
__device__ __forceinline__ int a_source_row(const GemmParams& p, int gp) {
    if (!p.a_rows) return gp;
    return min(max(p.a_rows[gp] / p.a_div, 0), p.a_nrows - 1);
}
__device__ __forceinline__ int out_dest_row(const GemmParams& p, int gp) {
    if (!p.out_rows) return gp;
    const int d = p.out_rows[gp];
    return (d >= 0 && d < p.out_nrows) ? d : -1;
}

// ------------------------------------------------------------------------------------
// Stream path.
//   grid  = m-tiles(upper bound) x NGO blocks of S waves (S = p.split, 1..MOE_MAX_SPLIT_K).
//   block = one 16-row m-tile x OPB consecutive 16-column output blocks; for SwiGLU the OPB
//           gate blocks and the OPB up blocks (columns I + ...) of the same outputs, so a wave
//           holds NCB = OPB (x2 for SwiGLU) weight column blocks.  One activation fragment of
//           the tile serves all NCB of them: a 16-row fragment is four times the bytes of a
//           1 KiB weight unit, and a CU's vector-memory pipeline moves 64 bytes per clock.
//           Wave w of the block streams the w-th of S equal K slices; the S partial sums meet
//           in LDS and are added in the fixed order 0, 1, .., S-1 by wave 0, which runs the
//           epilogue.  Splitting K inside the block multiplies the waves of a decode step
//           (which has few output blocks) without a second launch or a workspace.
//   scales= per-channel and group scales multiply fp32 sums: a group-128 scale the sum of
//           one super-block's MFMAs, a per-channel scale the final sum.  Mathematically this
//           is the sum over the scaled weights; it skips the fp16 rounding of each scaled
//           weight and saves a packed multiply per weight pair.
// ------------------------------------------------------------------------------------
// The body of one stream-path block: block `bid` of the call's grid, run by S waves of which
// this is wave w (wave-uniform; S = 1 runs without LDS or barriers, so several such blocks can
// share one workgroup); red: LDS for [S - 1][NCB][64] partial sums of waves 1..S-1.  TAG tells
// apart the kernels that run the same body (a specialization of its own per calling kernel).
template <int WT, int ACT, bool GROUPED, int PF, int PA, int OPB, int TAG = 0>
__device__ __forceinline__ void stream_body(const GemmParams& p, int ngo, int bid, int S, int w,
                                            f32x4* __restrict__ red) {
    constexpr int KSB = WTraits<WT>::KSB;
    constexpr int KSTEPS = KSB / 32;
    constexpr bool SWI = (ACT == MOE_ACT_SWIGLU);
    constexpr int NCB = SWI ? 2 * OPB : OPB;
    const int lane = threadIdx.x & (kWave - 1);

    // (m-tile, output column group), m-tile slowest so that the blocks of existing tiles come
    // first and the surplus of the upper-bound grid exits last
    const int cgo = bid % ngo;
    const int mt = bid / ngo;
    int e, row0, rows;
    if (p.tiles16) {
        // the decode tile table: both loads are issued before the count is compared (the
        // grid's upper bound keeps 1 + mt inside the table)
        const int n = p.tiles16[0];
        const int v = p.tiles16[1 + mt];
        if (mt >= n) return;                                            // block-uniform
        tile16_unpack(v, e, row0, rows);
    } else if (!p.offsets) {
        // dense rows (one expert, no offsets): m-tile mt holds rows 16 mt .. of all R rows
        e = 0;
        row0 = mt * 16;
        rows = min(16, p.R - row0);
        if (rows <= 0) return;                                          // block-uniform
    } else if (!find_m_tile<16>(p.offsets, p.E, p.R, mt, e, row0, rows)) {
        return;                                                         // block-uniform
    }

    const int K = p.K, N = p.N;
    const int nSB = K / KSB;
    const int chunk = (nSB + S - 1) / S;
    const int kb0 = min(nSB, w * chunk);
    const int kb1 = min(nSB, kb0 + chunk);

    const int ncbw = N / 16;
    const int nbo = SWI ? ncbw / 2 : ncbw;       // output column blocks
    int ncol[NCB];
    const u32x4* wp[NCB];
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
        // SwiGLU: the up block of output block o sits nbo blocks after its gate block
        const int cbw = (c < OPB) ? cgo * OPB + c : nbo + cgo * OPB + (c - OPB);
        ncol[c] = cbw * 16 + (lane & 15);
        wp[c] = (const u32x4*)p.w + ((size_t)(e * ncbw + cbw) * nSB) * kWave + lane;
    }
    const int G = GROUPED ? K / 128 : 1;         // groups of 128 rows along K
    const uint16_t* sp = p.scales + (size_t)e * G * N;

    // A fragment source: row (lane & 15) of the tile, 8 halves at k = 8 * (lane >> 4).  With a
    // row map the source row is a dependent load; it is issued before the weights and read
    // after them, so the weights do not wait for it.
    const int arow = lane & 15;
    const bool arow_ok = arow < rows;
    const int gp = row0 + (arow_ok ? arow : 0);
    const int amap = p.a_rows ? p.a_rows[gp] : gp;
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc[NCB];
#pragma unroll
    for (int c = 0; c < NCB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Two rings: weights (HBM, the long latency) PF super-blocks ahead, activations (a few
    // rows, cached) PA ahead.  An activation slot is four times a weight slot in registers,
    // so the short ring leaves room for more resident waves.
    static_assert(PF % PA == 0, "activation slots follow the weight slots");
    u32x4 braw[PF][NCB];
    f16x8 araw[PA][KSTEPS];
    uint32_t sraw[PF][NCB] = {};           // fp16 scale bits, zero-extended

    auto issue_w = [&](int slot, int kb) {
        const int kl = min(kb, kb1 - 1);        // clamped: tail loads repeat the last block
#pragma unroll
        for (int c = 0; c < NCB; ++c) {
            braw[slot][c] = load_weights16(wp[c] + (size_t)kl * kWave);
            if constexpr (GROUPED) sraw[slot][c] = (uint32_t)sp[(size_t)((kl * KSB) >> 7) * N + ncol[c]];
        }
    };

    if (kb0 < kb1) {
        // ring of PF register slots: slot u holds super-block kc + u of the current group
#pragma unroll
        for (int u = 0; u < PF; ++u) issue_w(u, kb0 + u);
        __builtin_amdgcn_sched_barrier(0);
    }
    const int asrc = p.a_rows ? min(max(amap / p.a_div, 0), p.a_nrows - 1) : amap;
    const f16x8* ap = (const f16x8*)(p.a + (size_t)asrc * K) + (lane >> 4);
    auto issue_a = [&](int slot, int kb) {
        const int kl = min(kb, kb1 - 1);
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) araw[slot][j] = ap[(kl * KSB + j * 32) / 8];
    };

    const I2F4Consts k4;
    const f16x2 one2 = {(f16)1.0f, (f16)1.0f};
    auto compute = [&](const u32x4 (&bq)[NCB], const uint32_t (&sq)[NCB],
                       const f16x8 (&aq)[KSTEPS]) {
#pragma unroll
        for (int c = 0; c < NCB; ++c) {
            if constexpr (GROUPED) {
                // two interleaved chains (even / odd K-steps): a dependent MFMA chain stalls
                f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < KSTEPS; ++j) {
                    if (j & 1) t1 = mfma16x16x32(aq[j], weight_frag<WT, false>(bq[c], j, one2, k4), t1);
                    else t0 = mfma16x16x32(aq[j], weight_frag<WT, false>(bq[c], j, one2, k4), t0);
                }
                const f32x4 t = t0 + t1;
                const float s = (float)__builtin_bit_cast(f16, (uint16_t)sq[c]);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[c][i] = __builtin_fmaf(t[i], s, acc[c][i]);
            } else {
#pragma unroll
                for (int j = 0; j < KSTEPS; ++j)
                    acc[c] = mfma16x16x32(aq[j], weight_frag<WT, false>(bq[c], j, one2, k4), acc[c]);
            }
        }
    };

    if (kb0 < kb1) {
#pragma unroll
        for (int u = 0; u < PA; ++u) issue_a(u, kb0 + u);
        int kc = kb0;
        // steady state, branch-free: compute from slot u in place, then refill slot u with the
        // block PF ahead and activation slot u % PA with the block PA ahead (no register
        // copies of in-flight loads, so no early waits)
        for (; kc + PF <= kb1; kc += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                compute(braw[u], sraw[u], araw[u % PA]);
                issue_w(u, kc + u + PF);
                issue_a(u % PA, kc + u + PA);
            }
        }
        // tail: fewer than PF blocks left, their weights already in their slots
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            if (kc + u < kb1) {
                compute(braw[u], sraw[u], araw[u % PA]);
                issue_a(u % PA, kc + u + PA);
            }
        }
        // every ring slot holds a load (a repeat of the last block where the slice ran out)
#pragma unroll
        for (int u = 0; u < PF; ++u) {
#pragma unroll
            for (int c = 0; c < NCB; ++c) {
                consume(braw[u][c]);
                if constexpr (GROUPED) consume(sraw[u][c]);
            }
        }
#pragma unroll
        for (int u = 0; u < PA; ++u)
#pragma unroll
            for (int j = 0; j < KSTEPS; ++j) consume(araw[u][j]);
    }

    // fixed-order reduction of the K slices
    if (S > 1) {
        if (w > 0) {
#pragma unroll
            for (int c = 0; c < NCB; ++c) red[((w - 1) * NCB + c) * kWave + lane] = acc[c];
        }
        lds_barrier();
        if (w > 0) return;
        for (int s = 1; s < S; ++s) {
#pragma unroll
            for (int c = 0; c < NCB; ++c) acc[c] += red[((s - 1) * NCB + c) * kWave + lane];
        }
    }

    // The activation fragment is the MFMA's first operand here, so lane l holds output
    // column (l & 15) of rows 4*(l >> 4) .. +3: one scale per lane, the same column as the
    // lane's weight fragment (the output of a decode block is a few hundred bytes, so its
    // 2-byte stores cost nothing).
    if constexpr (!GROUPED && WT != MOE_W_FP16) {
#pragma unroll
        for (int c = 0; c < NCB; ++c) {
            const float sc = f16_bits_to_f32(sp[ncol[c]]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[c][i] *= sc;
        }
    }
    const int n_out = SWI ? N / 2 : N;
    uint16_t* ocol = p.out + cgo * OPB * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * (lane >> 4) + i;      // row of the tile
        if (r >= rows) break;
        const float rs = p.row_scale ? p.row_scale[row0 + r] : 1.0f;
        const int dst = out_dest_row(p, row0 + r);
        if (dst < 0) continue;
#pragma unroll
        for (int o = 0; o < OPB; ++o) {
            float v;
            if constexpr (SWI) v = silu(acc[o][i]) * acc[OPB + o][i];
            else if constexpr (ACT == MOE_ACT_RELU) v = fmaxf(acc[o][i], 0.0f);
            else v = acc[o][i];
            if (p.row_scale) v *= rs;
            ocol[(size_t)dst * n_out + o * 16] = f32_to_f16_bits(v);
        }
    }
}


}  // namespace moe
