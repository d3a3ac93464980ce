// Grouped GEMM over all experts with weights dequantized in registers.
//
// "Who Says Elephants Can't Run", section 3 (Fig. 1, workflow): every expert's GEMM runs in
// one grouped launch, one sub-matrix per expert; section 4: the dequantization is fused
// into the GEMM; section 3 optimized I2F: codes become fp16 through the exponent-of-1024
// construction.  The dequantized weight is Algorithm 1's W_dq = code * S.
//
// Two paths share the packed layout and the MFMA 16x16x32 fp16 fragment shapes:
//   stream : 16-row m-tiles, one block per 16 output columns, A fragments straight from
//            global memory, weights streamed once with a deep register prefetch.  Meant for
//            the few rows per expert of decode / verify (the Specter page's fine-grained
//            expert kernels); optional K split across the waves of a block, reduced in LDS
//            in a fixed order.
//   tile   : 64-row m-tiles, 4 waves x (64 or 32) weight columns, A staged through LDS
//            (double buffered), weights double buffered in registers.  Meant for large M.
// Experts with no rows launch no work that reads weights.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "stream.hpp"

namespace moe {

// Output fragment layout.  The MFMA is issued with the weight fragment as its first operand
// and the activation fragment as its second, i.e. it computes Y^T = W^T X^T; lane l then holds
// row (l & 15) of its 16-row subtile and the 4 consecutive columns 4*(l >> 4) .. +3 of its
// 16-column block, so results leave in 8-byte stores.
__device__ __forceinline__ void store4_f16(uint16_t* dst, float a, float b, float c, float d) {
    f16x2 lo = {(f16)a, (f16)b}, hi = {(f16)c, (f16)d};
    uint2 v;
    v.x = __builtin_bit_cast(uint32_t, lo);
    v.y = __builtin_bit_cast(uint32_t, hi);
    *(uint2*)dst = v;
}

__device__ __forceinline__ f32x4 load4_scale(const uint16_t* src) {
    const uint2 v = *(const uint2*)src;
    const f16x2 lo = __builtin_bit_cast(f16x2, v.x), hi = __builtin_bit_cast(f16x2, v.y);
    return f32x4{(float)lo[0], (float)lo[1], (float)hi[0], (float)hi[1]};
}

template <int WT, int ACT, bool GROUPED, int PF, int PA, int OPB>
__global__ __launch_bounds__(64 * MOE_MAX_SPLIT_K) void gemm_stream_kernel(GemmParams p, int ngo) {
    extern __shared__ f32x4 red[];          // [S - 1][NCB][64] partial sums of waves 1..S-1
    // wave index, held in a scalar register (the compiler cannot see it is wave-uniform)
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    stream_body<WT, ACT, GROUPED, PF, PA, OPB>(p, ngo, blockIdx.x, blockDim.x / kWave, w, red);
}

// The stream launch with a second, dense GEMM beside it ([S] Method step 5: the step's expert
// sub-computations in one launch): workgroups [0, nwg) run the grouped GEMM p, the rest the fp16
// GEMM ps over all of its rows (the decode step's shared experts, E = 1, every token), each
// dense block's K split over the workgroup's W waves.  With p unsplit (rs == 1) each wave of a
// grouped workgroup runs a block of its own (block W * workgroup + wave), so the dense GEMM's
// long K streams still get W waves; otherwise every workgroup runs one block of rs == W waves.
constexpr int kDenseSidePF = 8;
constexpr int kDenseSideWaves = 4;
template <int WT, int ACT, bool GROUPED, int PF, int PA, int OPB, int SACT>
__global__ __launch_bounds__(64 * MOE_MAX_SPLIT_K) void gemm_stream_side_kernel(GemmParams p, int ngo,
                                                                              int nb, int nwg,
                                                                              GemmParams ps,
                                                                              int ngo_s) {
    extern __shared__ f32x4 red[];
    constexpr int kTagSide = 16 + ((((WT * 3 + ACT) * 2 + (GROUPED ? 1 : 0)) * 16 + PF) * 4 + OPB) * 3 + SACT;
    const int W = blockDim.x / kWave;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if ((int)blockIdx.x < nwg) {
        if (p.split == 1) {
            const int b = (int)blockIdx.x * W + w;
            if (b < nb) stream_body<WT, ACT, GROUPED, PF, PA, OPB, 1 + SACT>(p, ngo, b, 1, 0, red);
        } else {
            stream_body<WT, ACT, GROUPED, PF, PA, OPB, 1 + SACT>(p, ngo, blockIdx.x, W, w, red);
        }
    } else {
        stream_body<MOE_W_FP16, SACT, false, kDenseSidePF, 2, 1, kTagSide>(
            ps, ngo_s, (int)blockIdx.x - nwg, W, w, red);
    }
}

// ------------------------------------------------------------------------------------
// Tile path.
//   block tile  = 16*MS rows x (4 waves x NS column blocks of 16); a wave owns its NS weight
//                 column blocks for all the tile's rows, so each weight byte of the tile is
//                 loaded and expanded by one wave only.  SwiGLU: NS/2 gate blocks + the
//                 matching NS/2 up blocks.
//   K stage     = 128 rows of K (64 for fp16 weights).  Integer codes: the A stage (rows x KC
//                 fp16) goes from memory straight into a ring of three LDS buffers, two
//                 stages ahead; fp16 weights: it is loaded to registers two stages ahead and
//                 written to LDS one stage ahead (double buffered).  The weights are loaded
//                 one stage ahead into two register buffers that alternate.  The activation
//                 rows are usually not in L2 (a previous kernel's output, or x read through
//                 perm), so their latency is the longer one.  LDS rows are not padded:
//                 16-byte chunk c of row r sits at chunk position c ^ (r & 15), so the 16
//                 lanes of an A-fragment read (16 rows, one chunk) hit distinct 4-bank groups.
//   partial     = a tile with fewer valid rows runs the body specialised for its number of
//                 16-row subtiles (1..MS), so it neither loads nor multiplies absent rows.
//   K groups    = fp16 weights on a small grid: 2 or 4 groups of 4 waves split the K stages
//                 and add their fp32 partial tiles through LDS (see tile_body).
//   occupancy   = 2+ blocks per CU, so each SIMD interleaves at least two waves.
// ------------------------------------------------------------------------------------
// K per stage: 128 rows for int4/int8 codes (one 128-group), 64 for fp16 weights (whose
// register double buffer is 4x larger per row).  256-row int4 stages measured slower: the
// extra registers cost more than the longer cover of the next stage's load latency.
template <int WT> constexpr int tile_kc() { return WT == MOE_W_FP16 ? 64 : 128; }

// A stages held in LDS: a ring of three for integer codes (loaded straight into LDS, two stages
// ahead), two for fp16 weights (register-staged).
template <int WT> constexpr int tile_a_stages() { return WT == MOE_W_FP16 ? 2 : 3; }


// Epilogue staging: row stride (halves) of a wave's output region in LDS, padded by 16 bytes
// so the 16 rows of one fragment store start in different banks.
template <int ACT, int NS> constexpr int tile_epi_stride() {
    return (ACT == MOE_ACT_SWIGLU ? NS / 2 : NS) * 16 + 8;
}
// LDS of one block: the A stages of its KG groups, the fp32 partial tiles of groups 1..KG-1,
// or the 4 waves' epilogue regions, whichever is largest.
template <int WT, int ACT, int MS, int NS, int KG = 1> constexpr int tile_lds_halves() {
    const int stages = KG * tile_a_stages<WT>() * 16 * MS * tile_kc<WT>();
    const int partial = (KG - 1) * 4 * MS * NS * kWave * 4 * 2;
    const int epi = 4 * 16 * MS * tile_epi_stride<ACT, NS>();
    const int m = stages > epi ? stages : epi;
    return m > partial ? m : partial;
}

// Weight loads of the tile path while LDS-DMA loads are in flight.  The compiler counts
// outstanding vector loads exactly only while every pending load fills registers: with LDS-DMA
// loads pending it waits for all of them (vmcnt 0) before a register load's first use, which
// would drain the A stages loaded two ahead at every stage.  These weight loads are therefore
// issued as instructions of their own; the per-stage wait counts them (vector memory loads
// complete in order), and tie_to_wait() makes every later use of a register depend on an
// instruction placed after that wait.  Between the load and the wait nothing reads or moves the
// destination registers (the test suite checks the generated code for this).
__device__ __forceinline__ void issue_load16(u32x4& dst, const void* ptr) {
    asm volatile("global_load_dwordx4 %0, %1, off ; weight load" : "=&v"(dst) : "v"(ptr) : "memory");
}
__device__ __forceinline__ void issue_load_u16(uint32_t& dst, const void* ptr) {
    asm volatile("global_load_ushort %0, %1, off ; weight load" : "=&v"(dst) : "v"(ptr) : "memory");
}
template <typename T>
__device__ __forceinline__ void tie_to_wait(T& v) {
    asm volatile("; weights ready %0" : "+v"(v));
}

// KG > 1 (fp16 weights only): the block holds KG groups of 4 waves; group g runs the K stages
// [g * n, (g + 1) * n) of the tile with its own A buffers, and groups 1..KG-1 hand their fp32
// partial tiles to group 0 through LDS, which adds them in group order and writes the tile.
template <int WT, int ACT, bool GROUPED, int MA, int NS, int BM, int KG = 1, bool NATIVE = false>
__device__ __forceinline__ void tile_body(const GemmParams& p, f16* __restrict__ lds, int e,
                                          int row0, int rows, int cbg) {
    constexpr int KSB = WTraits<WT>::KSB;
    constexpr int KC = tile_kc<WT>();
    constexpr int KSTEPS = KC / 32;                  // MFMA K-steps per stage
    constexpr int KSPS = KSB / 32;                   // K-steps per super-block
    constexpr int SBPS = KC / KSB;                   // super-blocks per stage per column block
    constexpr int CPR = KC / 8;                      // 16-byte chunks per LDS row
    // the fragment reads below XOR with (lane row & (CPR - 1)), which equals the staged row's
    // (r & (CPR - 1)) only while CPR divides 16
    static_assert(CPR <= 16, "A swizzle assumes at most 16 chunks per LDS row");
    constexpr int ATOT = MA * 16 * CPR;              // A chunks per stage
    constexpr int ACH = (ATOT + 255) / 256;          // A chunks per thread per stage
    constexpr int LDS_BUF = BM * KC;                 // halves per buffer
    constexpr bool SWI = (ACT == MOE_ACT_SWIGLU);
    constexpr int NO = SWI ? NS / 2 : NS;            // output column blocks per wave

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (threadIdx.x / kWave) & 3;      // column wave within the group
    const int kg = threadIdx.x / 256;                // K group
    const int tid = threadIdx.x & 255;
    const int K = p.K, N = p.N;
    const int nSB = K / KSB;
    const int ncbw = N / 16;
    const int nbo = SWI ? ncbw / 2 : ncbw;

    int ob[NO];
    bool ob_ok[NO];
#pragma unroll
    for (int c = 0; c < NO; ++c) {
        const int o = (cbg * 4 + wave) * NO + c;
        ob_ok[c] = o < nbo;
        ob[c] = ob_ok[c] ? o : 0;
    }
    const u32x4* wp[NS];
    int ncol[NS];
#pragma unroll
    for (int c = 0; c < NS; ++c) {
        const int cbw = SWI ? ob[c % NO] + (c / NO) * nbo : ob[c];
        wp[c] = (const u32x4*)p.w + ((size_t)(e * ncbw + cbw) * nSB) * kWave + lane;
        ncol[c] = cbw * 16 + (lane & 15);
    }
    const int G = GROUPED ? K / 128 : 1;
    const uint16_t* sp = p.scales + (size_t)e * G * N;

    // A staging.  With integer codes (DMA_A) the A stages go straight from memory into an LDS
    // ring of AD buffers (global_load_lds: lane i of a wave-wide load writes bytes 16 i ..
    // 16 i + 15 after the wave's LDS base), two stages ahead, with no registers or LDS store
    // instructions of their own.  Chunk q of a buffer (16 bytes; row q / CPR, position
    // q % CPR) receives the row's chunk (q % CPR) ^ (row & (CPR - 1)), the same swizzle the
    // fragment reads below undo.  Rows past the tile repeat its last row.  Each wave issues NA
    // wave-wide loads per stage.  fp16 weights, whose per-stage weight loads are four times
    // larger, keep the register-staged path below, which measured faster for them.
    constexpr bool DMA_A = WT != MOE_W_FP16;
    static_assert(KG == 1 || !DMA_A, "K groups are built for the register-staged A path only");
    constexpr int AD = tile_a_stages<WT>();
    constexpr int NAB = DMA_A ? (ATOT > 256 ? ATOT : 256) / kWave : 4;  // wave-wide loads / stage
    constexpr int NA = NAB / 4;
    static_assert(NAB % 4 == 0 && LDS_BUF * 2 >= NAB * 1024, "DMA stage layout");
    const char* adma[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int q = (wave * NA + i) * kWave + lane;
        const int r = q / CPR, cp = q % CPR;
        const int c = cp ^ (r & (CPR - 1));
        adma[i] = (const char*)(p.a + (size_t)a_source_row(p, row0 + min(r, rows - 1)) * K) + c * 16;
    }
    auto dma_a = [&](int st, int buf) {
#pragma unroll
        for (int i = 0; i < NA; ++i)
            __builtin_amdgcn_global_load_lds(
                adma[i] + (size_t)st * KC * 2,
                (__attribute__((address_space(3))) void*)(lds + buf * LDS_BUF + (wave * NA + i) * 512),
                16, 0, 0);
    };
    // register-staged A: chunk q = tid + 256 i -> row q / CPR, chunk q % CPR, into the group's
    // two LDS buffers
    f16* const lds_a = lds + (KG > 1 ? kg * 2 * LDS_BUF : 0);
    const u32x4* asrc[ACH];
    int adst[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int q = min(tid + 256 * i, ATOT - 1);
        const int r = q / CPR, c = q % CPR;
        asrc[i] = (const u32x4*)(p.a + (size_t)a_source_row(p, row0 + min(r, rows - 1)) * K) + c;
        adst[i] = r * KC + ((c ^ (r & (CPR - 1))) * 8);
    }
    // WD weight buffers and (register-staged path) WD A register sets, which rotate statically
    // (the stage loops below run WD stages per iteration; copying a buffer whose loads are in
    // flight would make the compiler wait for every outstanding load).  A stage's weights are
    // loaded WD - 1 stages ahead and its A rows WD stages ahead, then stored to the idle LDS
    // buffer at the end of the stage before.  Four-deep rings on the fp16 shapes with few
    // blocks (the shared experts of a 288-token step) measured no faster than two.
    constexpr int WD = 2;
    u32x4 areg[WD][ACH];
    auto load_a = [&](int set, int st) {
#pragma unroll
        for (int i = 0; i < ACH; ++i)
            if (ATOT % 256 == 0 || tid + 256 * i < ATOT) areg[set][i] = asrc[i][st * CPR];
    };
    auto store_a = [&](int set, int buf) {
#pragma unroll
        for (int i = 0; i < ACH; ++i)
            if (ATOT % 256 == 0 || tid + 256 * i < ATOT)
                *(u32x4*)(lds_a + buf * LDS_BUF + adst[i]) = areg[set][i];
    };

    // group scales: one per (column block, super-block) -- a super-block never spans groups
    constexpr int SCS = GROUPED ? SBPS : 1;
    u32x4 bbuf[WD][NS][SBPS];
    uint32_t sbuf[WD][NS][SCS] = {};
    auto load_b = [&](u32x4 (&b)[NS][SBPS], uint32_t (&sc)[NS][SCS], int st) {
#pragma unroll
        for (int c = 0; c < NS; ++c) {
#pragma unroll
            for (int q = 0; q < SBPS; ++q) {
                b[c][q] = wp[c][(size_t)(st * SBPS + q) * kWave];
                if constexpr (GROUPED)
                    sc[c][q] = (uint32_t)sp[(size_t)((st * KC + q * KSB) >> 7) * N + ncol[c]];
            }
        }
    };
    // the same loads issued by hand (DMA path), and the ties that follow their wait
    auto issue_b = [&](u32x4 (&b)[NS][SBPS], uint32_t (&sc)[NS][SCS], int st) {
#pragma unroll
        for (int c = 0; c < NS; ++c) {
#pragma unroll
            for (int q = 0; q < SBPS; ++q) {
                issue_load16(b[c][q], wp[c] + (size_t)(st * SBPS + q) * kWave);
                if constexpr (GROUPED)
                    issue_load_u16(sc[c][q], sp + (size_t)((st * KC + q * KSB) >> 7) * N + ncol[c]);
            }
        }
    };
    auto tie_b = [&](u32x4 (&b)[NS][SBPS], uint32_t (&sc)[NS][SCS]) {
#pragma unroll
        for (int c = 0; c < NS; ++c) {
#pragma unroll
            for (int q = 0; q < SBPS; ++q) {
                tie_to_wait(b[c][q]);
                if constexpr (GROUPED) tie_to_wait(sc[c][q]);
            }
        }
    };

    const I2F4Consts k4;
    f32x4 acc[MA][NS];
#pragma unroll
    for (int m = 0; m < MA; ++m)
#pragma unroll
        for (int c = 0; c < NS; ++c) acc[m][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nstage = K / KC;
    const int lrow = lane & 15;
    // one stage's MFMAs from the A stage in abuf and the weights in bcur / scur
    auto compute_stage = [&](const f16* abuf, const u32x4 (&bcur)[NS][SBPS],
                             const uint32_t (&scur)[NS][SCS]) {
        // the weight fragments of K-step ks+1 are expanded while the MFMAs of ks issue
        auto expand = [&](f16x8 (&bq)[NS], int ks) {
#pragma unroll
            for (int c = 0; c < NS; ++c) {
                const f16 sv = __builtin_bit_cast(f16, (uint16_t)scur[c][GROUPED ? ks / KSPS : 0]);
                const f16x2 s2 = {sv, sv};
                bq[c] = weight_frag<WT, GROUPED, NATIVE>(bcur[c][ks / KSPS], ks % KSPS, s2, k4);
            }
        };
        f16x8 bq[NS];
        expand(bq, 0);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const int pos = (ks * 4 + (lane >> 4)) ^ (lrow & (CPR - 1));
            f16x8 af[MA];
#pragma unroll
            for (int m = 0; m < MA; ++m) af[m] = *(const f16x8*)(abuf + (m * 16 + lrow) * KC + pos * 8);
            f16x8 bn[NS];
            if (ks + 1 < KSTEPS) expand(bn, ks + 1);
#pragma unroll
            for (int m = 0; m < MA; ++m)
#pragma unroll
                for (int c = 0; c < NS; ++c) acc[m][c] = mfma16x16x32(bq[c], af[m], acc[m][c]);
            if (ks + 1 < KSTEPS) {
#pragma unroll
                for (int c = 0; c < NS; ++c) bq[c] = bn[c];
            }
        }
    };

    if constexpr (DMA_A) {
        // prologue: A stage 0, the weights of stage 0, then A stages 1 .. AD-2
        dma_a(0, 0);
        __builtin_amdgcn_sched_barrier(0);
        issue_b(bbuf[0], sbuf[0], 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s0 = 1; s0 < AD - 1; ++s0) dma_a(min(s0, nstage - 1), s0);

        // Waits.  Per stage a wave issues, in this order, the weight / scale loads of stage
        // st + 1 and NA A loads (stage st + AD - 1); vector memory loads complete in order.  At
        // the top of stage st only the NA A loads issued after the weights of stage st (those
        // of stage st + AD - 2) may still be outstanding: once at most NA are, the weights of
        // stage st and this wave's A loads of stage st (issued earlier still) are done.  The
        // barrier after the wait makes every wave's A loads of stage st visible and frees the
        // buffer stage st - 1 used, which the stage's new A loads overwrite.  (The barrier is
        // issued bare: the compiler's fence before a block barrier would wait for all A loads
        // in flight.)  The count holds for the first stages too, whose prologue order is A
        // stage 0, the weights of stage 0, A stages 1 .. AD - 2.
        constexpr int NWAIT = NA;
        static_assert(NWAIT < 64, "vmcnt field");
        constexpr int WAITCNT = (NWAIT & 15) | ((NWAIT >> 4) << 14) | (7 << 4) | (15 << 8);

        auto stage = [&](int st, u32x4 (&bc)[NS][SBPS], uint32_t (&sc)[NS][SCS],
                         u32x4 (&bn)[NS][SBPS], uint32_t (&sn)[NS][SCS]) {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(WAITCNT);
            __builtin_amdgcn_sched_barrier(0);
            tie_b(bc, sc);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            issue_b(bn, sn, min(st + 1, nstage - 1));
            __builtin_amdgcn_sched_barrier(0);
            dma_a(min(st + AD - 1, nstage - 1), (st + AD - 1) % AD);
            // keep the prefetch at the top: the scheduler would otherwise sink the loads next
            // to their first use at the end of the stage and expose their full latency
            __builtin_amdgcn_sched_barrier(0);
            compute_stage(lds + (st % AD) * LDS_BUF, bc, sc);
        };
        for (int st = 0; st < nstage; st += 2) {
            stage(st, bbuf[0], sbuf[0], bbuf[1], sbuf[1]);
            if (st + 1 < nstage) stage(st + 1, bbuf[1], sbuf[1], bbuf[0], sbuf[0]);
        }
        // the last stages loaded repeats of the last one; they must land before the epilogue
        // reuses the LDS
        __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));
        __syncthreads();
    } else {
        // this group's stages: [s0, s0 + ns)
        const int ns = nstage / KG;
        const int s0 = kg * ns;
        load_a(0, s0);
#pragma unroll
        for (int u = 0; u < WD - 1; ++u) load_b(bbuf[u], sbuf[u], s0 + min(u, ns - 1));
#pragma unroll
        for (int u = 1; u < WD; ++u) load_a(u, s0 + min(u, ns - 1));
        store_a(0, 0);
        __syncthreads();

        // The stage body is branch-free: the last stages prefetch (and store to the idle LDS
        // buffer) copies of the last one, so the compiler can count outstanding loads exactly
        // and keep the following stages' loads in flight across the whole compute of this one.
        // Stage st computes from weight buffer st % WD and refills the buffer stage st - 1
        // used with stage st + WD - 1; it refills A set st % WD (stored to LDS before the
        // stage) with stage st + WD and stores set (st + 1) % WD for the next stage.
        auto stage = [&](int st, int set_new, int set_old, const u32x4 (&bc)[NS][SBPS],
                         const uint32_t (&sc)[NS][SCS], u32x4 (&bn)[NS][SBPS],
                         uint32_t (&sn)[NS][SCS]) {
            const int nxt = s0 + min(st + WD - 1, ns - 1);
            load_a(set_new, s0 + min(st + WD, ns - 1));
            load_b(bn, sn, nxt);
            // keep the prefetch at the top (see above)
            __builtin_amdgcn_sched_barrier(0);
            compute_stage(lds_a + (st & 1) * LDS_BUF, bc, sc);
            store_a(set_old, (st + 1) & 1);
            __syncthreads();
        };
        static_assert(WD % 2 == 0, "the LDS buffers alternate with the stage parity");
        // whole rounds of WD stages with no branch between them (a join of paths with different
        // loads in flight makes the compiler wait for nearly all of them), then the rest
        int st = 0;
        for (; st + WD <= ns; st += WD) {
#pragma unroll
            for (int u = 0; u < WD; ++u)
                stage(st + u, u, (u + 1) % WD, bbuf[u], sbuf[u], bbuf[(u + WD - 1) % WD],
                      sbuf[(u + WD - 1) % WD]);
        }
#pragma unroll
        for (int u = 0; u < WD - 1; ++u) {
            if (st + u < ns)
                stage(st + u, u, (u + 1) % WD, bbuf[u], sbuf[u], bbuf[(u + WD - 1) % WD],
                      sbuf[(u + WD - 1) % WD]);
        }
#pragma unroll
        for (int set = 0; set < WD; ++set)
#pragma unroll
            for (int i = 0; i < ACH; ++i) consume(areg[set][i]);
        if constexpr (KG > 1) {
            // groups 1..KG-1 hand their partial tiles to group 0, which adds them in group
            // order (the A buffers are free once the last stage's barrier has passed)
            f32x4* part = (f32x4*)lds;
            auto slot = [&](int g, int m, int c) { return (((g - 1) * 4 + wave) * MA + m) * NS + c; };
            if (kg > 0) {
#pragma unroll
                for (int m = 0; m < MA; ++m)
#pragma unroll
                    for (int c = 0; c < NS; ++c) part[slot(kg, m, c) * kWave + lane] = acc[m][c];
            }
            __syncthreads();
            if (kg == 0) {
                for (int g = 1; g < KG; ++g)
#pragma unroll
                    for (int m = 0; m < MA; ++m)
#pragma unroll
                        for (int c = 0; c < NS; ++c) acc[m][c] += part[slot(g, m, c) * kWave + lane];
            }
            __syncthreads();
        }
    }

    // the last stages prefetched repeats of the last one, which nothing reads
#pragma unroll
    for (int b = 0; b < WD; ++b)
#pragma unroll
        for (int c = 0; c < NS; ++c) {
#pragma unroll
            for (int q = 0; q < SBPS; ++q) consume(bbuf[b][c][q]);
#pragma unroll
            for (int q = 0; q < SCS; ++q) consume(sbuf[b][c][q]);
        }

    if constexpr (KG > 1) {
        if (kg > 0) return;                      // group 0 writes the tile
    }

    // epilogue: lane holds row (lane & 15) of each subtile, 4 consecutive columns per block
    const int q4 = 4 * (lane >> 4);
    if constexpr (!GROUPED && WT != MOE_W_FP16) {
#pragma unroll
        for (int c = 0; c < NS; ++c) {
            const int cbw = SWI ? ob[c % NO] + (c / NO) * nbo : ob[c];
            const f32x4 sc = load4_scale(sp + cbw * 16 + q4);
#pragma unroll
            for (int m = 0; m < MA; ++m) acc[m][c] *= sc;
        }
    }
    // The results leave through LDS (free once the last stage's barrier has passed): each
    // wave writes its rows x (NO * 16) tile into a private region, then reads it back row-wise
    // so every global store writes whole 16-byte pieces of an output row, 8 or 4 lanes per
    // row back to back -- full cache lines instead of 32-byte pieces of 16 rows.
    constexpr int RW = NO * 16;                    // output columns of the wave
    constexpr int RS = tile_epi_stride<ACT, NS>(); // LDS row stride in halves
    f16* region = lds + wave * (BM * RS);
#pragma unroll
    for (int m = 0; m < MA; ++m) {
        const int r = m * 16 + lrow;
        const float rs = (p.row_scale && r < rows) ? p.row_scale[row0 + r] : 1.0f;
#pragma unroll
        for (int c = 0; c < NO; ++c) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (SWI) v[i] = silu(acc[m][c][i]) * acc[m][c + NO][i];
                else if constexpr (ACT == MOE_ACT_RELU) v[i] = fmaxf(acc[m][c][i], 0.0f);
                else v[i] = acc[m][c][i];
                v[i] *= rs;
            }
            const f16x2 lo = {(f16)v[0], (f16)v[1]}, hi = {(f16)v[2], (f16)v[3]};
            uint2 w2;
            w2.x = __builtin_bit_cast(uint32_t, lo);
            w2.y = __builtin_bit_cast(uint32_t, hi);
            *(uint2*)(region + r * RS + c * 16 + q4) = w2;
        }
    }
    constexpr int LPR = RW / 8;                    // lanes per output row (16 bytes each)
    constexpr int RPI = kWave / LPR;               // rows per store instruction
    const int lr = lane / LPR, lc = lane % LPR;
    const int n_out = SWI ? N / 2 : N;
    const int ob0 = (cbg * 4 + wave) * NO;         // first output block of the wave
    const bool col_ok = ob0 + lc / 2 < nbo;
    uint16_t* obase = p.out + ob0 * 16 + lc * 8;
    // a pass may cover more rows than the tile holds (RPI need not divide MA * 16): only rows
    // below `rows` (<= MA * 16 <= BM) are read, so every read stays in the wave's own region
#pragma unroll
    for (int i = 0; i < (MA * 16 + RPI - 1) / RPI; ++i) {
        const int r = i * RPI + lr;
        if (r < rows && col_ok) {
            const u32x4 v = *(const u32x4*)(region + r * RS + lc * 8);
            const int dst = out_dest_row(p, row0 + r);
            if (dst >= 0) *(u32x4*)(obase + (size_t)dst * n_out) = v;
        }
    }
}

// Blocks per CU the tile kernel is built for: two (one for 128-row tiles), three for the 64x256
// tile with 4-bit codes and per-channel scales, whose body fits the 168 registers of three waves
// per SIMD without spilling (with the exponent-of-1024 conversion; the conversion instructions
// need more and keep two).
template <int WT, bool GROUPED, int MS, int NS, int KG, bool NATIVE> constexpr int tile_min_blocks() {
    if (KG != 1 || MS >= 8) return 1;
    return (MS == 4 && NS == 4 && WT == MOE_W_INT4 && !GROUPED && !NATIVE) ? 3 : 2;
}

template <int WT, int ACT, bool GROUPED, int MS, int NS, int KG, bool NATIVE = false>
__global__ __launch_bounds__(256 * KG, (tile_min_blocks<WT, GROUPED, MS, NS, KG, NATIVE>())) void gemm_tile_kernel(GemmParams p, int ncbg, int mt_ub,
                                                           int grid_real, int a_major) {
    constexpr int BM = 16 * MS;
    // the A ring starts the block's LDS (its DMA writes stay aligned); 16 bytes after the body's
    // LDS carry the tile from the wave that looks it up to the others
    constexpr int kBodyHalves = tile_lds_halves<WT, ACT, MS, NS, KG>();
    __shared__ __attribute__((aligned(1024))) f16 lds[kBodyHalves + 8];
    int* const tile_info = (int*)(lds + kBodyHalves);

    // XCD-aware order: hardware block b runs on XCD b % 8.  The real tiles (counted from the
    // offsets, not the host's upper bound) are split into 8 equal contiguous ranges, one per
    // XCD, so that tiles sharing an operand share an L2.  a_major: m-tile slowest, so an
    // activation tile is read by one XCD (for all its column groups); otherwise column group
    // slowest, so an expert's weight block is read by one XCD.
    (void)mt_ub; (void)grid_real;
    int L = -1, mtiles = 0;
    auto logical_mt = [&](int total) {
        mtiles = total;
        const int real = total * ncbg;
        const int G8 = (real + 7) / 8;
        const int j = blockIdx.x / 8;
        L = (blockIdx.x % 8) * G8 + j;
        if (j >= G8 || L >= real) return -1;
        return a_major ? L / ncbg : L % total;
    };
    // one wave looks the tile up and hands it to the others: every block reads the same few
    // offsets at launch, so four waves per block would quadruple the requests on one L2 channel
    if (threadIdx.x < kWave) {
        int mt, e0, r0, nr;
        const bool ok = lookup_m_tile<BM>(p.offsets, p.E, p.R, logical_mt, mt, e0, r0, nr);
        if (threadIdx.x == 0) {
            tile_info[0] = ok ? e0 : -1;
            tile_info[1] = r0;
            tile_info[2] = nr;
            tile_info[3] = ok ? (a_major ? L % ncbg : L / mtiles) : 0;
        }
    }
    __syncthreads();
    const int e = __builtin_amdgcn_readfirstlane(tile_info[0]);
    if (e < 0) return;
    const int row0 = __builtin_amdgcn_readfirstlane(tile_info[1]);
    const int rows = __builtin_amdgcn_readfirstlane(tile_info[2]);
    const int cbg = __builtin_amdgcn_readfirstlane(tile_info[3]);
    // body specialised for the tile's number of 16-row subtiles (1, 2, 3, 4; 5-6 as 6; MS)
    static_assert(MS >= 3, "the subtile cases below assume tiles of at least 48 rows");
    switch ((rows + 15) / 16) {
        case 1: tile_body<WT, ACT, GROUPED, 1, NS, BM, KG, NATIVE>(p, lds, e, row0, rows, cbg); break;
        case 2: tile_body<WT, ACT, GROUPED, 2, NS, BM, KG, NATIVE>(p, lds, e, row0, rows, cbg); break;
        case 3: tile_body<WT, ACT, GROUPED, 3, NS, BM, KG, NATIVE>(p, lds, e, row0, rows, cbg); break;
        case 4:
            tile_body<WT, ACT, GROUPED, (MS >= 4 ? 4 : MS), NS, BM, KG, NATIVE>(p, lds, e, row0, rows, cbg);
            break;
        case 5: case 6:
            tile_body<WT, ACT, GROUPED, (MS >= 6 ? 6 : MS), NS, BM, KG, NATIVE>(p, lds, e, row0, rows, cbg);
            break;
        default: tile_body<WT, ACT, GROUPED, MS, NS, BM, KG, NATIVE>(p, lds, e, row0, rows, cbg); break;
    }
}

// ------------------------------------------------------------------------------------
// Host side: path choice, split choice, launch.
// ------------------------------------------------------------------------------------
static inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

// Output blocks per wave of the stream path.  A unit's activation fragment is 4 KiB for 4-bit
// codes, 2 KiB for 8-bit codes and 1 KiB for fp16 weights, against 1 KiB of weights per column
// block: four weight column blocks per wave for 4-bit codes (two output blocks for SwiGLU,
// whose gate and up blocks pair up), two for 8-bit codes, one for fp16 weights (where more
// column blocks per wave would only mean fewer waves), as far as the output blocks divide.
static int stream_opb(int N, int act, int wtype) {
    const bool swi = act == MOE_ACT_SWIGLU;
    const int nbo = swi ? N / 32 : N / 16;
    const int ncb = wtype == MOE_W_INT4 ? 4 : (wtype == MOE_W_INT8 ? 2 : 1);
    int o = swi ? (ncb >= 2 ? ncb / 2 : 1) : ncb;
    while (o > 1 && nbo % o != 0) o /= 2;
    return o;
}


int gemm_choose_path(int R, int E, int K, int N, int wtype, int act, int forced) {
    (void)K; (void)N; (void)wtype; (void)act;
    if (forced == MOE_PATH_STREAM || forced == MOE_PATH_TILE) return forced;
    // average rows per (possibly) active expert
    const int active = R < E ? R : E;
    const double rows_per_expert = active > 0 ? (double)R / active : 0.0;
    return rows_per_expert >= 16.0 ? MOE_PATH_TILE : MOE_PATH_STREAM;
}

int gemm_choose_split(int R, int E, int K, int N, int wtype, int act, int forced) {
    if (forced >= 1) return forced > MOE_MAX_SPLIT_K ? MOE_MAX_SPLIT_K : forced;
    const int KSB = (wtype == MOE_W_INT4) ? 128 : (wtype == MOE_W_INT8 ? 64 : 32);
    const int nSB = K / KSB;
    const int active = R < E ? R : E;
    const int nbo = (act == MOE_ACT_SWIGLU) ? N / 32 : N / 16;
    const long blocks = (long)active * cdiv(R, active > 0 ? active * 16 : 16) * (nbo / stream_opb(N, act, wtype));
    // Split only a launch with fewer than four blocks per CU: with a few thousand streams,
    // extra waves per SIMD measured no faster (the streams already share each SIMD's VALU
    // issue for the in-register dequantization), while a single-token step (two experts of
    // 4096 x 12800: 400 blocks) took 35.0 against 38.2 us split four ways instead of two; each
    // slice keeps at least 8 super-blocks so its load ring stays filled.
    int s = 1;
    while (s < MOE_MAX_SPLIT_K && blocks * s < 1024 && nSB / (2 * s) >= 8) s *= 2;
    return s;
}

template <int WT, int ACT, bool GROUPED, int PF, int OPB>
static hipError_t side_launch(const GemmParams& p, int ngo, long blocks, const GemmParams& ps,
                              hipStream_t stream) {
    // the dense GEMM's grid: 16-row m-tiles of its R rows x one 16-column output block each,
    // K split over the workgroup's W waves (the grouped GEMM's split, or kDenseSideWaves waves
    // sharing a workgroup with W unsplit grouped blocks)
    const int W = p.split == 1 ? kDenseSideWaves : p.split;
    const long nwg = p.split == 1 ? (blocks + W - 1) / W : blocks;
    const int nbo_s = (ps.act == MOE_ACT_SWIGLU) ? ps.N / 32 : ps.N / 16;
    const long blocks_s = (long)cdiv(ps.R, 16) * nbo_s;
    if (nwg + blocks_s > 0x7fffffffL) return hipErrorInvalidValue;
    constexpr int NCB = (ACT == MOE_ACT_SWIGLU) ? 2 * OPB : OPB;
    const int ncb_s = (ps.act == MOE_ACT_SWIGLU) ? 2 : 1;
    const size_t lds = (size_t)(W - 1) * (NCB > ncb_s ? NCB : ncb_s) * 64 * sizeof(f32x4);
    const unsigned grid = (unsigned)(nwg + blocks_s), threads = 64u * (unsigned)W;
    // the shared experts' first GEMM: SwiGLU (the only activation built for the side GEMM)
    if (ps.act != MOE_ACT_SWIGLU) return hipErrorInvalidValue;
    gemm_stream_side_kernel<WT, ACT, GROUPED, PF, 2, OPB, MOE_ACT_SWIGLU><<<grid, threads, lds, stream>>>(
        p, ngo, (int)blocks, (int)nwg, ps, nbo_s);
    return hipGetLastError();
}

template <int WT, int ACT, bool GROUPED, int OPB>
static hipError_t stream_launch(const GemmParams& p, int ngo, long blocks, hipStream_t stream,
                                const GemmParams* side) {
    constexpr int NCB = (ACT == MOE_ACT_SWIGLU) ? 2 * OPB : OPB;
    const unsigned threads = 64u * (unsigned)p.split;
    const size_t lds = (size_t)(p.split - 1) * NCB * 64 * sizeof(f32x4);
    // weight ring: about 16 KiB per wave for a decode step (few streams, each keeps that much
    // in flight), half that otherwise (registers for more resident waves); the activation
    // ring is two units deep
    constexpr int PF_DEC = NCB >= 4 ? 4 : 8;
    constexpr int PF = NCB >= 4 ? 2 : 4;
    if (side) {
        // only the decode step (integer codes) runs a dense GEMM beside the grouped one
        if constexpr (WT != MOE_W_FP16) {
            if (p.R > 128) return hipErrorInvalidValue;
            return side_launch<WT, ACT, GROUPED, PF_DEC, OPB>(p, ngo, blocks, *side, stream);
        } else {
            return hipErrorInvalidValue;
        }
    }
    if (p.R <= 128)
        gemm_stream_kernel<WT, ACT, GROUPED, PF_DEC, 2, OPB><<<(unsigned)blocks, threads, lds, stream>>>(p, ngo);
    else
        gemm_stream_kernel<WT, ACT, GROUPED, PF, 2, OPB><<<(unsigned)blocks, threads, lds, stream>>>(p, ngo);
    return hipGetLastError();
}

template <int WT, int ACT, bool GROUPED>
static hipError_t stream_dispatch(const GemmParams& p, hipStream_t stream,
                                  const GemmParams* side = nullptr) {
    const int nbo = (ACT == MOE_ACT_SWIGLU) ? p.N / 32 : p.N / 16;
    const int opb = stream_opb(p.N, ACT, WT);
    const int ngo = nbo / opb;
    const int active = p.R < p.E ? p.R : p.E;
    const int mt_ub = cdiv(p.R, 16) + active;
    const long blocks = (long)mt_ub * ngo;
    if (blocks > 0x7fffffffL || p.split < 1 || p.split > MOE_MAX_SPLIT_K) return hipErrorInvalidValue;
    if (p.tiles16 && mt_ub > kDecodeMaxTiles) return hipErrorInvalidValue;   // table bound
    // only the combinations stream_opb chooses are instantiated
    if constexpr (WT == MOE_W_INT4 && ACT != MOE_ACT_SWIGLU) {
        if (opb == 4) return stream_launch<WT, ACT, GROUPED, 4>(p, ngo, blocks, stream, side);
    }
    if constexpr (WT != MOE_W_FP16) {
        if (opb == 2) return stream_launch<WT, ACT, GROUPED, 2>(p, ngo, blocks, stream, side);
    }
    return stream_launch<WT, ACT, GROUPED, 1>(p, ngo, blocks, stream, side);
}

// Tile kernels built with the native int-to-float conversion as well: integer codes, per-channel
// scales, ReLU or no activation, and the tiles gemm_choose_tile picks for those (48x256, 48x128,
// 64x128, 64x256).
template <int WT, int ACT, bool GROUPED, int MS, int NS>
constexpr bool kNativeTile = WT != MOE_W_FP16 && ACT != MOE_ACT_SWIGLU && !GROUPED &&
                             ((MS == 3 && (NS == 4 || NS == 2)) || (MS == 4 && (NS == 2 || NS == 4)));

bool gemm_native_supported(int wtype, int act, int group, int tile) {
    return wtype != MOE_W_FP16 && act != MOE_ACT_SWIGLU && group == 0 &&
           (tile == MOE_TILE_48x256 || tile == MOE_TILE_48x128 || tile == MOE_TILE_64x128 ||
            tile == MOE_TILE_64x256);
}

template <int WT, int ACT, bool GROUPED, int MS, int NS>
static hipError_t tile_launch(const GemmParams& p, hipStream_t stream) {
    constexpr int BM = 16 * MS;
    const int ncbw = p.N / 16;
    const int nbo = (ACT == MOE_ACT_SWIGLU) ? ncbw / 2 : ncbw;
    const int out_per_wave = (ACT == MOE_ACT_SWIGLU) ? NS / 2 : NS;
    const int ncbg = cdiv(nbo, 4 * out_per_wave);
    const int active = p.R < p.E ? p.R : p.E;
    const int mt_ub = cdiv(p.R, BM) + active;
    const long real = (long)mt_ub * ncbg;
    const long grid = (real + 7) / 8 * 8;
    if (grid > 0x7fffffffL) return hipErrorInvalidValue;
    // Which operand to keep XCD-local, by the bytes each order fetches into the XCDs' L2s
    // (4 MiB each; the logical tiles are split into 8 contiguous ranges, one per XCD):
    //   m-tile major: the activation rows once; an expert's weights once per XCD range its
    //     tiles cross (its m-tiles re-read them from the L2), or once per m-tile where one
    //     expert's weights exceed an L2;
    //   column-group major: the weights once; the activation rows once per XCD (at most one
    //     per column group), or once per column group where they exceed an L2.
    // Measured: a single dense expert (the fp16 shared experts, 288 x 2048 x 5632) takes
    // 21 us column-group major against 25 us (its m-tiles fetch every weight once each); the
    // mid-sized routed GEMMs (about one m-tile per expert) read their rows once m-tile major.
    // Well above the ridge point (300 flop per byte) the re-reads come from the last-level
    // cache under MFMA-bound work and the order measured the same (Phi-3.5-MoE-shaped prefill:
    // 1840 against 1855 us): there the m-tile-major order stays.
    const int wbits = (WT == MOE_W_INT4) ? 4 : (WT == MOE_W_INT8 ? 8 : 16);
    const double l2 = 4.0 * 1024 * 1024;
    const double a_bytes = 2.0 * (p.a_rows ? min(p.a_nrows, p.R) : p.R) * p.K;  // distinct rows
    const double w_e = (double)p.K * p.N * wbits / 8.0;
    const double w_bytes = active * w_e;
    const double m_e = fmax(1.0, (double)p.R / ((double)active * BM));      // m-tiles / expert
    const double xcd_range = fmax(1.0, (double)real / 8.0);
    const double s_w = w_e > l2 ? m_e : fmin(m_e, 1.0 + (m_e * ncbg - 1.0) / xcd_range);
    const double s_a = a_bytes > l2 ? (double)ncbg : fmin(8.0, (double)ncbg);
    const bool mfma_bound = 2.0 * p.R * p.K * p.N > 300.0 * (w_bytes + a_bytes);
    const int a_major = (mfma_bound || a_bytes + w_bytes * s_w < w_bytes + a_bytes * s_a) ? 1 : 0;
    // fp16 weights on a grid smaller than the machine: split each tile's K stages over 2 or 4
    // groups of 4 waves in the block (the register-staged A path takes any split that divides
    // the stages; integer codes keep one group)
    // (only splits whose LDS fits a workgroup: the partial tiles grow with the tile)
    constexpr int kLdsMax = 160 * 1024 - 64;
    // four groups put four waves of the block on each SIMD: 128 registers, which only the
    // tiles with at most 8 accumulator fragments per wave fit without spilling
    constexpr bool kFit4 = MS * NS <= 8 && 2 * tile_lds_halves<WT, ACT, MS, NS, 4>() <= kLdsMax;
    constexpr bool kFit2 = 2 * tile_lds_halves<WT, ACT, MS, NS, 2>() <= kLdsMax;
    int kg = 1;
    if constexpr (WT == MOE_W_FP16) {
        const int nstage = p.K / tile_kc<WT>();
        if (kFit4 && real <= 192 && nstage % 4 == 0) kg = 4;
        else if (kFit2 && real <= 384 && nstage % 2 == 0) kg = 2;
    }
    if (kg == 4) {
        if constexpr (WT == MOE_W_FP16 && kFit4)
            gemm_tile_kernel<WT, ACT, GROUPED, MS, NS, 4><<<(unsigned)grid, 1024, 0, stream>>>(
                p, ncbg, mt_ub, (int)real, a_major);
    } else if (kg == 2) {
        if constexpr (WT == MOE_W_FP16 && kFit2)
            gemm_tile_kernel<WT, ACT, GROUPED, MS, NS, 2><<<(unsigned)grid, 512, 0, stream>>>(
                p, ncbg, mt_ub, (int)real, a_major);
    } else if (p.i2f == MOE_I2F_NATIVE) {
        // the conversion-instruction baseline: MT encoder shapes only (per-channel scales, no SwiGLU)
        if constexpr (kNativeTile<WT, ACT, GROUPED, MS, NS>)
            gemm_tile_kernel<WT, ACT, GROUPED, MS, NS, 1, true><<<(unsigned)grid, 256, 0, stream>>>(
                p, ncbg, mt_ub, (int)real, a_major);
        else
            return hipErrorInvalidValue;
    } else {
        gemm_tile_kernel<WT, ACT, GROUPED, MS, NS, 1><<<(unsigned)grid, 256, 0, stream>>>(
            p, ncbg, mt_ub, (int)real, a_major);
    }
    return hipGetLastError();
}

// Block tile of the tile path.  Measured on the layer shapes here (rotated weights, one GEMM per
// call): with integer codes, 48-row tiles beat 64-row ones wherever experts hold few rows (fewer
// padded rows in each expert's last tile, and about two full rounds of blocks instead of one and a
// half); 64x256 stays ahead for group scales once an expert holds about 96 rows or more, and for
// per-channel scales on grids of 1.5 rounds or more of its three blocks per CU (the MT encoder's
// first GEMM: 49 against 53 us; its second GEMM, with a quarter of the columns, stays at 48 rows).  8-bit codes keep to 128-column tiles (their 256-column
// bodies hold too many registers for three waves per SIMD).  fp16 weights: 64x256 when there are
// blocks for four per CU, else 64x128.  128x128 is only used when asked for.
int gemm_choose_tile(int R, int E, int N, int act, int wtype, bool grouped, int forced) {
    if (forced >= MOE_TILE_64x256 && forced <= MOE_TILE_48x128) return forced;
    const int active = R < E ? R : E;
    const int nbo = (act == MOE_ACT_SWIGLU) ? N / 32 : N / 16;
    const int opw = (act == MOE_ACT_SWIGLU) ? 2 : 4;           // output blocks per wave, 256 wide
    const long groups_wide = cdiv(nbo, 4 * opw);
    if (wtype == MOE_W_FP16) {
        const long blocks_wide = groups_wide * (cdiv(R, 64) + active / 2);
        return blocks_wide >= 4L * 256 ? MOE_TILE_64x256 : MOE_TILE_64x128;
    }
    const double rows_per_expert = active > 0 ? (double)R / active : 0.0;
    if (wtype == MOE_W_INT8) {
        const long blocks_wide = groups_wide * (cdiv(R, 64) + active / 2);
        return blocks_wide >= 4L * 256 ? MOE_TILE_48x128 : MOE_TILE_64x128;
    }
    if (grouped && rows_per_expert >= 96.0) return MOE_TILE_64x256;
    // per-channel scales: the 64x256 body runs three blocks per CU; it takes a grid of at least
    // one and a half rounds of those (3 x 256 CUs) for its four-subtile dequantization to pay
    if (!grouped && groups_wide * (cdiv(R, 64) + active / 2) >= 3L * 256 * 3 / 2) return MOE_TILE_64x256;
    const long blocks_48 = groups_wide * (cdiv(R, 48) + active / 2);
    return blocks_48 >= 256 ? MOE_TILE_48x256 : MOE_TILE_48x128;
}

template <int WT, int ACT, bool GROUPED>
static hipError_t tile_dispatch(const GemmParams& p, hipStream_t stream) {
    // A single dense fp16 expert without SwiGLU on fewer than 128 tiles of 64x128 (the shared
    // experts' down projection: 288 x 2816 x 2048 makes 80) takes 64x64 tiles, twice the blocks
    // on a chip it leaves mostly idle (measured 18.4 against 24.7 us; 48x64 tiles 18.8).
    if constexpr (WT == MOE_W_FP16 && ACT != MOE_ACT_SWIGLU) {
        if (p.E == 1 && p.tile == 0 && (long)cdiv(p.R, 64) * (p.N / 128) < 128)
            return tile_launch<WT, ACT, GROUPED, 4, 1>(p, stream);
    }
    switch (gemm_choose_tile(p.R, p.E, p.N, ACT, WT, GROUPED, p.tile)) {
        case MOE_TILE_64x256: return tile_launch<WT, ACT, GROUPED, 4, 4>(p, stream);
        case MOE_TILE_128x128: return tile_launch<WT, ACT, GROUPED, 8, 2>(p, stream);
        case MOE_TILE_48x256: return tile_launch<WT, ACT, GROUPED, 3, 4>(p, stream);
        case MOE_TILE_48x128: return tile_launch<WT, ACT, GROUPED, 3, 2>(p, stream);
        default: return tile_launch<WT, ACT, GROUPED, 4, 2>(p, stream);
    }
}

#define MOE_DISPATCH(FN, p, stream)                                                        \
    do {                                                                                   \
        const bool grouped = (p).group != 0;                                               \
        switch ((p).wtype * 100 + (p).act * 10 + (grouped ? 1 : 0)) {                      \
            case 0 * 100 + 0 * 10 + 0: return FN<MOE_W_INT4, MOE_ACT_NONE, false>(p, stream);   \
            case 0 * 100 + 0 * 10 + 1: return FN<MOE_W_INT4, MOE_ACT_NONE, true>(p, stream);    \
            case 0 * 100 + 1 * 10 + 0: return FN<MOE_W_INT4, MOE_ACT_RELU, false>(p, stream);   \
            case 0 * 100 + 1 * 10 + 1: return FN<MOE_W_INT4, MOE_ACT_RELU, true>(p, stream);    \
            case 0 * 100 + 2 * 10 + 0: return FN<MOE_W_INT4, MOE_ACT_SWIGLU, false>(p, stream); \
            case 0 * 100 + 2 * 10 + 1: return FN<MOE_W_INT4, MOE_ACT_SWIGLU, true>(p, stream);  \
            case 1 * 100 + 0 * 10 + 0: return FN<MOE_W_INT8, MOE_ACT_NONE, false>(p, stream);   \
            case 1 * 100 + 0 * 10 + 1: return FN<MOE_W_INT8, MOE_ACT_NONE, true>(p, stream);    \
            case 1 * 100 + 1 * 10 + 0: return FN<MOE_W_INT8, MOE_ACT_RELU, false>(p, stream);   \
            case 1 * 100 + 1 * 10 + 1: return FN<MOE_W_INT8, MOE_ACT_RELU, true>(p, stream);    \
            case 1 * 100 + 2 * 10 + 0: return FN<MOE_W_INT8, MOE_ACT_SWIGLU, false>(p, stream); \
            case 1 * 100 + 2 * 10 + 1: return FN<MOE_W_INT8, MOE_ACT_SWIGLU, true>(p, stream);  \
            case 2 * 100 + 0 * 10 + 0: return FN<MOE_W_FP16, MOE_ACT_NONE, false>(p, stream);   \
            case 2 * 100 + 1 * 10 + 0: return FN<MOE_W_FP16, MOE_ACT_RELU, false>(p, stream);   \
            case 2 * 100 + 2 * 10 + 0: return FN<MOE_W_FP16, MOE_ACT_SWIGLU, false>(p, stream); \
            default: return hipErrorInvalidValue;                                          \
        }                                                                                  \
    } while (0)

hipError_t launch_gemm_stream(const GemmParams& p, hipStream_t stream) {
    MOE_DISPATCH(stream_dispatch, p, stream);
}

hipError_t launch_gemm_stream_side(const GemmParams& p, const GemmParams& side,
                                   hipStream_t stream) {
    if (side.wtype != MOE_W_FP16 || side.offsets || side.a_rows || side.out_rows || side.tiles16)
        return hipErrorInvalidValue;
    const bool grouped = p.group != 0;
    switch (p.wtype * 100 + p.act * 10 + (grouped ? 1 : 0)) {
        case 0 * 100 + 0 * 10 + 0: return stream_dispatch<MOE_W_INT4, MOE_ACT_NONE, false>(p, stream, &side);
        case 0 * 100 + 0 * 10 + 1: return stream_dispatch<MOE_W_INT4, MOE_ACT_NONE, true>(p, stream, &side);
        case 0 * 100 + 1 * 10 + 0: return stream_dispatch<MOE_W_INT4, MOE_ACT_RELU, false>(p, stream, &side);
        case 0 * 100 + 1 * 10 + 1: return stream_dispatch<MOE_W_INT4, MOE_ACT_RELU, true>(p, stream, &side);
        case 0 * 100 + 2 * 10 + 0: return stream_dispatch<MOE_W_INT4, MOE_ACT_SWIGLU, false>(p, stream, &side);
        case 0 * 100 + 2 * 10 + 1: return stream_dispatch<MOE_W_INT4, MOE_ACT_SWIGLU, true>(p, stream, &side);
        case 1 * 100 + 0 * 10 + 0: return stream_dispatch<MOE_W_INT8, MOE_ACT_NONE, false>(p, stream, &side);
        case 1 * 100 + 0 * 10 + 1: return stream_dispatch<MOE_W_INT8, MOE_ACT_NONE, true>(p, stream, &side);
        case 1 * 100 + 1 * 10 + 0: return stream_dispatch<MOE_W_INT8, MOE_ACT_RELU, false>(p, stream, &side);
        case 1 * 100 + 1 * 10 + 1: return stream_dispatch<MOE_W_INT8, MOE_ACT_RELU, true>(p, stream, &side);
        case 1 * 100 + 2 * 10 + 0: return stream_dispatch<MOE_W_INT8, MOE_ACT_SWIGLU, false>(p, stream, &side);
        case 1 * 100 + 2 * 10 + 1: return stream_dispatch<MOE_W_INT8, MOE_ACT_SWIGLU, true>(p, stream, &side);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_tile(const GemmParams& p, hipStream_t stream) {
    MOE_DISPATCH(tile_dispatch, p, stream);
}

}  // namespace moe
