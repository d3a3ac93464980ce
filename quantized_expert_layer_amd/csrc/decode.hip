// The routed layer for the few tokens of a decode or verify step:
//
//   1. decode_route_sort_kernel  top-k gating of every token, the stable sort of the T*k
//                                slots by expert, and the table of 16-row m-tiles of the
//                                sorted rows, in one workgroup (the keys stay in LDS).
//   2. gemm_stream_kernel        grouped GEMM 1 (gate/up or W1) over all active experts, rows
//                                read through perm, each block's tile read from the table.
//   3. gemm_combine_kernel       grouped GEMM 2 (down or W2): every 16 output columns of the
//                                layer are shared by `nsplit` blocks, each of which streams
//                                its share of the active experts' weight units for all tokens,
//                                so the gate weight, the unpermute and the sum over a token's k
//                                experts happen in its epilogue, in fp32, and no per-slot row
//                                goes to memory.
//   4. combine_reduce_kernel     (nsplit > 1) adds the blocks' fp32 token sums in split order
//                                and the addend, and writes the fp16 output.
//
// With shared experts (fp16, SwiGLU, every token, weight 1) launches 2 and 3 are their _side
// variants: after the routed blocks come the blocks of the shared experts' dense first GEMM
// (into sh_h) and second GEMM (into sh_y), and sh_y is the addend of launch 4.
//
// "Specter" summary, Method steps, step 5 and Technical novelty: the draft model's expert
// sub-computations run in one fused launch, and the verify step groups tokens by expert into
// one GEMM per expert and scatters the results back.  "Who Says Elephants Can't Run",
// section 3 workflow: sort by expert index, permute, grouped GEMM, unpermute with
// expert_scale.  Here the second GEMM's launch also does the unpermute and the combine.
#include "common.hpp"
#include "launch.hpp"
#include "stream.hpp"
#include "route.hpp"
#include "sort.hpp"

namespace moe {

// ------------------------------------------------------------------------------------
// 1. Gating + sort + tile table.  One block of kSortWaves waves; the 16-lane rows route one
//    token each (wave w tokens 4w .. 4w + 3); then wave 0 sorts the slots (few enough that one
//    wave beats the block-wide sort) and lists the 16-row m-tiles of every expert's sorted rows
//    (expert order).
// ------------------------------------------------------------------------------------
template <int PER_LANE>
__global__ __launch_bounds__(kSortWaves * kWave) void decode_route_sort_kernel(
    const float* __restrict__ logits, const uint8_t* __restrict__ active, int T, int E, int k,
    int gate_all, int32_t* __restrict__ ids, float* __restrict__ wts, DecodeWs ws) {
    __shared__ int keys[MOE_DECODE_MAX_ROWS];
    __shared__ float kw[MOE_DECODE_MAX_ROWS];
    __shared__ int cnt[MOE_MAX_EXPERTS];
    __shared__ int offs[MOE_MAX_EXPERTS + 1];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    // one token per 16-lane row: wave w routes tokens 4w .. 4w + 3 (T <= 64 = 16 waves x 4)
    if (4 * wave < T) {
        const int t = 4 * wave + (lane >> 4);
        const int j = lane & 15;
        // a finished token (active[t] == 0) takes no expert: e = -1, w = 0
        const bool live = t < T && (!active || active[t]);
        int e;
        float w;
        topk_row<PER_LANE>(live ? logits + (size_t)t * E : nullptr, E, k, gate_all, lane, e, w);
        if (t < T && j < k) {
            ids[t * k + j] = e;
            wts[t * k + j] = w;
            keys[t * k + j] = e;
            kw[t * k + j] = w;
        }
    }
    // the other waves hand over LDS keys only (their global stores need not land first)
    lds_barrier();
    if (wave != 0) return;
    sort_wave(T * k, E, [&](int f) { return keys[f]; }, [&](int f) { return kw[f]; }, cnt, offs,
              ws.perm, ws.inv_perm, ws.offsets, ws.w_perm);
    lds_wave_fence();
    // tile table: expert e's rows offs[e] .. offs[e+1]-1 in tiles of 16, experts in order.
    // At most sum_e ceil(c_e / 16) <= T*k / 16 + E <= kDecodeMaxTiles entries.
    int base = 0;
    for (int c0 = 0; c0 < E; c0 += kWave) {
        const int e = c0 + lane;
        int lo = 0, n = 0;
        if (e < E) {
            lo = offs[e];
            n = offs[e + 1] - lo;
        }
        const int nt = (n + 15) >> 4;
        const int incl = wave_incl_scan(nt);
        const int b0 = base + incl - nt;
        for (int i = 0; i < nt; ++i)
            ws.tiles[1 + b0 + i] = tile16_pack(e, lo + 16 * i, min(16, n - 16 * i));
        base += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    if (lane == 0) ws.tiles[0] = base;
}

// Second GEMM: waves per block, and 16-column blocks per wave (one activation fragment serves
// the weight units of all of them: a CU's vector-memory pipeline moves 64 bytes per clock, and
// a 16-row activation fragment is four times the bytes of a 1 KiB weight unit).
constexpr int kCombineWaves = 8;
constexpr int kCombineNcb = 2;

// ------------------------------------------------------------------------------------
// 3. Grouped GEMM 2 + gate weight + unpermute + combine.
//
//   grid   = (N / (16 NCB) column groups) x nsplit; block = S waves.
//   work   = the units (m-tile, super-block) of every active expert for the block's 16 NCB
//            columns: m-tiles are the 16-row tiles of each expert's sorted rows (from the tile
//            table), super-blocks the 1 KiB weight units along K of each 16-column block.  The
//            S * nsplit waves that share a column group take equal consecutive ranges of that
//            unit sequence (split s the s-th group of S ranges), so every weight byte of the
//            active experts is read by one wave, and a wave loads a unit's activation fragment
//            once for its NCB column blocks.
//   math   = as the stream path: MFMA 16x16x32 with the activation (H rows) first, so lane l
//            holds column (l & 15) of rows 4(l >> 4) .. +3; group scales multiply the fp32
//            sum of a super-block, a per-channel scale the sum of an m-tile.
//   combine= when a wave finishes an m-tile (or its range), each valid row p adds
//            w_perm[p] * y[p] into the wave's fp32 token sums in LDS at token perm[p] / k.
//            An expert holds at most one slot of a token, so the lanes of one such update
//            write distinct words.  The block then adds its S waves in the order 0..S-1: with
//            nsplit == 1 it adds the addend and writes the fp16 output, otherwise it writes
//            its fp32 sums to part[split], which combine_reduce_kernel adds in split order.
//            Every sum has a fixed order, so results are deterministic.  (The blocks of one
//            column group do not hand their sums to the last of them: that needs a
//            device-scope release per block, which on this chip writes back the whole L2 of
//            the XCD and cost more than the second launch.)
// ------------------------------------------------------------------------------------
// Block `bid` of the launch; tok_sum: LDS for [S][T][NC] token sums.  TAG: a specialization
// of its own per calling kernel.
template <int WT, bool GROUPED, int PF, int PA, int NCB, int TAG = 0>
__device__ __forceinline__ void combine_body(const CombineParams& p, int bid,
                                             float* __restrict__ tok_sum) {
    constexpr int KSB = WTraits<WT>::KSB;
    constexpr int KSTEPS = KSB / 32;
    constexpr int NC = 16 * NCB;                              // columns of a block
    constexpr bool CHANNEL = !GROUPED && WT != MOE_W_FP16;   // per-channel scales
    __shared__ int tile_v[kDecodeMaxTiles];
    __shared__ int tok_of[MOE_DECODE_MAX_ROWS];
    __shared__ float gate_of[MOE_DECODE_MAX_ROWS];

    const int lane = threadIdx.x & (kWave - 1);
    // wave index, held in a scalar register (the compiler cannot see it is wave-uniform)
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int S = blockDim.x / kWave;
    const int ncb = p.N / 16;
    const int ncg = p.N / NC;
    const int cg = bid % ncg;
    const int sp = bid / ncg;
    const int K = p.K, N = p.N, T = p.T, R = p.R;
    const int nSB = K / KSB;
    // the table's count: at most kDecodeMaxTiles by construction, clamped all the same
    const int n_tiles = min(max(p.tiles[0], 0), kDecodeMaxTiles);

    for (int i = threadIdx.x; i < S * T * NC; i += blockDim.x) tok_sum[i] = 0.0f;
    for (int i = threadIdx.x; i < R; i += blockDim.x) {
        const int f = p.perm[i];
        tok_of[i] = (f >= 0 && f < T * p.k) ? f / p.k : -1;
        gate_of[i] = p.w_perm[i];
    }
    for (int i = threadIdx.x; i < n_tiles; i += blockDim.x) tile_v[i] = p.tiles[1 + i];
    lds_barrier();

    // this wave's unit range [ua, ub)
    const int U = n_tiles * nSB;
    const int G = S * p.nsplit;
    const int chunk = (U + G - 1) / G;
    const int ua = min(U, (sp * S + w) * chunk), ub = min(U, ua + chunk);
    const int NG = GROUPED ? K / 128 : 1;
    float* my_sum = tok_sum + w * T * NC;
    int col[NCB];
#pragma unroll
    for (int c = 0; c < NCB; ++c) col[c] = (cg * NCB + c) * 16 + (lane & 15);

    if (ua < ub) {
        // Two rings, as in the stream path: weights PF units ahead, activations (H rows, in
        // L2) PA ahead, each with its own issue cursor over the unit sequence.  Tiles come from
        // the sort, so their rows lie in [0, R) and their expert in [0, E).
        static_assert(PF % PA == 0, "activation slots follow the weight slots");
        u32x4 braw[PF][NCB];
        f16x8 araw[PA][KSTEPS];
        uint32_t sraw[PF][NCB] = {};

        struct Cursor {
            int iu, im, ik, e, r0, n;
        };
        // table entries are wave-uniform: read into scalar registers
        auto tile_at = [&](int i) { return __builtin_amdgcn_readfirstlane(tile_v[i]); };
        auto start = [&](Cursor& c) {
            c.iu = ua;
            c.im = ua / nSB;
            c.ik = ua % nSB;
            tile16_unpack(tile_at(c.im), c.e, c.r0, c.n);
        };
        // past the range the last unit is issued again (never consumed)
        auto advance = [&](Cursor& c) {
            if (c.iu + 1 < ub) {
                ++c.iu;
                if (++c.ik == nSB) {
                    c.ik = 0;
                    ++c.im;
                    tile16_unpack(tile_at(c.im), c.e, c.r0, c.n);
                }
            }
        };
        Cursor cw, ca;
        start(cw);
        start(ca);
        auto issue_w = [&](int slot) {
#pragma unroll
            for (int c = 0; c < NCB; ++c) {
                const u32x4* wp = (const u32x4*)p.w +
                                  ((size_t)(cw.e * ncb + cg * NCB + c) * nSB + cw.ik) * kWave + lane;
                braw[slot][c] = load_weights16(wp);
                if constexpr (GROUPED)
                    sraw[slot][c] = p.scales[((size_t)cw.e * NG + ((cw.ik * KSB) >> 7)) * N + col[c]];
                else if constexpr (CHANNEL)
                    sraw[slot][c] = p.scales[(size_t)cw.e * N + col[c]];
            }
            advance(cw);
        };
        auto issue_a = [&](int slot) {
            const int arow = ca.r0 + min(lane & 15, ca.n - 1);
            const f16x8* ap = (const f16x8*)(p.h + (size_t)arow * K + ca.ik * KSB) + (lane >> 4);
#pragma unroll
            for (int j = 0; j < KSTEPS; ++j) araw[slot][j] = ap[j * 4];
            advance(ca);
        };

        const I2F4Consts k4;
        const f16x2 one2 = {(f16)1.0f, (f16)1.0f};
        f32x4 acc[NCB];
#pragma unroll
        for (int c = 0; c < NCB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        int cu = ua, cm = ua / nSB, ck = ua % nSB;      // consume cursor
        auto flush = [&](const uint32_t (&sbits)[NCB]) {
            int te, r0, nr;
            tile16_unpack(tile_at(cm), te, r0, nr);
#pragma unroll
            for (int c = 0; c < NCB; ++c) {
                f32x4 v = acc[c];
                if constexpr (CHANNEL) {
                    const float s = f16_bits_to_f32((uint16_t)sbits[c]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] *= s;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * (lane >> 4) + i;
                    if (r < nr) {
                        const int t = tok_of[r0 + r];
                        if (t >= 0) my_sum[t * NC + c * 16 + (lane & 15)] += gate_of[r0 + r] * v[i];
                    }
                }
                acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        };
        auto consume_unit = [&](int slot, int aslot) {
#pragma unroll
            for (int c = 0; c < NCB; ++c) {
                if constexpr (GROUPED) {
                    // two interleaved chains (even / odd K-steps): a dependent MFMA chain stalls
                    f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < KSTEPS; ++j) {
                        if (j & 1) t1 = mfma16x16x32(araw[aslot][j], weight_frag<WT, false>(braw[slot][c], j, one2, k4), t1);
                        else t0 = mfma16x16x32(araw[aslot][j], weight_frag<WT, false>(braw[slot][c], j, one2, k4), t0);
                    }
                    const f32x4 t = t0 + t1;
                    const float s = f16_bits_to_f32((uint16_t)sraw[slot][c]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[c][i] = __builtin_fmaf(t[i], s, acc[c][i]);
                } else {
#pragma unroll
                    for (int j = 0; j < KSTEPS; ++j)
                        acc[c] = mfma16x16x32(araw[aslot][j], weight_frag<WT, false>(braw[slot][c], j, one2, k4), acc[c]);
                }
            }
            if (ck == nSB - 1 || cu == ub - 1) flush(sraw[slot]);
            ++cu;
            if (++ck == nSB) {
                ck = 0;
                ++cm;
            }
        };

#pragma unroll
        for (int u = 0; u < PF; ++u) issue_w(u);
#pragma unroll
        for (int u = 0; u < PA; ++u) issue_a(u);
        int kc = ua;
        for (; kc + PF <= ub; kc += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                consume_unit(u, u % PA);
                issue_w(u);
                issue_a(u % PA);
            }
        }
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            if (kc + u < ub) {
                consume_unit(u, u % PA);
                issue_a(u % PA);
            }
        }
        // every ring slot holds a load (a repeat of the last unit where the range ran out)
#pragma unroll
        for (int u = 0; u < PF; ++u) {
#pragma unroll
            for (int c = 0; c < NCB; ++c) {
                consume(braw[u][c]);
                consume(sraw[u][c]);
            }
        }
#pragma unroll
        for (int u = 0; u < PA; ++u)
#pragma unroll
            for (int j = 0; j < KSTEPS; ++j) consume(araw[u][j]);
    }
    lds_barrier();

    // the S waves' token sums, added in wave order; then the addend and the fp16 output, or
    // this split's fp32 sums
    const int c0 = cg * NC;
    for (int i = threadIdx.x; i < T * NC; i += blockDim.x) {
        const int t = i / NC, c = i % NC;
        float v = 0.0f;
        for (int s = 0; s < S; ++s) v += tok_sum[(s * T + t) * NC + c];
        if (p.nsplit > 1) {
            p.part[((size_t)sp * T + t) * N + c0 + c] = v;
        } else {
            if (p.addend) v += f16_bits_to_f32(p.addend[(size_t)t * N + c0 + c]);
            p.out[(size_t)t * N + c0 + c] = f32_to_f16_bits(v);
        }
    }
}

template <int WT, bool GROUPED, int PF, int PA, int NCB>
__global__ __launch_bounds__(64 * kCombineWaves) void gemm_combine_kernel(CombineParams p) {
    extern __shared__ float tok_sum[];                        // [S][T][NC]
    combine_body<WT, GROUPED, PF, PA, NCB>(p, blockIdx.x, tok_sum);
}

// The second launch with the shared experts' second GEMM beside it ([S] Method step 5): blocks
// [0, nb) run the routed GEMM 2 + combine above (writing fp32 partials, which the reduction adds
// with the shared experts' output), the rest the dense fp16 GEMM ps (H_shared . W2_shared over
// every token, 8 waves splitting K).
template <int WT, bool GROUPED, int PF, int PA, int NCB>
__global__ __launch_bounds__(64 * kCombineWaves) void gemm_combine_side_kernel(CombineParams p, int nb,
                                                                              GemmParams ps,
                                                                              int ngo_s) {
    extern __shared__ float dyn[];
    if ((int)blockIdx.x < nb)
        combine_body<WT, GROUPED, PF, PA, NCB, 1>(p, blockIdx.x, dyn);
    else
        stream_body<MOE_W_FP16, MOE_ACT_NONE, false, 8, 2, 1, 64 + WT * 2 + (GROUPED ? 1 : 0)>(
            ps, ngo_s, blockIdx.x - nb, blockDim.x / kWave,
            __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), (f32x4*)dyn);
}

// ------------------------------------------------------------------------------------
// 4. out[t, c] = fp16( part[0, t, c] + .. + part[nsplit - 1, t, c] + addend[t, c] ), fp32 in
//    that order; one thread per 4 consecutive columns.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_reduce_kernel(const float* __restrict__ part,
                                                             int nsplit,
                                                             const uint16_t* __restrict__ addend,
                                                             uint16_t* __restrict__ out, int T,
                                                             int N) {
    const int n4 = N / 4;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T * n4) return;
    const size_t at = (size_t)(i / n4) * N + (size_t)(i % n4) * 4;
    f32x4 v = *(const f32x4*)(part + at);
    for (int s = 1; s < nsplit; ++s) v += *(const f32x4*)(part + (size_t)s * T * N + at);
    if (addend) v += load4_f16(addend + at);
    store4_f16_bits(out + at, v);
}

// ------------------------------------------------------------------------------------
// Host side.
// ------------------------------------------------------------------------------------
// Blocks of the second GEMM: enough that every CU holds two of them (the 16-column blocks
// of a d = 2048 layer number only 128), so each wave's share of the weight units is short
// enough to be in flight at once.
constexpr int kCombineTargetBlocks = 256;
constexpr int kCombineMaxSplit = 8;

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int decode_combine_split(int d, bool shared) {
    const int ncg = d / (16 * kCombineNcb);
    int s = 1;
    while (s < kCombineMaxSplit && ncg * s < kCombineTargetBlocks) s *= 2;
    // with shared experts the reduction launch adds their output: at least two splits
    return (shared && s < 2) ? 2 : s;
}

size_t decode_workspace_layout(int T, int k, int E, int d, int inter, int wtype,
                               int shared_inter, DecodeWs* ws, char* base) {
    (void)wtype;
    const size_t R = (size_t)T * k;
    const int nsplit = decode_combine_split(d, shared_inter > 0);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return base ? base + at : nullptr;
    };
    char* perm = take(R * 4);
    char* inv = take(R * 4);
    char* offs = take(((size_t)E + 1) * 4);
    char* wperm = take(R * 4);
    char* tiles = take((size_t)(1 + kDecodeMaxTiles) * 4);
    char* h = take(R * (size_t)inter * 2);
    char* part = take(nsplit > 1 ? (size_t)nsplit * T * d * 4 : 0);
    char* sh_h = take((size_t)T * shared_inter * 2);
    char* sh_y = take(shared_inter > 0 ? (size_t)T * d * 2 : 0);
    if (ws) {
        ws->sh_h = shared_inter > 0 ? (uint16_t*)sh_h : nullptr;
        ws->sh_y = shared_inter > 0 ? (uint16_t*)sh_y : nullptr;
        ws->perm = (int32_t*)perm;
        ws->inv_perm = (int32_t*)inv;
        ws->offsets = (int32_t*)offs;
        ws->w_perm = (float*)wperm;
        ws->tiles = (int32_t*)tiles;
        ws->h = (uint16_t*)h;
        ws->part = nsplit > 1 ? (float*)part : nullptr;
    }
    return off;
}

template <int WT, bool GROUPED>
static hipError_t combine_launch(const CombineParams& p, hipStream_t stream,
                                 const GemmParams* side) {
    const unsigned grid = (unsigned)(p.N / (16 * kCombineNcb) * p.nsplit);
    size_t lds = (size_t)kCombineWaves * p.T * 16 * kCombineNcb * sizeof(float);
    if (side) {
        // the shared experts' second GEMM beside the routed one: its output is the addend,
        // added by the reduction launch below (so the combine blocks must write partials);
        // integer-coded routed weights only
        if constexpr (WT == MOE_W_FP16) {
            return hipErrorInvalidValue;
        } else {
            if (p.nsplit < 2 || side->split != kCombineWaves || side->act != MOE_ACT_NONE)
                return hipErrorInvalidValue;
            const int ngo_s = side->N / 16;
            const long blocks_s = (long)((side->R + 15) / 16) * ngo_s;
            const size_t lds_s = (size_t)(kCombineWaves - 1) * 64 * sizeof(f32x4);
            if (lds_s > lds) lds = lds_s;
            gemm_combine_side_kernel<WT, GROUPED, 4, 2, kCombineNcb>
                <<<grid + (unsigned)blocks_s, kCombineWaves * kWave, lds, stream>>>(
                    p, (int)grid, *side, ngo_s);
        }
    } else {
        gemm_combine_kernel<WT, GROUPED, 4, 2, kCombineNcb><<<grid, kCombineWaves * kWave, lds, stream>>>(p);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || p.nsplit == 1) return err;
    const int threads = p.T * (p.N / 4);
    combine_reduce_kernel<<<(threads + 255) / 256, 256, 0, stream>>>(p.part, p.nsplit, p.addend,
                                                                    p.out, p.T, p.N);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    DecodeWs ws;
    decode_workspace_layout(a.T, a.k, a.E, a.d, a.inter, a.wtype, a.sw1 ? a.shared_inter : 0, &ws,
                            (char*)a.ws);
    const int R = a.T * a.k;

    static_assert(MOE_DECODE_MAX_TOKENS <= 4 * kSortWaves, "one token per 16-lane row");
    if (a.E <= 16)
        decode_route_sort_kernel<1><<<1, kSortWaves * kWave, 0, stream>>>(
            a.logits, a.active, a.T, a.E, a.k, a.gate_all, a.ids, a.wts, ws);
    else if (a.E <= 64)
        decode_route_sort_kernel<4><<<1, kSortWaves * kWave, 0, stream>>>(
            a.logits, a.active, a.T, a.E, a.k, a.gate_all, a.ids, a.wts, ws);
    else if (a.E <= 128)
        decode_route_sort_kernel<8><<<1, kSortWaves * kWave, 0, stream>>>(
            a.logits, a.active, a.T, a.E, a.k, a.gate_all, a.ids, a.wts, ws);
    else
        decode_route_sort_kernel<16><<<1, kSortWaves * kWave, 0, stream>>>(
            a.logits, a.active, a.T, a.E, a.k, a.gate_all, a.ids, a.wts, ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    const int n1 = (a.act == MOE_ACT_SWIGLU) ? 2 * a.inter : a.inter;
    GemmParams g;
    g.a = a.x;
    g.a_rows = ws.perm;
    g.a_div = a.k;
    g.a_nrows = a.T;
    g.out_rows = nullptr;
    g.out_nrows = R;
    g.offsets = ws.offsets;
    g.w = a.w1;
    g.scales = a.s1;
    g.row_scale = nullptr;
    g.out = ws.h;
    g.R = R;
    g.E = a.E;
    g.K = a.d;
    g.N = n1;
    g.wtype = a.wtype;
    g.group = a.group;
    g.act = a.act;
    g.split = gemm_choose_split(R, a.E, a.d, n1, a.wtype, a.act, 0);
    g.tile = 0;
    g.i2f = MOE_I2F_TRICK;
    g.tiles16 = ws.tiles;
    // the shared experts (fp16, every token): their first GEMM runs beside the routed GEMM 1,
    // their second beside the routed GEMM 2, and the reduction adds their output
    const bool shared = a.sw1 != nullptr;
    GemmParams sg1, sg2;
    if (shared) {
        sg1.a = a.x;
        sg1.a_rows = nullptr;
        sg1.a_div = 1;
        sg1.a_nrows = a.T;
        sg1.out_rows = nullptr;
        sg1.out_nrows = a.T;
        sg1.offsets = nullptr;
        sg1.w = a.sw1;
        sg1.scales = nullptr;
        sg1.row_scale = nullptr;
        sg1.out = ws.sh_h;
        sg1.R = a.T;
        sg1.E = 1;
        sg1.K = a.d;
        sg1.N = 2 * a.shared_inter;
        sg1.wtype = MOE_W_FP16;
        sg1.group = 0;
        sg1.act = MOE_ACT_SWIGLU;
        sg1.split = g.split;
        sg1.tile = 0;
        sg1.i2f = MOE_I2F_TRICK;
        sg1.tiles16 = nullptr;
        sg2 = sg1;
        sg2.a = ws.sh_h;
        sg2.w = a.sw2;
        sg2.out = ws.sh_y;
        sg2.K = a.shared_inter;
        sg2.N = a.d;
        sg2.act = MOE_ACT_NONE;
        sg2.split = kCombineWaves;
    }
    if (shared && R <= 128) {
        err = launch_gemm_stream_side(g, sg1, stream);
    } else {
        // (more routed rows than the side launch takes: the shared GEMM 1 follows on its own)
        err = launch_gemm_stream(g, stream);
        if (err == hipSuccess && shared) err = launch_gemm_stream(sg1, stream);
    }
    if (err != hipSuccess) return err;

    CombineParams c;
    c.h = ws.h;
    c.tiles = ws.tiles;
    c.perm = ws.perm;
    c.w_perm = ws.w_perm;
    c.w = a.w2;
    c.scales = a.s2;
    c.addend = shared ? ws.sh_y : a.addend;
    c.out = a.out;
    c.part = ws.part;
    c.R = R;
    c.E = a.E;
    c.K = a.inter;
    c.N = a.d;
    c.T = a.T;
    c.k = a.k;
    c.nsplit = decode_combine_split(a.d, shared);
    // the addend (e.g. shared experts computed on another stream) is first read here
    if (a.addend_ready && !shared) {
        err = hipStreamWaitEvent(stream, (hipEvent_t)a.addend_ready, 0);
        if (err != hipSuccess) return err;
    }
    const GemmParams* side = shared ? &sg2 : nullptr;
    const bool grouped = a.group != 0;
    switch (a.wtype * 2 + (grouped ? 1 : 0)) {
        case MOE_W_INT4 * 2 + 0: return combine_launch<MOE_W_INT4, false>(c, stream, side);
        case MOE_W_INT4 * 2 + 1: return combine_launch<MOE_W_INT4, true>(c, stream, side);
        case MOE_W_INT8 * 2 + 0: return combine_launch<MOE_W_INT8, false>(c, stream, side);
        case MOE_W_INT8 * 2 + 1: return combine_launch<MOE_W_INT8, true>(c, stream, side);
        case MOE_W_FP16 * 2 + 0:
            if (shared) return hipErrorInvalidValue;
            return combine_launch<MOE_W_FP16, false>(c, stream, nullptr);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
