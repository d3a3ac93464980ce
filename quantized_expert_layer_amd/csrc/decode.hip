// The routed layer for the few tokens of a decode or verify step, in three launches:
//
//   1. decode_route_sort_kernel  top-k gating of every token and the stable sort of the T*k
//                                slots by expert, in one workgroup (the keys stay in LDS).
//   2. gemm_stream_kernel        grouped GEMM 1 (gate/up or W1) over all active experts, rows
//                                read through perm (the stream path of the grouped GEMM).
//   3. gemm_combine_kernel       grouped GEMM 2 (down or W2) whose blocks own 16 output
//                                columns of the layer for every token, so the gate weight,
//                                the unpermute and the sum over a token's k experts happen in
//                                its epilogue, in fp32, and no per-slot row goes to memory.
//
// "Specter" summary, Method steps, step 5 and Technical novelty: the draft model's expert
// sub-computations run in one fused launch, and the verify step groups tokens by expert into
// one GEMM per expert and scatters the results back.  "Who Says Elephants Can't Run",
// section 3 workflow: sort by expert index, permute, grouped GEMM, unpermute with
// expert_scale.  Here the second GEMM's launch also does the unpermute and the combine.
#include "common.hpp"
#include "launch.hpp"
#include "route.hpp"
#include "sort.hpp"

namespace moe {

// ------------------------------------------------------------------------------------
// 1. Gating + sort.  One block of kSortWaves waves; wave w routes tokens w, w + 16, ...;
//    then wave 0 sorts the slots (few enough that one wave beats the block-wide sort).
// ------------------------------------------------------------------------------------
template <int PER_LANE>
__global__ __launch_bounds__(kSortWaves * kWave) void decode_route_sort_kernel(
    const float* __restrict__ logits, const uint8_t* __restrict__ active, int T, int E, int k,
    int gate_all, int32_t* __restrict__ ids, float* __restrict__ wts, DecodeWs ws) {
    __shared__ int keys[MOE_DECODE_MAX_ROWS];
    __shared__ float kw[MOE_DECODE_MAX_ROWS];
    __shared__ int cnt[MOE_MAX_EXPERTS];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    for (int t = wave; t < T; t += kSortWaves) {
        int e = -1;              // a finished token (active[t] == 0) takes no expert
        float w = 0.0f;
        if (!active || active[t])
            topk_token<PER_LANE>(logits + (size_t)t * E, E, k, gate_all, lane, e, w);
        if (lane < k) {
            ids[t * k + lane] = e;
            wts[t * k + lane] = w;
            keys[t * k + lane] = e;
            kw[t * k + lane] = w;
        }
    }
    __syncthreads();
    if (wave != 0) return;
    sort_wave(T * k, E, [&](int f) { return keys[f]; }, [&](int f) { return kw[f]; }, cnt,
              ws.perm, ws.inv_perm, ws.offsets, ws.w_perm);
}

// ------------------------------------------------------------------------------------
// 3. Grouped GEMM 2 + gate weight + unpermute + combine.
//
//   grid   = N / 16 column blocks; block = S waves.
//   work   = the units (m-tile, super-block) of every active expert for the block's 16
//            columns: m-tiles are the 16-row tiles of each expert's sorted rows, super-blocks
//            the 1 KiB weight units along K.  Wave w takes the w-th of S equal ranges of the
//            unit sequence, so every weight byte of the active experts is read by one wave.
//   math   = as the stream path: MFMA 16x16x32 with the activation (H rows) first, so lane l
//            holds column (l & 15) of rows 4(l >> 4) .. +3; group scales multiply the fp32
//            sum of a super-block, a per-channel scale the sum of an m-tile.
//   combine= when a wave finishes an m-tile (or its range), each valid row p adds
//            w_perm[p] * y[p] into the wave's fp32 token sums in LDS at token perm[p] / k.
//            An expert holds at most one slot of a token, so the lanes of one such update
//            write distinct words.  The block then adds its S waves in the order 0..S-1 and
//            the addend, and writes the fp16 output.  Every sum has a fixed order, so results
//            are deterministic.  (Splitting a column block's units over several blocks would
//            need a device-wide release before the last block adds the parts; on this chip
//            that writes back the whole L2 of the XCD per block and cost more than it gained.)
// ------------------------------------------------------------------------------------
constexpr int kCombineMaxTiles = MOE_DECODE_MAX_ROWS / 16 + MOE_MAX_EXPERTS;

template <int WT, bool GROUPED, int PF>
__global__ __launch_bounds__(64 * MOE_MAX_SPLIT_K) void gemm_combine_kernel(CombineParams p) {
    constexpr int KSB = WTraits<WT>::KSB;
    constexpr int KSTEPS = KSB / 32;
    constexpr bool CHANNEL = !GROUPED && WT != MOE_W_FP16;   // per-channel scales
    __shared__ int tile_e[kCombineMaxTiles], tile_r0[kCombineMaxTiles], tile_n[kCombineMaxTiles];
    __shared__ int tok_of[MOE_DECODE_MAX_ROWS];
    __shared__ float gate_of[MOE_DECODE_MAX_ROWS];
    __shared__ int n_tiles;
    extern __shared__ float tok_sum[];                        // [S][T][16]

    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int S = blockDim.x / kWave;
    const int ncb = p.N / 16;
    const int cb = blockIdx.x;
    const int K = p.K, N = p.N, T = p.T, R = p.R;
    const int nSB = K / KSB;
    const int col = cb * 16 + (lane & 15);

    for (int i = threadIdx.x; i < S * T * 16; i += blockDim.x) tok_sum[i] = 0.0f;
    for (int i = threadIdx.x; i < R; i += blockDim.x) {
        const int f = p.perm[i];
        tok_of[i] = (f >= 0 && f < T * p.k) ? f / p.k : -1;
        gate_of[i] = p.w_perm[i];
    }
    // m-tile table (wave 0): experts in chunks of 64 lanes, prefix sum of their tile counts
    if (w == 0) {
        int base = 0;
        for (int c0 = 0; c0 < p.E; c0 += kWave) {
            const int e = c0 + lane;
            int lo = 0, hi = 0;
            if (e < p.E) {
                lo = min(max(p.offsets[e], 0), R);
                hi = min(max(p.offsets[e + 1], 0), R);
            }
            const int cnt = max(hi - lo, 0);
            const int nt = (cnt + 15) / 16;
            const int incl = wave_incl_scan(nt);
            const int b0 = base + incl - nt;
            for (int i = 0; i < nt && b0 + i < kCombineMaxTiles; ++i) {
                tile_e[b0 + i] = e;
                tile_r0[b0 + i] = lo + 16 * i;
                tile_n[b0 + i] = min(16, cnt - 16 * i);
            }
            base += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
        if (lane == 0) n_tiles = min(base, kCombineMaxTiles);
    }
    __syncthreads();

    // this wave's unit range [ua, ub)
    const int U = n_tiles * nSB;
    const int chunk = (U + S - 1) / S;
    const int ua = min(U, w * chunk), ub = min(U, ua + chunk);
    const int G = GROUPED ? K / 128 : 1;
    float* my_sum = tok_sum + w * T * 16;

    if (ua < ub) {
        u32x4 braw[PF];
        f16x8 araw[PF][KSTEPS];
        uint32_t sraw[PF] = {};

        // issue cursor: unit (im, ik); m-tile fields cached in registers
        int iu = ua, im = ua / nSB, ik = ua % nSB;
        int ie = tile_e[im], ir0 = tile_r0[im], inr = tile_n[im];
        auto issue = [&](int slot) {
            const u32x4* wp = (const u32x4*)p.w + ((size_t)(ie * ncb + cb) * nSB + ik) * kWave + lane;
            braw[slot] = load_weights16(wp);
            if constexpr (GROUPED)
                sraw[slot] = p.scales[((size_t)ie * G + ((ik * KSB) >> 7)) * N + col];
            else if constexpr (CHANNEL)
                sraw[slot] = p.scales[(size_t)ie * N + col];
            const int arow = ir0 + min(lane & 15, inr - 1);
            const f16x8* ap = (const f16x8*)(p.h + (size_t)arow * K + ik * KSB) + (lane >> 4);
#pragma unroll
            for (int j = 0; j < KSTEPS; ++j) araw[slot][j] = ap[j * 4];
            // advance; past the range the last unit is issued again (never consumed)
            if (iu + 1 < ub) {
                ++iu;
                if (++ik == nSB) {
                    ik = 0;
                    ++im;
                    ie = tile_e[im];
                    ir0 = tile_r0[im];
                    inr = tile_n[im];
                }
            }
        };

        const I2F4Consts k4;
        const f16x2 one2 = {(f16)1.0f, (f16)1.0f};
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        int cu = ua, cm = ua / nSB, ck = ua % nSB;      // consume cursor
        auto flush = [&](uint32_t sbits) {
            f32x4 v = acc;
            if constexpr (CHANNEL) {
                const float s = f16_bits_to_f32((uint16_t)sbits);
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] *= s;
            }
            const int r0 = tile_r0[cm], nr = tile_n[cm];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * (lane >> 4) + i;
                if (r < nr) {
                    const int t = tok_of[r0 + r];
                    if (t >= 0) my_sum[t * 16 + (lane & 15)] += gate_of[r0 + r] * v[i];
                }
            }
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
        };
        auto consume_unit = [&](int slot) {
            if constexpr (GROUPED) {
                // two interleaved chains (even / odd K-steps): a dependent MFMA chain stalls
                f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < KSTEPS; ++j) {
                    if (j & 1) t1 = mfma16x16x32(araw[slot][j], weight_frag<WT, false>(braw[slot], j, one2, k4), t1);
                    else t0 = mfma16x16x32(araw[slot][j], weight_frag<WT, false>(braw[slot], j, one2, k4), t0);
                }
                const f32x4 t = t0 + t1;
                const float s = f16_bits_to_f32((uint16_t)sraw[slot]);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(t[i], s, acc[i]);
            } else {
#pragma unroll
                for (int j = 0; j < KSTEPS; ++j)
                    acc = mfma16x16x32(araw[slot][j], weight_frag<WT, false>(braw[slot], j, one2, k4), acc);
            }
            if (ck == nSB - 1 || cu == ub - 1) flush(sraw[slot]);
            ++cu;
            if (++ck == nSB) {
                ck = 0;
                ++cm;
            }
        };

#pragma unroll
        for (int u = 0; u < PF; ++u) issue(u);
        int kc = ua;
        for (; kc + PF <= ub; kc += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                consume_unit(u);
                issue(u);
            }
        }
#pragma unroll
        for (int u = 0; u < PF; ++u)
            if (kc + u < ub) consume_unit(u);
        // every ring slot holds a load (a repeat of the last unit where the range ran out)
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            consume(braw[u]);
            consume(sraw[u]);
#pragma unroll
            for (int j = 0; j < KSTEPS; ++j) consume(araw[u][j]);
        }
    }
    __syncthreads();

    // the S waves' token sums, added in wave order, then the addend
    const int c0 = cb * 16;
    for (int i = threadIdx.x; i < T * 16; i += blockDim.x) {
        const int t = i >> 4, c = i & 15;
        float v = 0.0f;
        for (int s = 0; s < S; ++s) v += tok_sum[(s * T + t) * 16 + c];
        if (p.addend) v += f16_bits_to_f32(p.addend[(size_t)t * N + c0 + c]);
        p.out[(size_t)t * N + c0 + c] = f32_to_f16_bits(v);
    }
}

// ------------------------------------------------------------------------------------
// Host side.
// ------------------------------------------------------------------------------------
constexpr int kCombineWaves = 8;

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t decode_workspace_layout(int T, int k, int E, int d, int inter, int wtype, DecodeWs* ws,
                               char* base) {
    (void)d;
    (void)wtype;
    const size_t R = (size_t)T * k;
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
    char* h = take(R * (size_t)inter * 2);
    if (ws) {
        ws->perm = (int32_t*)perm;
        ws->inv_perm = (int32_t*)inv;
        ws->offsets = (int32_t*)offs;
        ws->w_perm = (float*)wperm;
        ws->h = (uint16_t*)h;
    }
    return off;
}

template <int WT, bool GROUPED>
static hipError_t combine_launch(const CombineParams& p, hipStream_t stream) {
    const unsigned grid = (unsigned)(p.N / 16);
    const size_t lds = (size_t)kCombineWaves * p.T * 16 * sizeof(float);
    gemm_combine_kernel<WT, GROUPED, 8><<<grid, kCombineWaves * kWave, lds, stream>>>(p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    DecodeWs ws;
    decode_workspace_layout(a.T, a.k, a.E, a.d, a.inter, a.wtype, &ws, (char*)a.ws);
    const int R = a.T * a.k;

    if (a.E <= 64)
        decode_route_sort_kernel<1><<<1, kSortWaves * kWave, 0, stream>>>(
            a.logits, a.active, a.T, a.E, a.k, a.gate_all, a.ids, a.wts, ws);
    else if (a.E <= 128)
        decode_route_sort_kernel<2><<<1, kSortWaves * kWave, 0, stream>>>(
            a.logits, a.active, a.T, a.E, a.k, a.gate_all, a.ids, a.wts, ws);
    else
        decode_route_sort_kernel<4><<<1, kSortWaves * kWave, 0, stream>>>(
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
    err = launch_gemm_stream(g, stream);
    if (err != hipSuccess) return err;

    CombineParams c;
    c.h = ws.h;
    c.offsets = ws.offsets;
    c.perm = ws.perm;
    c.w_perm = ws.w_perm;
    c.w = a.w2;
    c.scales = a.s2;
    c.addend = a.addend;
    c.out = a.out;
    c.R = R;
    c.E = a.E;
    c.K = a.inter;
    c.N = a.d;
    c.T = a.T;
    c.k = a.k;
    // the addend (e.g. shared experts computed on another stream) is first read here
    if (a.addend_ready) {
        err = hipStreamWaitEvent(stream, (hipEvent_t)a.addend_ready, 0);
        if (err != hipSuccess) return err;
    }
    const bool grouped = a.group != 0;
    switch (a.wtype * 2 + (grouped ? 1 : 0)) {
        case MOE_W_INT4 * 2 + 0: return combine_launch<MOE_W_INT4, false>(c, stream);
        case MOE_W_INT4 * 2 + 1: return combine_launch<MOE_W_INT4, true>(c, stream);
        case MOE_W_INT8 * 2 + 0: return combine_launch<MOE_W_INT8, false>(c, stream);
        case MOE_W_INT8 * 2 + 1: return combine_launch<MOE_W_INT8, true>(c, stream);
        case MOE_W_FP16 * 2 + 0: return combine_launch<MOE_W_FP16, false>(c, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
