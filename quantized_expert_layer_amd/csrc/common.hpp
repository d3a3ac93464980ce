// Shared device/host definitions of the MoE expert-layer kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_wq.h"

namespace moe {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ------------------------------------------------------------------------------------
// Packed weight layout (shared by every kernel that reads weights).
//
// A weight matrix of expert e is K x N (K = reduction).  It is cut into 16-column blocks
// (cb = n / 16).  Each column block is stored contiguously along K as a run of 1 KiB
// "super-blocks"; a super-block holds the operand of one MFMA 16x16x32 B fragment per
// 32-row K-step for all 64 lanes:  lane l owns column cb*16 + (l & 15) and, within each
// K-step, rows 8*(l >> 4) .. 8*(l >> 4) + 7.  Lane l's 16 bytes of a super-block are at
// byte offset 16*l, so one 16-byte load per lane fetches a whole super-block.
//   INT4: 4 K-steps (128 rows) per super-block; word j of lane l = K-step j; the 8 codes
//         (offset +8) sit in nibble order [e0,e2,e4,e6,e1,e3,e5,e7].
//   INT8: 2 K-steps (64 rows); words 2j, 2j+1 = K-step j, rows 0..3 and 4..7; bytes in
//         natural order, offset +128 (offset-binary).
//   FP16: 1 K-step (32 rows); the 8 halves of the lane in row order.
// Address of super-block (e, cb, kb): ((e * (N/16) + cb) * (K / KSB) + kb) * 1024 bytes.
// ------------------------------------------------------------------------------------
template <int WT> struct WTraits;
template <> struct WTraits<MOE_W_INT4> { static constexpr int KSB = 128; };
template <> struct WTraits<MOE_W_INT8> { static constexpr int KSB = 64; };
template <> struct WTraits<MOE_W_FP16> { static constexpr int KSB = 32; };

__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

// Exponent-of-1024 int-to-float construction ("Who Says Elephants Can't Run", section 3,
// optimized I2F).  0x6400 is fp16 1024 with an all-zero mantissa; OR-ing an integer Y < 1024
// into the mantissa gives the fp16 value 1024 + Y, and one packed fp16 subtraction removes
// the offset.  INT4 nibbles four bits up the half-word land as 16*u: (1024 + 16u)/16 - 72 =
// u - 8 with a single packed fma, exact in fp16.
// (w & mask) | magic in one v_and_or_b32.  Written out because the compiler otherwise splits
// it into v_and + v_or (both constants would need the single scalar operand slot of VOP3).
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "v"(mask), "s"(magic));
    return r;
}

struct I2F4Consts {
    uint32_t lo, hi;                 // nibble masks, kept in VGPRs
    __device__ __forceinline__ I2F4Consts() {
        asm("v_mov_b32 %0, 0x000F000F" : "=v"(lo));
        asm("v_mov_b32 %0, 0x00F000F0" : "=v"(hi));
    }
};

__device__ __forceinline__ void i2f_int4(uint32_t w, f16x2 out[4], const I2F4Consts& k) {
    const uint32_t magic = 0x64006400u;
    const uint32_t w8 = w >> 8;
    const f16x2 sub_lo = {(f16)1032.0f, (f16)1032.0f};
    const f16x2 mul_hi = {(f16)0.0625f, (f16)0.0625f};
    const f16x2 sub_hi = {(f16)-72.0f, (f16)-72.0f};
    out[0] = as_f16x2(and_or(w, k.lo, magic)) - sub_lo;             // [e0, e1]
    out[1] = as_f16x2(and_or(w, k.hi, magic)) * mul_hi + sub_hi;    // [e2, e3]
    out[2] = as_f16x2(and_or(w8, k.lo, magic)) - sub_lo;            // [e4, e5]
    out[3] = as_f16x2(and_or(w8, k.hi, magic)) * mul_hi + sub_hi;   // [e6, e7]
}

__device__ __forceinline__ void i2f_int4(uint32_t w, f16x2 out[4]) {
    const I2F4Consts k;
    i2f_int4(w, out, k);
}

// 8-bit variant: byte u = q + 128 goes into the mantissa of 1024, then 1152 = 1024 + 128
// is subtracted.  v_perm_b32 builds [0x64|b0, 0x64|b1] in one instruction.
__device__ __forceinline__ void i2f_int8(uint32_t w, f16x2 out[2]) {
    const f16x2 sub = {(f16)1152.0f, (f16)1152.0f};
    out[0] = as_f16x2(__builtin_amdgcn_perm(0x64646464u, w, 0x05010400u)) - sub;  // [e0,e1]
    out[1] = as_f16x2(__builtin_amdgcn_perm(0x64646464u, w, 0x05030402u)) - sub;  // [e2,e3]
}

// The same codes through the conversion instructions instead (the baseline of the construction
// above): each byte of a word becomes fp32 with v_cvt_f32_ubyte0..3, two values are packed to
// fp16 (the integers below 256 are exact, so the rounding mode does not matter), and the
// storage offset is subtracted.  4-bit codes first split the word into its low and high
// nibbles (w & 0x0F0F0F0F, (w >> 4) & 0x0F0F0F0F): byte b of the low part is nibble 2b, of the
// high part nibble 2b + 1, which by the nibble order [e0,e2,e4,e6,e1,e3,e5,e7] hold
// e0 e4 e1 e5 and e2 e6 e3 e7.
__device__ __forceinline__ f16x2 cvt_pair(float a, float b) {
    return __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(a, b));
}
// byte b of w as fp32 (the backend selects v_cvt_f32_ubyte<b> for this pattern)
template <int B>
__device__ __forceinline__ float ubyte_f32(uint32_t w) {
    return (float)((w >> (8 * B)) & 0xFFu);
}
__device__ __forceinline__ void i2f_int4_native(uint32_t w, f16x2 out[4]) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const f16x2 off = {(f16)8.0f, (f16)8.0f};
    out[0] = cvt_pair(ubyte_f32<0>(lo), ubyte_f32<2>(lo)) - off;    // [e0, e1]
    out[1] = cvt_pair(ubyte_f32<0>(hi), ubyte_f32<2>(hi)) - off;    // [e2, e3]
    out[2] = cvt_pair(ubyte_f32<1>(lo), ubyte_f32<3>(lo)) - off;    // [e4, e5]
    out[3] = cvt_pair(ubyte_f32<1>(hi), ubyte_f32<3>(hi)) - off;    // [e6, e7]
}
__device__ __forceinline__ void i2f_int8_native(uint32_t w, f16x2 out[2]) {
    const f16x2 off = {(f16)128.0f, (f16)128.0f};
    out[0] = cvt_pair(ubyte_f32<0>(w), ubyte_f32<1>(w)) - off;      // [e0, e1]
    out[1] = cvt_pair(ubyte_f32<2>(w), ubyte_f32<3>(w)) - off;      // [e2, e3]
}

__device__ __forceinline__ f16x8 pack8(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
    f16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// ------------------------------------------------------------------------------------
// Weight fragment expansion: K-step j of a lane's 16-byte super-block slice -> B operand.
// Group scales (group 128) are folded in by one fp16 multiply, giving exactly Algorithm 1's
// fp16 weight; per-channel scales are applied to the fp32 result instead.
// ------------------------------------------------------------------------------------
template <int WT, bool SCALE, bool NATIVE = false>
__device__ __forceinline__ f16x8 weight_frag(const u32x4& raw, int j, f16x2 s2,
                                             const I2F4Consts& k4) {
    f16x2 q[4];
    if constexpr (WT == MOE_W_INT4) {
        if constexpr (NATIVE) i2f_int4_native(raw[j], q);
        else i2f_int4(raw[j], q, k4);
    } else if constexpr (WT == MOE_W_INT8) {
        if constexpr (NATIVE) {
            i2f_int8_native(raw[2 * j], q);
            i2f_int8_native(raw[2 * j + 1], q + 2);
        } else {
            i2f_int8(raw[2 * j], q);
            i2f_int8(raw[2 * j + 1], q + 2);
        }
    } else {
        return __builtin_bit_cast(f16x8, raw);
    }
    if constexpr (SCALE) {
#pragma unroll
        for (int h = 0; h < 4; ++h) q[h] = q[h] * s2;
    }
    return pack8(q[0], q[1], q[2], q[3]);
}

__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (f16)v);   // round to nearest even
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(f16, b);
}

// Four fp16 values (8-byte aligned) to fp32, and four fp32 values to fp16 (round to nearest
// even) in one 8-byte store.
__device__ __forceinline__ f32x4 load4_f16(const uint16_t* src) {
    const uint2 v = *(const uint2*)src;
    const f16x2 lo = __builtin_bit_cast(f16x2, v.x), hi = __builtin_bit_cast(f16x2, v.y);
    return f32x4{(float)lo[0], (float)lo[1], (float)hi[0], (float)hi[1]};
}
__device__ __forceinline__ void store4_f16_bits(uint16_t* dst, f32x4 v) {
    const f16x2 lo = {(f16)v[0], (f16)v[1]}, hi = {(f16)v[2], (f16)v[3]};
    uint2 o;
    o.x = __builtin_bit_cast(uint32_t, lo);
    o.y = __builtin_bit_cast(uint32_t, hi);
    *(uint2*)dst = o;
}

// Block barrier that orders LDS accesses only.  __syncthreads() also waits for every global
// store the wave has in flight (vmcnt 0), which costs a memory round trip where the other waves
// only need LDS data.  Callers use it where no wave reads global memory written by another
// wave of the block before the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// The same ordering for the LDS accesses of one wave (no barrier: a wave's LDS accesses take
// effect in program order; this keeps the compiler from moving them across the point).
__device__ __forceinline__ void lds_wave_fence() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
}

// Marks a register value as read here, so its load has completed and its registers are not
// handed to other values before this point.  Used where a prefetch ring ends: the ring's last
// (repeated) loads are never consumed otherwise, and a register that still awaits one must not
// be reused by the epilogue.
template <typename T>
__device__ __forceinline__ void consume(const T& v) {
    asm volatile("; consume %0" : : "v"(v));
}

// Non-temporal 16-byte load of packed weights (streamed once; keep caches for activations).
__device__ __forceinline__ u32x4 load_weights16(const u32x4* p) {
    return __builtin_nontemporal_load(p);
}

// Inclusive prefix sum over the 64 lanes of a wave.  Row shifts by 1, 2, 4 and 8 lanes give the
// sums within each row of 16 lanes; broadcasting lane 15 into rows 1 and 3, then lane 31 into rows
// 2 and 3, adds the totals of the rows before.  A lane that a shift or broadcast does not reach
// adds 0 (the `old` operand).  Six DPP additions instead of a chain of cross-lane permutes.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return v;
}

// ------------------------------------------------------------------------------------
// Tile lookup in one pass over the offsets: the total number of m-tiles (sum over experts of
// ceil(c_e / BM)) and, for logical tile index `want` (a function of that total), the expert,
// first row and row count.  Experts are visited in order, 64 per lane chunk; only the chunks
// that hold experts are scanned.  Row counts come from the offsets clamped into [0, R], so any
// offsets array yields in-bounds rows.  Executed by a whole wave; results are wave-uniform.
// Returns false when `want` maps past the last tile.
// ------------------------------------------------------------------------------------
template <int BM, typename F>
__device__ __forceinline__ bool lookup_m_tile(const int32_t* __restrict__ offsets, int E, int R,
                                              F want_of_total, int& mt_out, int& e_out,
                                              int& row0, int& rows) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int MAXC = (MOE_MAX_EXPERTS + kWave - 1) / kWave;
    const int nc = (E + kWave - 1) / kWave;          // chunks holding experts (wave-uniform)
    int lo[MAXC], hi[MAXC], tl[MAXC], incl[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int e = c * kWave + lane;
        lo[c] = hi[c] = 0;
        if (c < nc && e < E) {
            lo[c] = min(max(offsets[e], 0), R);
            hi[c] = min(max(offsets[e + 1], 0), R);
        }
    }
    int total = 0;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        tl[c] = (max(hi[c] - lo[c], 0) + BM - 1) / BM;
        incl[c] = total;
        if (c < nc) {
            const int v = wave_incl_scan(tl[c]);
            incl[c] = total + v;
            total += __builtin_amdgcn_readlane(v, kWave - 1);
        }
    }
    total = __builtin_amdgcn_readfirstlane(total);
    const int mt = want_of_total(total);
    if (mt < 0 || mt >= total) return false;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        if (c >= nc) break;
        const int excl = incl[c] - tl[c];
        const unsigned long long hit = __ballot(tl[c] > 0 && mt >= excl && mt < incl[c]);
        if (hit) {
            const int src = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
            const int my_row0 = lo[c] + (mt - excl) * BM;
            const int my_rows = min(BM, hi[c] - my_row0);
            mt_out = mt;
            e_out = c * kWave + src;
            row0 = __builtin_amdgcn_readlane(my_row0, src);
            rows = __builtin_amdgcn_readlane(my_rows, src);
            return rows > 0 && row0 >= 0 && row0 + rows <= R;
        }
    }
    return false;
}

// ------------------------------------------------------------------------------------
// Tile table of a decode step: the gating + sort launch lists every 16-row m-tile of the
// sorted rows (expert e, first row r0, rows n in 1..16), so a later launch finds its tile with
// one load instead of a scan over the offsets.  Entry 0 holds the number of tiles; tile i is
// entry 1 + i, packed as e | r0 << 9 | (n - 1) << 19 (e < 512, r0 < 1024).
// ------------------------------------------------------------------------------------
constexpr int kDecodeMaxTiles = MOE_DECODE_MAX_ROWS / 16 + MOE_MAX_EXPERTS;
static_assert(MOE_MAX_EXPERTS <= 512 && MOE_DECODE_MAX_ROWS <= 1024, "tile packing");

__device__ __forceinline__ int tile16_pack(int e, int r0, int n) {
    return e | (r0 << 9) | ((n - 1) << 19);
}
__device__ __forceinline__ void tile16_unpack(int v, int& e, int& r0, int& n) {
    e = v & 511;
    r0 = (v >> 9) & 1023;
    n = ((v >> 19) & 15) + 1;
}

template <int BM>
__device__ __forceinline__ bool find_m_tile(const int32_t* __restrict__ offsets, int E, int R,
                                            int mt, int& e_out, int& row0, int& rows) {
    int m;
    return lookup_m_tile<BM>(offsets, E, R, [mt](int) { return mt; }, m, e_out, row0, rows);
}

}  // namespace moe
