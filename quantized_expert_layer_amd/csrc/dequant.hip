// Standalone dequantization, Algorithm 1 of "Who Says Elephants Can't Run" (section 3):
//   for e, m, n:  W_dq[e, m, n] = IntToFloat(W[e, m, n]) * S[e, g(m), n]
// IntToFloat is the exponent-of-1024 construction (exact), the product is one fp16 multiply
// (round to nearest even), so each output is the correctly rounded fp16 product.
// One thread per (super-block, lane): it expands that lane's 16 bytes into the logical
// [E, K, N] layout.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

template <int WT>
__global__ __launch_bounds__(256) void dequant_kernel(const u32x4* __restrict__ w,
                                                      const uint16_t* __restrict__ scales,
                                                      int group, int E, int K, int N,
                                                      uint16_t* __restrict__ out) {
    constexpr int KSB = WTraits<WT>::KSB;
    const int nSB = K / KSB, ncb = N / 16;
    const int G = group ? K / group : 1;
    const size_t n_units = (size_t)E * ncb * nSB;          // super-blocks
    const size_t unit = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    if (unit >= n_units) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int kb = (int)(unit % nSB);
    const int cb = (int)((unit / nSB) % ncb);
    const int e = (int)(unit / ((size_t)nSB * ncb));
    const int n = cb * 16 + (lane & 15);
    const u32x4 raw = w[unit * kWave + lane];
    uint16_t* o = out + (size_t)e * K * N + n;

#pragma unroll
    for (int j = 0; j < KSB / 32; ++j) {                 // K-steps in the super-block
        const int k0 = kb * KSB + j * 32 + 8 * (lane >> 4);
        const int g = group ? k0 / group : 0;
        const f16 s = __builtin_bit_cast(f16, scales[((size_t)e * G + g) * N + n]);
        const f16x2 s2 = {s, s};
        f16x2 q[4];
        if constexpr (WT == MOE_W_INT4) {
            i2f_int4(raw[j], q);
        } else {
            i2f_int8(raw[2 * j], q);
            i2f_int8(raw[2 * j + 1], q + 2);
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            // bit-cast the whole pair: a bit-cast of a single vector element is not used
            // because hipcc mistranslates it (the high element reads as the low one)
            const uint32_t v = __builtin_bit_cast(uint32_t, q[h] * s2);
            o[(size_t)(k0 + 2 * h) * N] = (uint16_t)(v & 0xFFFFu);
            o[(size_t)(k0 + 2 * h + 1) * N] = (uint16_t)(v >> 16);
        }
    }
}

hipError_t launch_dequant(const void* w, const uint16_t* scales, int wtype, int group, int E,
                          int K, int N, uint16_t* out, hipStream_t stream) {
    const int KSB = (wtype == MOE_W_INT4) ? 128 : 64;
    const size_t units = (size_t)E * (N / 16) * (K / KSB);
    const size_t blocks = (units * kWave + 255) / 256;
    if (wtype == MOE_W_INT4)
        dequant_kernel<MOE_W_INT4><<<blocks, 256, 0, stream>>>((const u32x4*)w, scales, group, E,
                                                               K, N, out);
    else
        dequant_kernel<MOE_W_INT8><<<blocks, 256, 0, stream>>>((const u32x4*)w, scales, group, E,
                                                               K, N, out);
    return hipGetLastError();
}

}  // namespace moe
