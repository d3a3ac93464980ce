// BF16 recovery from bit fields ("ZipMoE" note, key design: BF16 bit-field lossless
// compression).  Expert tensors are stored as one exponent byte per value (the 8 exponent
// bits; the stream that gets compressed) and one sign-mantissa byte per value (sign in bit 7,
// the 7 mantissa bits below).  Once the exponents are decompressed, this kernel merges the two
// byte streams back into the original BF16 bits:
//     bf16 = (sm & 0x80) << 8 | e << 7 | (sm & 0x7F)
// Each thread handles 16 values: one 16-byte load of each stream, two 16-byte stores.  The
// work is a pure stream (2 bytes read, 2 written per value), bound by HBM.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// two values from byte pairs: e and sm hold [b0, 0, b1, 0] (one byte per 16-bit half)
__device__ __forceinline__ uint32_t merge2(uint32_t e, uint32_t sm) {
    return ((sm & 0x00800080u) << 8) | (e << 7) | (sm & 0x007F007Fu);
}

__global__ __launch_bounds__(256) void bf16_recombine_kernel(const u32x4* __restrict__ e16,
                                                             const u32x4* __restrict__ sm16,
                                                             size_t nchunk,
                                                             const uint8_t* __restrict__ e,
                                                             const uint8_t* __restrict__ sm,
                                                             size_t n,
                                                             u32x4* __restrict__ out) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nchunk; i += stride) {
        const u32x4 ev = __builtin_nontemporal_load(e16 + i);
        const u32x4 sv = __builtin_nontemporal_load(sm16 + i);
        u32x4 o0, o1;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // v_perm: selector bytes 0..3 pick bytes of the second operand, 4 a zero byte
            const uint32_t elo = __builtin_amdgcn_perm(0u, ev[w], 0x04010400u);
            const uint32_t ehi = __builtin_amdgcn_perm(0u, ev[w], 0x04030402u);
            const uint32_t slo = __builtin_amdgcn_perm(0u, sv[w], 0x04010400u);
            const uint32_t shi = __builtin_amdgcn_perm(0u, sv[w], 0x04030402u);
            const uint32_t a = merge2(elo, slo), b = merge2(ehi, shi);
            if (w < 2) { o0[2 * w] = a; o0[2 * w + 1] = b; }
            else { o1[2 * (w - 2)] = a; o1[2 * (w - 2) + 1] = b; }
        }
        out[2 * i] = o0;
        out[2 * i + 1] = o1;
    }
    // the last n % 16 values, one per thread of the first block
    const size_t tail0 = nchunk * 16;
    if (blockIdx.x == 0) {
        uint16_t* o16 = (uint16_t*)out;
        for (size_t k = tail0 + threadIdx.x; k < n; k += blockDim.x)
            o16[k] = (uint16_t)(((sm[k] & 0x80u) << 8) | ((uint32_t)e[k] << 7) | (sm[k] & 0x7Fu));
    }
}

hipError_t launch_bf16_recombine(const uint8_t* e, const uint8_t* sm, size_t n, uint16_t* out,
                                 hipStream_t stream) {
    const size_t nchunk = n / 16;
    const size_t want = (nchunk + 255) / 256;
    const unsigned grid = (unsigned)(want < 1 ? 1 : (want < 16384 ? want : 16384));
    bf16_recombine_kernel<<<grid, 256, 0, stream>>>((const u32x4*)e, (const u32x4*)sm, nchunk, e,
                                                    sm, n, (u32x4*)out);
    return hipGetLastError();
}

}  // namespace moe
