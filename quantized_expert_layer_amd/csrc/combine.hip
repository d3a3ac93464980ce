// Unpermute + expert_scale ("Who Says Elephants Can't Run", section 3 workflow: rows go back
// to their original order and are scaled by the gate weight), summing the k rows of a token:
//   out[t] = fp16( sum_{j ascending} w[t,j] * y[inv_perm[t*k + j]]  + addend[t] )
// in fp32, one rounding at the end.  8 columns (16 bytes) per thread.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

__device__ __forceinline__ void add8(float acc[8], u32x4 v, float w) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const f16x2 p = as_f16x2(v[h]);
        acc[2 * h] += w * (float)p[0];
        acc[2 * h + 1] += w * (float)p[1];
    }
}

__global__ __launch_bounds__(256) void combine_kernel(const u32x4* __restrict__ y,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ w,
                                                      const u32x4* __restrict__ addend,
                                                      uint32_t total, int T, int k, uint32_t d16,
                                                      u32x4* __restrict__ out) {
    const uint32_t R = (uint32_t)T * (uint32_t)k;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += gridDim.x * blockDim.x) {
        const uint32_t t = i / d16;
        const uint32_t c = i - t * d16;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const int pos = inv_perm[t * k + j];
            if ((uint32_t)pos >= R) continue;          // dropped slot (or invalid index)
            const float wj = w ? w[t * k + j] : 1.0f;
            add8(acc, y[(size_t)pos * d16 + c], wj);
        }
        if (addend) add8(acc, addend[i], 1.0f);
        u32x4 r;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            f16x2 p;
            p[0] = (f16)acc[2 * h];
            p[1] = (f16)acc[2 * h + 1];
            r[h] = __builtin_bit_cast(uint32_t, p);
        }
        out[i] = r;
    }
}

hipError_t launch_combine(const uint16_t* y, const int32_t* inv_perm, const float* w,
                          const uint16_t* addend, int T, int k, int d, uint16_t* out,
                          hipStream_t stream) {
    const uint32_t d16 = (uint32_t)d / 8u;
    const uint32_t total = (uint32_t)T * d16;
    const uint32_t want = (total + 255u) / 256u;
    const int grid = (int)(want < 8192u ? want : 8192u);
    combine_kernel<<<grid, 256, 0, stream>>>((const u32x4*)y, inv_perm, w, (const u32x4*)addend,
                                             total, T, k, d16, (u32x4*)out);
    return hipGetLastError();
}

}  // namespace moe
