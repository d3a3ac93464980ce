// Attainable-peak probes: a plain HBM read stream and a plain MFMA loop on gfx950, timed by the
// caller next to the layer's kernels so that each kernel's fraction of the published peak can
// be read against what simple code reaches on the same device.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// Grid-stride read of n16 16-byte words with 4 independent loads in flight per thread; each
// block writes the XOR of everything it read (so the loads cannot be dropped).
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src,
                                                         size_t n16, uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
    uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v ^= __shfl_xor(v, s, kWave);
    __shared__ uint32_t part[4];
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = v;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Each wave runs 16 independent chains of v_mfma_f32_16x16x32_f16 on all-ones operands (with 8
// the compiler moves every accumulator through other registers each iteration, and the loop
// reaches about 60% of this one), so every MFMA adds exactly 32 to each accumulator element;
// out[thread] = sum over the chains of element 0 = 16 * 32 * iters (exact in fp32 for
// iters < 2^15).
constexpr int kProbeChains = 16;
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* __restrict__ out) {
    f16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) { a[i] = (f16)1.0f; b[i] = (f16)1.0f; }
    f32x4 acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c) acc[c] = mfma16x16x32(a, b, acc[c]);
    }
    float v = 0.f;
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) v += acc[c][0];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = v;
}

}  // namespace moe

extern "C" {

int32_t moe_probe_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                       void* stream) {
    if (blocks < 1 || bytes % 16 != 0) return MOE_ERR_INVALID;
    if (bytes == 0) return MOE_OK;
    if (!src || !sink || ((uintptr_t)src & 15u) != 0 || ((uintptr_t)sink & 3u) != 0)
        return MOE_ERR_INVALID;
    if (int32_t st = moe::device_status()) return st;
    moe::probe_read_kernel<<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>(
        (const moe::u32x4*)src, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int32_t moe_probe_mfma(int32_t iters, float* out, int32_t blocks, void* stream) {
    if (blocks < 1 || iters < 0 || iters >= (1 << 15)) return MOE_ERR_INVALID;
    if (!out || ((uintptr_t)out & 3u) != 0) return MOE_ERR_INVALID;
    if (int32_t st = moe::device_status()) return st;
    moe::probe_mfma_kernel<<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>(iters, out);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
