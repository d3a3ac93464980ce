// Internal launchers (one per kernel family).  Arguments are validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// MOE_OK when the current device is a usable gfx950, else MOE_ERR_NO_DEVICE (cached per device).
int32_t device_status();

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int gate_all,
                             int32_t* ids, float* wts, hipStream_t stream);

hipError_t launch_sort(const int32_t* ids, const float* wts, int R, int E,
                       int32_t* perm, int32_t* inv_perm, int32_t* offsets, float* w_perm,
                       hipStream_t stream);

hipError_t launch_gather(const uint16_t* x, const int32_t* perm, int R, int k, int d,
                         uint16_t* x_perm, hipStream_t stream);

hipError_t launch_combine(const uint16_t* y, const int32_t* inv_perm, const float* w,
                          const uint16_t* addend, int T, int k, int d, uint16_t* out,
                          hipStream_t stream);

hipError_t launch_dequant(const void* w, const uint16_t* scales, int wtype, int group,
                          int E, int K, int N, uint16_t* out, hipStream_t stream);

struct GemmParams {
    const uint16_t* a;
    const int32_t* a_rows;   // NULL: GEMM row p reads a[p]; else a[a_rows[p] / a_div]
    int a_div, a_nrows;      // divisor of a_rows, rows of a (source rows are clamped into it)
    const int32_t* out_rows; // NULL: GEMM row p writes out[p]; else out[out_rows[p]]
    int out_nrows;           // rows of out (other destinations are not written)
    const int32_t* offsets;
    const void* w;
    const uint16_t* scales;
    const float* row_scale;
    uint16_t* out;
    int R, E, K, N;
    int wtype, group, act;
    int split;           // stream path: waves per block splitting K (1..MOE_MAX_SPLIT_K)
    int tile;            // enum moe_tile (0 = automatic)
};

// Path/split decisions (host-only, deterministic in the arguments).
int gemm_choose_path(int R, int E, int K, int N, int wtype, int act, int forced);
int gemm_choose_split(int R, int E, int K, int N, int wtype, int act, int forced);
int gemm_choose_tile(int R, int E, int N, int act, int forced);

hipError_t launch_gemm_stream(const GemmParams& p, hipStream_t stream);
hipError_t launch_gemm_tile(const GemmParams& p, hipStream_t stream);

}  // namespace moe
