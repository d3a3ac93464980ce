// Internal launchers (one per kernel family).  Arguments are validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// MOE_OK when the current device is a usable gfx950, else MOE_ERR_NO_DEVICE (cached per device).
int32_t device_status();

hipError_t launch_route_topk(const float* logits, const uint8_t* active, int T, int E, int k,
                             int gate_all, int32_t* ids, float* wts, hipStream_t stream);

// ws: sort_workspace_bytes(R, E) bytes (none up to 1024 slots)
size_t sort_workspace_bytes(int R, int E);
hipError_t launch_sort(const int32_t* ids, const float* wts, int R, int E,
                       int32_t* perm, int32_t* inv_perm, int32_t* offsets, float* w_perm,
                       void* ws, hipStream_t stream);

hipError_t launch_gather(const uint16_t* x, const int32_t* perm, int R, int k, int d,
                         uint16_t* x_perm, hipStream_t stream);

hipError_t launch_combine(const uint16_t* y, const int32_t* inv_perm, const float* w,
                          const uint16_t* addend, int T, int k, int d, uint16_t* out,
                          hipStream_t stream);

hipError_t launch_elb_accumulate(const int32_t* ids, int L, int n, int E, int32_t* counts,
                                 hipStream_t stream);
hipError_t launch_elb_top_m(const int32_t* counts, int L, int E, int M, int32_t* experts,
                            int32_t* top_counts, hipStream_t stream);

hipError_t launch_bf16_recombine(const uint8_t* e, const uint8_t* sm, size_t n, uint16_t* out,
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
    int i2f;             // enum moe_i2f
    const int32_t* tiles16;  // stream path: NULL, or the decode tile table (16-row m-tiles)
};

// Path/split decisions (host-only, deterministic in the arguments).
int gemm_choose_path(int R, int E, int K, int N, int wtype, int act, int forced);
int gemm_choose_split(int R, int E, int K, int N, int wtype, int act, int forced);
int gemm_choose_tile(int R, int E, int N, int act, int wtype, bool grouped, int forced);
// Whether the native int-to-float conversion is built for this call (tile path).
bool gemm_native_supported(int wtype, int act, int group, int tile);

hipError_t launch_gemm_stream(const GemmParams& p, hipStream_t stream);
// The stream launch of a decode step's first GEMM (integer codes, at most 128 rows) with a
// dense fp16 SwiGLU GEMM over all rows of `side` in the same launch (offsets, row maps and tile
// table NULL; side.split is not read: its K is split over the launch's waves per workgroup,
// p.split, or 4 when p is unsplit).
hipError_t launch_gemm_stream_side(const GemmParams& p, const GemmParams& side,
                                   hipStream_t stream);
hipError_t launch_gemm_tile(const GemmParams& p, hipStream_t stream);

// ---- decode step (few tokens): gating + sort, GEMM 1, GEMM 2 with the combine ----
// Workspace of one decode call, carved from the caller's buffer (256-byte aligned parts).
struct DecodeWs {
    int32_t* perm;           // [R]
    int32_t* inv_perm;       // [R]
    int32_t* offsets;        // [E + 1]
    float* w_perm;           // [R]
    int32_t* tiles;          // [1 + kDecodeMaxTiles] tile table (count, then packed tiles)
    uint16_t* h;             // fp16 [R, inter] GEMM 1 output, sorted rows
    float* part;             // fp32 [nsplit, T, d] partial token sums of GEMM 2 (nsplit > 1)
    uint16_t* sh_h;          // fp16 [T, shared_inter] shared experts' hidden rows (or NULL)
    uint16_t* sh_y;          // fp16 [T, d] shared experts' output (or NULL)
};

struct CombineParams {
    const uint16_t* h;       // fp16 [R, K] rows sorted by expert
    const int32_t* tiles;    // tile table of the sorted rows
    const int32_t* perm;     // [R] flat slot t*k + j of sorted row p
    const float* w_perm;     // [R] gate weight of sorted row p
    const void* w;           // packed weights [E, K, N]
    const uint16_t* scales;  // [E, G, N], NULL for fp16 weights
    const uint16_t* addend;  // fp16 [T, N] or NULL
    uint16_t* out;           // fp16 [T, N]
    float* part;             // fp32 [nsplit, T, N] when nsplit > 1
    int R, E, K, N, T, k;
    int nsplit;              // blocks sharing the units of one 16-column block
};

struct DecodeArgs {
    const float* logits;
    const uint8_t* active;   // [T] or NULL: tokens with 0 take no expert
    const uint16_t* x;
    int T, E, k, gate_all, d, inter, act;
    const void* w1;
    const uint16_t* s1;
    const void* w2;
    const uint16_t* s2;
    int wtype, group;
    const void* sw1;         // shared experts, fp16 packed [d, 2 shared_inter] (gate | up), or NULL
    const void* sw2;         //   and [shared_inter, d]; SwiGLU, weight 1, every token
    int shared_inter;
    const uint16_t* addend;
    void* addend_ready;      // hipEvent_t or NULL: waited for before the launch that adds addend
    int32_t* ids;
    float* wts;
    uint16_t* out;
    void* ws;
};

// Blocks sharing one column group of the decode step's second GEMM (a power of two; at least
// two with shared experts, whose output the reduction launch adds).
int decode_combine_split(int d, bool shared);
// Bytes of the decode workspace (shared_inter 0: no shared experts); with ws and base given,
// also the part addresses.
size_t decode_workspace_layout(int T, int k, int E, int d, int inter, int wtype, int shared_inter,
                               DecodeWs* ws, char* base);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace moe
