// C ABI of the MoE expert layer: argument validation, device check, dispatch.
// Validation runs before any HIP call, so argument errors are reported (and nothing is
// enqueued) even on a machine without a GPU.
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace {

constexpr int32_t kVersion = 100;

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// gfx950 check, cached per device id (immutable once written).
std::atomic<int> g_dev_state[64];   // 0 unknown, 1 usable, 2 unusable

int32_t check_device() {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return MOE_ERR_NO_DEVICE;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_NO_DEVICE;
    if (dev < 0 || dev >= 64) return MOE_ERR_NO_DEVICE;
    int st = g_dev_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_NO_DEVICE;
        const char* a = prop.gcnArchName;
        st = (a[0] == 'g' && a[1] == 'f' && a[2] == 'x' && a[3] == '9' && a[4] == '5' &&
              a[5] == '0') ? 1 : 2;
        g_dev_state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? MOE_OK : MOE_ERR_NO_DEVICE;
}

inline int32_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

struct GemmPlan {
    int path;
    int split;
    size_t ws;
};

GemmPlan plan_gemm(int32_t R, int32_t E, int32_t K, int32_t N, int32_t wtype, int32_t act,
                   const moe_gemm_opts* opts) {
    GemmPlan pl;
    const int forced_path = opts ? opts->path : MOE_PATH_AUTO;
    const int forced_split = opts ? opts->split_k : 0;
    pl.path = moe::gemm_choose_path(R, E, K, N, wtype, act, forced_path);
    pl.split = 1;
    if (pl.path == MOE_PATH_STREAM) pl.split = moe::gemm_choose_split(R, E, K, N, wtype, act, forced_split);
    pl.ws = 0;                                   // no kernel of either path needs one
    return pl;
}

int32_t validate_gemm(const uint16_t* a, const int32_t* offsets, int32_t R, int32_t E, int32_t K,
                      int32_t N, const void* w, const uint16_t* scales, int32_t wtype,
                      int32_t group, int32_t act, uint16_t* out, const moe_gemm_opts* opts) {
    if (R < 0 || E < 1 || E > MOE_MAX_EXPERTS || K <= 0 || N <= 0) return MOE_ERR_INVALID;
    if (wtype < MOE_W_INT4 || wtype > MOE_W_FP16) return MOE_ERR_INVALID;
    if (act < MOE_ACT_NONE || act > MOE_ACT_SWIGLU) return MOE_ERR_INVALID;
    if (group != 0 && group != 128) return MOE_ERR_UNSUPPORTED;
    if (wtype == MOE_W_FP16 && group != 0) return MOE_ERR_UNSUPPORTED;
    if (K % 128 != 0 || N % 16 != 0) return MOE_ERR_UNSUPPORTED;
    if (act == MOE_ACT_SWIGLU && N % 32 != 0) return MOE_ERR_UNSUPPORTED;
    if (opts) {
        if (opts->path < MOE_PATH_AUTO || opts->path > MOE_PATH_TILE) return MOE_ERR_INVALID;
        if (opts->split_k < 0 || opts->split_k > MOE_MAX_SPLIT_K) return MOE_ERR_INVALID;
        if (opts->tile < MOE_TILE_AUTO || opts->tile > MOE_TILE_48x128) return MOE_ERR_INVALID;
        if (opts->i2f != MOE_I2F_TRICK && opts->i2f != MOE_I2F_NATIVE) return MOE_ERR_INVALID;
        if (opts->i2f == MOE_I2F_NATIVE) {
            // built for the tile path of the MT encoder shapes only
            const int path = moe::gemm_choose_path(R, E, K, N, wtype, act, opts->path);
            const int tile = moe::gemm_choose_tile(R, E, N, act, wtype, group != 0, opts->tile);
            if (path != MOE_PATH_TILE || !moe::gemm_native_supported(wtype, act, group, tile))
                return MOE_ERR_UNSUPPORTED;
        }
    }
    if ((int64_t)R * K >= (int64_t)1 << 40) return MOE_ERR_UNSUPPORTED;
    if (R == 0) return MOE_OK;
    if (!a || !offsets || !w || !out) return MOE_ERR_INVALID;
    if (wtype != MOE_W_FP16 && !scales) return MOE_ERR_INVALID;
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(out, 16) || !aligned(offsets, 4))
        return MOE_ERR_INVALID;
    if (scales && !aligned(scales, 16)) return MOE_ERR_INVALID;
    return MOE_OK;
}

}  // namespace

// Scratch memory of moe_decode_layer_noalloc: a workspace that lives in the code object, so the
// call needs no allocation.  Each device that loads the library holds its own copy until the
// process ends; host code reaches it only through the address hipGetSymbolAddress returns for
// the current device (the array's name is a host-side stand-in, not a device address).
static __device__ __align__(256) uint8_t scratch[MOE_DECODE_SCRATCH_BYTES];

namespace {

std::atomic<void*> g_scratch_ptr[64];   // device address of `scratch`, per device id
std::mutex g_scratch_mu;

// Address of this device's `scratch`, looked up once per device (with that device current).
void* scratch_address(int dev) {
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!ptr) {
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

}  // namespace

namespace moe {
int32_t device_status() { return check_device(); }
}  // namespace moe

extern "C" {

int32_t moe_version(void) { return kVersion; }

const char* moe_status_str(int32_t s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID: return "MOE_ERR_INVALID: invalid argument";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or option not supported";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
        case MOE_ERR_NO_DEVICE: return "MOE_ERR_NO_DEVICE: no usable gfx950 device";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error";
        default: return "unknown status";
    }
}

int32_t moe_route_topk_active(const float* logits, const uint8_t* active, int32_t T, int32_t E,
                              int32_t k, int32_t gate_mode, int32_t* topk_ids, float* topk_w,
                              void* stream) {
    if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E)
        return MOE_ERR_INVALID;
    if (gate_mode != MOE_GATE_SOFTMAX_TOPK && gate_mode != MOE_GATE_SOFTMAX_ALL)
        return MOE_ERR_INVALID;
    if ((int64_t)T * E >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID;
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return MOE_ERR_INVALID;
    if (int32_t st = check_device()) return st;
    return hip_status(moe::launch_route_topk(logits, active, T, E, k,
                                             gate_mode == MOE_GATE_SOFTMAX_ALL, topk_ids, topk_w,
                                             (hipStream_t)stream));
}

int32_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t gate_mode,
                       int32_t* topk_ids, float* topk_w, void* stream) {
    return moe_route_topk_active(logits, nullptr, T, E, k, gate_mode, topk_ids, topk_w, stream);
}

size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E) {
    if (T <= 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS) return 0;
    if ((int64_t)T * k >= (int64_t)1 << 31) return 0;
    return moe::sort_workspace_bytes(T * k, E);
}

int32_t moe_permute(const int32_t* topk_ids, const float* topk_w, const uint16_t* x, int32_t T,
                    int32_t k, int32_t E, int32_t d, int32_t* perm, int32_t* inv_perm,
                    int32_t* expert_offsets, uint16_t* x_perm, float* w_perm, void* ws,
                    size_t ws_bytes, void* stream) {
    if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS || d <= 0)
        return MOE_ERR_INVALID;
    if (d % 8 != 0) return MOE_ERR_UNSUPPORTED;
    const int64_t R = (int64_t)T * k;
    if (R >= (int64_t)1 << 31 || R * (d / 8) >= (int64_t)1 << 32) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!topk_ids || !perm || !inv_perm || !expert_offsets) return MOE_ERR_INVALID;
    if (x_perm && !x) return MOE_ERR_INVALID;
    if (w_perm && !topk_w) return MOE_ERR_INVALID;
    if ((x_perm && (!aligned(x, 16) || !aligned(x_perm, 16))) || !aligned(topk_ids, 4) ||
        !aligned(perm, 4) || !aligned(inv_perm, 4) || !aligned(expert_offsets, 4))
        return MOE_ERR_INVALID;
    if ((topk_w && !aligned(topk_w, 4)) || (w_perm && !aligned(w_perm, 4))) return MOE_ERR_INVALID;
    const size_t need = moe::sort_workspace_bytes((int)R, E);
    if (need && (!ws || ws_bytes < need || !aligned(ws, 4))) return MOE_ERR_WORKSPACE;
    if (int32_t st = check_device()) return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = moe::launch_sort(topk_ids, topk_w, (int)R, E, perm, inv_perm, expert_offsets,
                                    w_perm, ws, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (!x_perm) return MOE_OK;               // the caller gathers inside the first GEMM
    return hip_status(moe::launch_gather(x, perm, (int)R, k, d, x_perm, s));
}

size_t moe_gemm_workspace_size(int32_t R, int32_t E, int32_t K, int32_t N, int32_t wtype,
                               int32_t act, const moe_gemm_opts* opts) {
    if (R <= 0 || E < 1 || K <= 0 || N <= 0) return 0;
    return plan_gemm(R, E, K, N, wtype, act, opts).ws;
}

static int32_t grouped_gemm(const uint16_t* a, int32_t a_nrows, const int32_t* a_rows,
                            int32_t a_div, const int32_t* expert_offsets, int32_t R, int32_t E,
                            int32_t K, int32_t N, const void* w_packed, const uint16_t* scales,
                            int32_t wtype, int32_t group_size, int32_t act,
                            const float* row_scale, uint16_t* out, int32_t out_nrows,
                            const int32_t* out_rows, const moe_gemm_opts* opts, void* ws,
                            size_t ws_bytes, void* stream) {
    if (int32_t st = validate_gemm(a, expert_offsets, R, E, K, N, w_packed, scales, wtype,
                                   group_size, act, out, opts))
        return st;
    if (a_rows && (a_div < 1 || a_nrows < 1)) return MOE_ERR_INVALID;
    if (out_rows && out_nrows < 0) return MOE_ERR_INVALID;
    if ((int64_t)a_nrows * K >= (int64_t)1 << 40) return MOE_ERR_UNSUPPORTED;
    if (R == 0) return MOE_OK;
    if (row_scale && !aligned(row_scale, 4)) return MOE_ERR_INVALID;
    if ((a_rows && !aligned(a_rows, 4)) || (out_rows && !aligned(out_rows, 4)))
        return MOE_ERR_INVALID;
    const GemmPlan pl = plan_gemm(R, E, K, N, wtype, act, opts);
    if (pl.ws > 0 && (!ws || ws_bytes < pl.ws || !aligned(ws, 16))) return MOE_ERR_WORKSPACE;
    if (int32_t st = check_device()) return st;

    moe::GemmParams p;
    p.a = a;
    p.a_rows = a_rows;
    p.a_div = a_rows ? a_div : 1;
    p.a_nrows = a_rows ? a_nrows : R;
    p.out_rows = out_rows;
    p.out_nrows = out_rows ? out_nrows : R;
    p.offsets = expert_offsets;
    p.w = w_packed;
    p.scales = scales;
    p.row_scale = row_scale;
    p.out = out;
    p.R = R;
    p.E = E;
    p.K = K;
    p.N = N;
    p.wtype = wtype;
    p.group = group_size;
    p.act = act;
    p.split = pl.split;
    p.tile = opts ? opts->tile : MOE_TILE_AUTO;
    p.i2f = opts ? opts->i2f : MOE_I2F_TRICK;
    p.tiles16 = nullptr;
    hipStream_t s = (hipStream_t)stream;
    return hip_status(pl.path == MOE_PATH_TILE ? moe::launch_gemm_tile(p, s)
                                               : moe::launch_gemm_stream(p, s));
}

int32_t moe_grouped_gemm_wq(const uint16_t* a, const int32_t* expert_offsets, int32_t R,
                            int32_t E, int32_t K, int32_t N, const void* w_packed,
                            const uint16_t* scales, int32_t wtype, int32_t group_size,
                            int32_t act, const float* row_scale, uint16_t* out,
                            const moe_gemm_opts* opts, void* ws, size_t ws_bytes, void* stream) {
    return grouped_gemm(a, R, nullptr, 1, expert_offsets, R, E, K, N, w_packed, scales, wtype,
                        group_size, act, row_scale, out, R, nullptr, opts, ws, ws_bytes, stream);
}

int32_t moe_grouped_gemm_wq_rows(const uint16_t* a, int32_t a_nrows, const int32_t* a_rows,
                                 int32_t a_row_div, const int32_t* expert_offsets, int32_t R,
                                 int32_t E, int32_t K, int32_t N, const void* w_packed,
                                 const uint16_t* scales, int32_t wtype, int32_t group_size,
                                 int32_t act, const float* row_scale, uint16_t* out,
                                 int32_t out_nrows, const int32_t* out_rows,
                                 const moe_gemm_opts* opts, void* ws, size_t ws_bytes,
                                 void* stream) {
    if (a_nrows < 0 || out_nrows < 0) return MOE_ERR_INVALID;
    return grouped_gemm(a, a_rows ? a_nrows : R, a_rows, a_row_div, expert_offsets, R, E, K, N,
                        w_packed, scales, wtype, group_size, act, row_scale, out,
                        out_rows ? out_nrows : R, out_rows, opts, ws, ws_bytes, stream);
}

static int32_t validate_decode(int32_t T, int32_t E, int32_t k, int32_t gate_mode, int32_t d,
                               int32_t inter, int32_t act, int32_t wtype, int32_t group) {
    if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E)
        return MOE_ERR_INVALID;
    if (gate_mode != MOE_GATE_SOFTMAX_TOPK && gate_mode != MOE_GATE_SOFTMAX_ALL)
        return MOE_ERR_INVALID;
    if (act < MOE_ACT_NONE || act > MOE_ACT_SWIGLU) return MOE_ERR_INVALID;
    if (wtype < MOE_W_INT4 || wtype > MOE_W_FP16) return MOE_ERR_INVALID;
    if (d <= 0 || inter <= 0) return MOE_ERR_INVALID;
    if (group != 0 && group != 128) return MOE_ERR_UNSUPPORTED;
    if (wtype == MOE_W_FP16 && group != 0) return MOE_ERR_UNSUPPORTED;
    if (d % 128 != 0 || inter % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if (T > MOE_DECODE_MAX_TOKENS || T * k > MOE_DECODE_MAX_ROWS) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)inter * MOE_DECODE_MAX_ROWS >= (int64_t)1 << 31 ||
        (int64_t)d * MOE_DECODE_MAX_ROWS >= (int64_t)1 << 31)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

size_t moe_decode_workspace_size(int32_t T, int32_t k, int32_t E, int32_t d, int32_t inter,
                                 int32_t wtype) {
    if (validate_decode(T, E, k, MOE_GATE_SOFTMAX_TOPK, d, inter, MOE_ACT_NONE, wtype, 0) !=
        MOE_OK)
        return 0;
    return moe::decode_workspace_layout(T, k, E, d, inter, wtype, 0, nullptr, nullptr);
}

// The shared experts of moe_decode_layer_shared: fp16 weights beside integer-coded routed ones.
static int32_t validate_shared(int32_t wtype, int32_t shared_inter) {
    if (shared_inter <= 0) return MOE_ERR_INVALID;
    if (wtype == MOE_W_FP16 || shared_inter % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)shared_inter * 2 * MOE_DECODE_MAX_TOKENS >= (int64_t)1 << 31)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

size_t moe_decode_shared_workspace_size(int32_t T, int32_t k, int32_t E, int32_t d,
                                        int32_t inter, int32_t wtype, int32_t shared_inter) {
    if (validate_decode(T, E, k, MOE_GATE_SOFTMAX_TOPK, d, inter, MOE_ACT_NONE, wtype, 0) !=
            MOE_OK ||
        validate_shared(wtype, shared_inter) != MOE_OK)
        return 0;
    return moe::decode_workspace_layout(T, k, E, d, inter, wtype, shared_inter, nullptr, nullptr);
}

// moe_decode_layer and moe_decode_layer_shared: sw1 == NULL for no shared experts.
static int32_t decode_layer(const float* logits, const uint8_t* active, const uint16_t* x,
                            int32_t T, int32_t E, int32_t k, int32_t gate_mode, int32_t d,
                            int32_t inter, int32_t act, const void* w1, const uint16_t* s1,
                            const void* w2, const uint16_t* s2, int32_t wtype, int32_t group_size,
                            const void* sw1, const void* sw2, int32_t shared_inter,
                            const uint16_t* addend, void* addend_ready, int32_t* topk_ids,
                            float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                            void* stream) {
    if (int32_t st = validate_decode(T, E, k, gate_mode, d, inter, act, wtype, group_size))
        return st;
    const bool shared = sw1 != nullptr;
    if (shared) {
        if (int32_t st = validate_shared(wtype, shared_inter)) return st;
    }
    if (T == 0) return MOE_OK;
    if (!logits || !x || !w1 || !w2 || !topk_ids || !topk_w || !out) return MOE_ERR_INVALID;
    if (wtype != MOE_W_FP16 && (!s1 || !s2)) return MOE_ERR_INVALID;
    if (shared && !sw2) return MOE_ERR_INVALID;
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) ||
        !aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(out, 16))
        return MOE_ERR_INVALID;
    if ((s1 && !aligned(s1, 16)) || (s2 && !aligned(s2, 16)) || (addend && !aligned(addend, 16)))
        return MOE_ERR_INVALID;
    if (shared && (!aligned(sw1, 16) || !aligned(sw2, 16))) return MOE_ERR_INVALID;
    const size_t need = moe::decode_workspace_layout(T, k, E, d, inter, wtype,
                                                     shared ? shared_inter : 0, nullptr, nullptr);
    if (!ws || ws_bytes < need || !aligned(ws, 16)) return MOE_ERR_WORKSPACE;
    if (int32_t st = check_device()) return st;
    moe::DecodeArgs a;
    a.logits = logits;
    a.active = active;
    a.x = x;
    a.T = T;
    a.E = E;
    a.k = k;
    a.gate_all = gate_mode == MOE_GATE_SOFTMAX_ALL;
    a.d = d;
    a.inter = inter;
    a.act = act;
    a.w1 = w1;
    a.s1 = s1;
    a.w2 = w2;
    a.s2 = s2;
    a.wtype = wtype;
    a.group = group_size;
    a.sw1 = shared ? sw1 : nullptr;
    a.sw2 = shared ? sw2 : nullptr;
    a.shared_inter = shared ? shared_inter : 0;
    a.addend = shared ? nullptr : addend;
    a.addend_ready = shared ? nullptr : addend_ready;
    a.ids = topk_ids;
    a.wts = topk_w;
    a.out = out;
    a.ws = ws;
    return hip_status(moe::launch_decode(a, (hipStream_t)stream));
}

int32_t moe_decode_layer(const float* logits, const uint8_t* active, const uint16_t* x,
                         int32_t T, int32_t E, int32_t k, int32_t gate_mode, int32_t d,
                         int32_t inter, int32_t act,
                         const void* w1, const uint16_t* s1, const void* w2,
                         const uint16_t* s2, int32_t wtype, int32_t group_size,
                         const uint16_t* addend, void* addend_ready, int32_t* topk_ids,
                         float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                         void* stream) {
    return decode_layer(logits, active, x, T, E, k, gate_mode, d, inter, act, w1, s1, w2, s2,
                        wtype, group_size, nullptr, nullptr, 0, addend, addend_ready, topk_ids,
                        topk_w, out, ws, ws_bytes, stream);
}

int32_t moe_decode_layer_shared(const float* logits, const uint8_t* active, const uint16_t* x,
                                int32_t T, int32_t E, int32_t k, int32_t gate_mode, int32_t d,
                                int32_t inter, int32_t act, const void* w1, const uint16_t* s1,
                                const void* w2, const uint16_t* s2, int32_t wtype,
                                int32_t group_size, const void* shared_w1,
                                const void* shared_w2, int32_t shared_inter, int32_t* topk_ids,
                                float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                                void* stream) {
    if (!shared_w1) return MOE_ERR_INVALID;
    return decode_layer(logits, active, x, T, E, k, gate_mode, d, inter, act, w1, s1, w2, s2,
                        wtype, group_size, shared_w1, shared_w2, shared_inter, nullptr, nullptr,
                        topk_ids, topk_w, out, ws, ws_bytes, stream);
}

int32_t moe_decode_layer_noalloc(const float* logits, const uint8_t* active, const uint16_t* x,
                                 int32_t T, int32_t E, int32_t k, int32_t gate_mode, int32_t d,
                                 int32_t inter, int32_t act, const void* w1, const uint16_t* s1,
                                 const void* w2, const uint16_t* s2, int32_t wtype,
                                 int32_t group_size, const uint16_t* addend, void* addend_ready,
                                 int32_t* topk_ids, float* topk_w, uint16_t* out, void* stream) {
    if (int32_t st = validate_decode(T, E, k, gate_mode, d, inter, act, wtype, group_size))
        return st;
    if (T == 0) return MOE_OK;
    const size_t need = moe::decode_workspace_layout(T, k, E, d, inter, wtype, 0, nullptr, nullptr);
    if (need > (size_t)MOE_DECODE_SCRATCH_BYTES) return MOE_ERR_UNSUPPORTED;
    if (int32_t st = check_device()) return st;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_NO_DEVICE;
    void* ws = scratch_address(dev);
    if (!ws) return MOE_ERR_HIP;
    // the rest is moe_decode_layer's validation and launch, on the scratch workspace
    return moe_decode_layer(logits, active, x, T, E, k, gate_mode, d, inter, act, w1, s1, w2, s2,
                            wtype, group_size, addend, addend_ready, topk_ids, topk_w, out, ws,
                            (size_t)MOE_DECODE_SCRATCH_BYTES, stream);
}

int32_t moe_unpermute_combine(const uint16_t* y_perm, const int32_t* inv_perm, const float* topk_w,
                              const uint16_t* addend, int32_t T, int32_t k, int32_t d,
                              uint16_t* out, void* stream) {
    if (T < 0 || k < 1 || k > MOE_MAX_TOPK || d <= 0) return MOE_ERR_INVALID;
    if (d % 8 != 0) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)T * k >= (int64_t)1 << 31 || (int64_t)T * (d / 8) >= (int64_t)1 << 32)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!y_perm || !inv_perm || !out) return MOE_ERR_INVALID;
    if (!aligned(y_perm, 16) || !aligned(out, 16) || !aligned(inv_perm, 4)) return MOE_ERR_INVALID;
    if ((addend && !aligned(addend, 16)) || (topk_w && !aligned(topk_w, 4))) return MOE_ERR_INVALID;
    if (int32_t st = check_device()) return st;
    return hip_status(moe::launch_combine(y_perm, inv_perm, topk_w, addend, T, k, d, out,
                                          (hipStream_t)stream));
}

int32_t moe_elb_accumulate(const int32_t* ids, int32_t L, int32_t T, int32_t k, int32_t E,
                           int32_t* counts, void* stream) {
    if (L < 0 || T < 0 || k < 1 || E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_INVALID;
    if ((int64_t)L * T * k >= (int64_t)1 << 31 || (int64_t)L * E >= (int64_t)1 << 31)
        return MOE_ERR_UNSUPPORTED;
    if (L == 0) return MOE_OK;
    if (!counts || (T > 0 && !ids)) return MOE_ERR_INVALID;
    if (!aligned(counts, 4) || (ids && !aligned(ids, 4))) return MOE_ERR_INVALID;
    if (int32_t st = check_device()) return st;
    return hip_status(moe::launch_elb_accumulate(ids, L, T * k, E, counts, (hipStream_t)stream));
}

int32_t moe_elb_top_m(const int32_t* counts, int32_t L, int32_t E, int32_t M, int32_t* experts,
                      int32_t* top_counts, void* stream) {
    if (L < 0 || E < 1 || E > MOE_MAX_EXPERTS || M < 1 || M > E) return MOE_ERR_INVALID;
    if ((int64_t)L * E >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
    if (L == 0) return MOE_OK;
    if (!counts || !experts) return MOE_ERR_INVALID;
    if (!aligned(counts, 4) || !aligned(experts, 4) || (top_counts && !aligned(top_counts, 4)))
        return MOE_ERR_INVALID;
    if (int32_t st = check_device()) return st;
    return hip_status(moe::launch_elb_top_m(counts, L, E, M, experts, top_counts,
                                            (hipStream_t)stream));
}

int32_t moe_bf16_recombine(const uint8_t* exponents, const uint8_t* sign_mantissa, size_t n,
                           uint16_t* out, void* stream) {
    if (n == 0) return MOE_OK;
    if (n >= (size_t)1 << 40) return MOE_ERR_UNSUPPORTED;
    if (!exponents || !sign_mantissa || !out) return MOE_ERR_INVALID;
    if (!aligned(exponents, 16) || !aligned(sign_mantissa, 16) || !aligned(out, 16))
        return MOE_ERR_INVALID;
    if (int32_t st = check_device()) return st;
    return hip_status(moe::launch_bf16_recombine(exponents, sign_mantissa, n, out,
                                                 (hipStream_t)stream));
}

int32_t moe_dequant(const void* w_packed, const uint16_t* scales, int32_t wtype, int32_t group_size,
                    int32_t E, int32_t K, int32_t N, uint16_t* w_out, void* stream) {
    if (E < 1 || E > MOE_MAX_EXPERTS || K <= 0 || N <= 0) return MOE_ERR_INVALID;
    if (wtype != MOE_W_INT4 && wtype != MOE_W_INT8) return MOE_ERR_INVALID;
    if (group_size != 0 && group_size != 128) return MOE_ERR_UNSUPPORTED;
    if (K % 128 != 0 || N % 16 != 0) return MOE_ERR_UNSUPPORTED;
    if (!w_packed || !scales || !w_out) return MOE_ERR_INVALID;
    if (!aligned(w_packed, 16) || !aligned(scales, 16) || !aligned(w_out, 16)) return MOE_ERR_INVALID;
    if (int32_t st = check_device()) return st;
    return hip_status(moe::launch_dequant(w_packed, scales, wtype, group_size, E, K, N, w_out,
                                          (hipStream_t)stream));
}

}  // extern "C"
