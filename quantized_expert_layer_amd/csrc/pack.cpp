// Host packer: logical codes [E, K, N] -> the library's packed weight layout.
//
// Packed layout (also described in common.hpp): 16-column blocks, each contiguous along K in
// 1 KiB super-blocks; lane l of a super-block owns column (l & 15) of the block and, inside
// every 32-row K-step, rows 8*(l >> 4) .. +7.
//   INT4: super-block = 128 rows; lane word j = K-step j; 8 codes stored as u = q + 8 in the
//         nibble order [e0,e2,e4,e6,e1,e3,e5,e7] ("Who Says Elephants Can't Run", section 3,
//         4-bit variant of the optimized I2F).
//   INT8: super-block = 64 rows; lane words 2j, 2j+1 = K-step j rows 0..3 / 4..7; bytes in
//         row order, stored as u = q + 128 (the 8-bit variant subtracts 1024 + 128).
//   FP16: super-block = 32 rows; the lane's 8 halves in row order.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "moe_wq.h"

namespace {

int ksb_of(int32_t wtype) { return wtype == MOE_W_INT4 ? 128 : (wtype == MOE_W_INT8 ? 64 : 32); }

bool shape_ok(int32_t wtype, int32_t E, int32_t K, int32_t N) {
    if (wtype < MOE_W_INT4 || wtype > MOE_W_FP16) return false;
    if (E < 1 || K <= 0 || N <= 0) return false;
    return K % 128 == 0 && N % 16 == 0;
}

// Pack experts [e_lo, e_hi); returns false if a code is out of range.
bool pack_range(const void* codes, int32_t wtype, int32_t K, int32_t N, uint32_t* out, int e_lo,
                int e_hi) {
    static const int kOrder[8] = {0, 2, 4, 6, 1, 3, 5, 7};   // code index at nibble p
    const int KSB = ksb_of(wtype);
    const int nSB = K / KSB, ncb = N / 16;
    bool ok = true;
    for (int e = e_lo; e < e_hi; ++e) {
        for (int cb = 0; cb < ncb; ++cb) {
            for (int kb = 0; kb < nSB; ++kb) {
                uint32_t* sbp = out + (((size_t)e * ncb + cb) * nSB + kb) * 256;
                for (int l = 0; l < 64; ++l) {
                    const int n = cb * 16 + (l & 15);
                    for (int w = 0; w < 4; ++w) {
                        uint32_t word = 0;
                        if (wtype == MOE_W_INT4) {
                            const int k0 = kb * 128 + w * 32 + 8 * (l >> 4);
                            const int8_t* c = (const int8_t*)codes + ((size_t)e * K + k0) * N + n;
                            for (int p = 0; p < 8; ++p) {
                                const int q = c[(size_t)kOrder[p] * N];
                                if (q < -8 || q > 7) ok = false;
                                word |= (uint32_t)((q + 8) & 0xF) << (4 * p);
                            }
                        } else if (wtype == MOE_W_INT8) {
                            const int k0 = kb * 64 + (w >> 1) * 32 + 8 * (l >> 4) + 4 * (w & 1);
                            const int8_t* c = (const int8_t*)codes + ((size_t)e * K + k0) * N + n;
                            for (int b = 0; b < 4; ++b)
                                word |= (uint32_t)((c[(size_t)b * N] + 128) & 0xFF) << (8 * b);
                        } else {
                            const int k0 = kb * 32 + 8 * (l >> 4) + 2 * w;
                            const uint16_t* c = (const uint16_t*)codes + ((size_t)e * K + k0) * N + n;
                            word = (uint32_t)c[0] | ((uint32_t)c[N] << 16);
                        }
                        sbp[l * 4 + w] = word;
                    }
                }
            }
        }
    }
    return ok;
}

}  // namespace

extern "C" {

size_t moe_packed_bytes(int32_t wtype, int32_t E, int32_t K, int32_t N) {
    if (!shape_ok(wtype, E, K, N)) return 0;
    const size_t n = (size_t)E * K * N;
    return wtype == MOE_W_INT4 ? n / 2 : (wtype == MOE_W_INT8 ? n : 2 * n);
}

int32_t moe_pack_wq(const void* codes, int32_t wtype, int32_t E, int32_t K, int32_t N,
                    void* packed) {
    if (!codes || !packed) return MOE_ERR_INVALID;
    if (wtype < MOE_W_INT4 || wtype > MOE_W_FP16 || E < 1 || K <= 0 || N <= 0)
        return MOE_ERR_INVALID;
    if (!shape_ok(wtype, E, K, N)) return MOE_ERR_UNSUPPORTED;
    const unsigned hw = std::max(1u, std::thread::hardware_concurrency());
    const int nthreads = (int)std::min<unsigned>(std::min<unsigned>(hw, 16u), (unsigned)E);
    std::vector<char> ok(nthreads, 1);
    std::vector<std::thread> pool;
    for (int t = 0; t < nthreads; ++t) {
        const int lo = (int)((int64_t)E * t / nthreads), hi = (int)((int64_t)E * (t + 1) / nthreads);
        pool.emplace_back([=, &ok]() {
            ok[t] = pack_range(codes, wtype, K, N, (uint32_t*)packed, lo, hi) ? 1 : 0;
        });
    }
    for (auto& th : pool) th.join();
    for (char v : ok)
        if (!v) return MOE_ERR_INVALID;
    return MOE_OK;
}

}  // extern "C"
