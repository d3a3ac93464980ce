/* Host-side AddressSanitizer driver: the weight packer and the C entry points' argument
 * validation, built with -fsanitize=address on their host code.  Every buffer the packer reads
 * or writes is allocated at exactly the size the header states, so a read or write past it is
 * reported.  Validation calls pass pointers that are never dereferenced (the calls must
 * return before touching them); valid calls return MOE_ERR_NO_DEVICE on a machine without a
 * gfx950 GPU.  Exit status 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_wq.h"

static int failures = 0;
#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond);  \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static void pack_case(int32_t wtype, int32_t E, int32_t K, int32_t N, unsigned seed) {
    const size_t n = (size_t)E * K * N;
    const size_t esz = wtype == MOE_W_FP16 ? 2 : 1;
    unsigned char* codes = (unsigned char*)malloc(n * esz);
    srand(seed);
    for (size_t i = 0; i < n; ++i) {
        if (wtype == MOE_W_INT4) codes[i] = (unsigned char)(int8_t)(rand() % 16 - 8);
        else if (wtype == MOE_W_INT8) codes[i] = (unsigned char)(rand() & 0xFF);
        else ((uint16_t*)codes)[i] = (uint16_t)(rand() & 0x7BFF);
    }
    const size_t bytes = moe_packed_bytes(wtype, E, K, N);
    CHECK(bytes == (wtype == MOE_W_INT4 ? n / 2 : n * esz));
    unsigned char* a = (unsigned char*)malloc(bytes);
    unsigned char* b = (unsigned char*)malloc(bytes);
    CHECK(moe_pack_wq(codes, wtype, E, K, N, a) == MOE_OK);
    CHECK(moe_pack_wq(codes, wtype, E, K, N, b) == MOE_OK);
    CHECK(memcmp(a, b, bytes) == 0);
    /* every code value appears once per packed byte count: the packer is a permutation of the
     * codes (INT8, FP16) or of their nibbles (INT4); compare the multisets */
    if (wtype == MOE_W_INT8) {
        size_t hc[256] = {0}, hp[256] = {0};
        for (size_t i = 0; i < n; ++i) ++hc[(unsigned char)(codes[i] + 128)];
        for (size_t i = 0; i < bytes; ++i) ++hp[a[i]];
        CHECK(memcmp(hc, hp, sizeof hc) == 0);
    } else if (wtype == MOE_W_INT4) {
        size_t hc[16] = {0}, hp[16] = {0};
        for (size_t i = 0; i < n; ++i) ++hc[(unsigned)((int8_t)codes[i] + 8)];
        for (size_t i = 0; i < bytes; ++i) { ++hp[a[i] & 15]; ++hp[a[i] >> 4]; }
        CHECK(memcmp(hc, hp, sizeof hc) == 0);
    }
    free(a);
    free(b);
    free(codes);
}

int main(void) {
    CHECK(moe_version() > 0);
    /* packer: every weight type, the smallest legal shapes, ragged expert counts */
    const int32_t shapes[][3] = {{1, 128, 16}, {3, 128, 48}, {2, 256, 64}, {5, 384, 96}, {1, 1024, 256}};
    for (int s = 0; s < 5; ++s)
        for (int32_t wt = MOE_W_INT4; wt <= MOE_W_FP16; ++wt)
            pack_case(wt, shapes[s][0], shapes[s][1], shapes[s][2], 17u + (unsigned)s);
    /* packer argument errors */
    unsigned char one[64];
    memset(one, 0, sizeof one);
    CHECK(moe_packed_bytes(MOE_W_INT4, 1, 100, 16) == 0);
    CHECK(moe_pack_wq(NULL, MOE_W_INT4, 1, 128, 16, one) == MOE_ERR_INVALID);
    CHECK(moe_pack_wq(one, 7, 1, 128, 16, one) == MOE_ERR_INVALID);
    CHECK(moe_pack_wq(one, MOE_W_INT4, 1, 100, 16, one) == MOE_ERR_UNSUPPORTED);
    {   /* an INT4 code outside [-8, 7] is rejected */
        unsigned char* c = (unsigned char*)calloc(128 * 16, 1);
        unsigned char* p = (unsigned char*)malloc(moe_packed_bytes(MOE_W_INT4, 1, 128, 16));
        c[77] = 9;
        CHECK(moe_pack_wq(c, MOE_W_INT4, 1, 128, 16, p) == MOE_ERR_INVALID);
        free(c);
        free(p);
    }

    /* validation of the device entry points (pointers never dereferenced) */
    void* F = (void*)(uintptr_t)0x10000;        /* 16-byte aligned */
    void* M = (void*)(uintptr_t)0x10002;        /* misaligned */
    CHECK(moe_route_topk((const float*)F, 4, 0, 2, 0, (int32_t*)F, (float*)F, NULL) == MOE_ERR_INVALID);
    CHECK(moe_route_topk((const float*)F, 4, 8, 9, 0, (int32_t*)F, (float*)F, NULL) == MOE_ERR_INVALID);
    CHECK(moe_permute((const int32_t*)F, NULL, NULL, 4, 2, 300, 64, (int32_t*)F, (int32_t*)F,
                      (int32_t*)F, NULL, NULL, NULL, 0, NULL) == MOE_ERR_INVALID);
    CHECK(moe_permute_workspace_size(4097, 2, 8) > 0);
    CHECK(moe_grouped_gemm_wq((const uint16_t*)F, (const int32_t*)F, 64, 8, 200, 64, F,
                              (const uint16_t*)F, MOE_W_INT4, 128, MOE_ACT_RELU, NULL, (uint16_t*)F,
                              NULL, NULL, 0, NULL) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_grouped_gemm_wq((const uint16_t*)M, (const int32_t*)F, 64, 8, 256, 64, F,
                              (const uint16_t*)F, MOE_W_INT4, 128, MOE_ACT_RELU, NULL, (uint16_t*)F,
                              NULL, NULL, 0, NULL) == MOE_ERR_INVALID);
    moe_gemm_opts o;
    memset(&o, 0, sizeof o);
    o.i2f = 3;
    CHECK(moe_grouped_gemm_wq((const uint16_t*)F, (const int32_t*)F, 64, 8, 256, 64, F,
                              (const uint16_t*)F, MOE_W_INT4, 128, MOE_ACT_RELU, NULL, (uint16_t*)F,
                              &o, NULL, 0, NULL) == MOE_ERR_INVALID);
    CHECK(moe_grouped_gemm_wq_rows((const uint16_t*)F, 8, (const int32_t*)F, 0, (const int32_t*)F,
                                   64, 8, 256, 64, F, (const uint16_t*)F, MOE_W_INT4, 128,
                                   MOE_ACT_RELU, NULL, (uint16_t*)F, 64, NULL, NULL, NULL, 0,
                                   NULL) == MOE_ERR_INVALID);
    CHECK(moe_decode_layer((const float*)F, NULL, (const uint16_t*)F, 65, 8, 2, 0, 256, 256,
                           MOE_ACT_RELU, F, (const uint16_t*)F, F, (const uint16_t*)F,
                           MOE_W_INT4, 0, NULL, NULL, (int32_t*)F, (float*)F, (uint16_t*)F,
                           F, 1u << 20, NULL) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_decode_workspace_size(17, 4, 60, 2048, 1408, MOE_W_INT4) > 0);
    CHECK(moe_decode_workspace_size(65, 1, 8, 256, 256, MOE_W_INT4) == 0);
    CHECK(moe_unpermute_combine((const uint16_t*)F, (const int32_t*)F, NULL, NULL, 4, 9, 64,
                                (uint16_t*)F, NULL) == MOE_ERR_INVALID);
    CHECK(moe_dequant(F, (const uint16_t*)M, MOE_W_INT4, 0, 2, 128, 16, (uint16_t*)F, NULL) ==
          MOE_ERR_INVALID);
    CHECK(moe_elb_top_m((const int32_t*)F, 2, 8, 9, (int32_t*)F, (int32_t*)F, NULL) ==
          MOE_ERR_INVALID);
    CHECK(moe_bf16_recombine((const uint8_t*)F, (const uint8_t*)F, 0, (uint16_t*)F, NULL) == MOE_OK);
    /* a valid call reaches the device check (no gfx950 here) */
    CHECK(moe_grouped_gemm_wq((const uint16_t*)F, (const int32_t*)F, 64, 8, 256, 64, F,
                              (const uint16_t*)F, MOE_W_INT4, 128, MOE_ACT_RELU, NULL, (uint16_t*)F,
                              NULL, NULL, 0, NULL) == MOE_ERR_NO_DEVICE);
    CHECK(moe_decode_layer_noalloc((const float*)F, NULL, (const uint16_t*)F, 17, 60, 4, 0, 2048,
                                   1408, MOE_ACT_SWIGLU, F, (const uint16_t*)F, F,
                                   (const uint16_t*)F, MOE_W_INT4, 128, NULL, NULL, (int32_t*)F,
                                   (float*)F, (uint16_t*)F, NULL) == MOE_ERR_NO_DEVICE);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("asan driver: all checks passed\n");
    return 0;
}
