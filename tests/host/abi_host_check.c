/*
 * Host-side checks of the C ABI (include/mnb.h) meant to run under
 * AddressSanitizer and UndefinedBehaviorSanitizer: argument validation,
 * status strings, packed sizes and grouped plans, written and re-checked on
 * the host. Every call here returns before anything would be enqueued on a
 * GPU (device pointers are never dereferenced on the host), so the program
 * needs no GPU. Exit status 0 when every check holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mnb.h"

static int failures = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

/* A fake, 256-byte aligned device address: only its value is ever used. */
static void *dev(uintptr_t k) { return (void *)(uintptr_t)(0x100000000ull + k * 0x100000ull); }

static void check_status_strings(void) {
    for (int s = -3; s < 20; ++s) {
        const char *t = mnb_status_string(s);
        CHECK(t != NULL && strlen(t) > 0);
    }
    CHECK(strcmp(mnb_status_string(MNB_OK), "ok") == 0);
    CHECK(mnb_abi_version() == MNB_ABI_VERSION);
}

static void check_packed_bytes(void) {
    const int bss[4] = {32, 64, 128, 256};
    for (int i = 0; i < 4; ++i) {
        for (int64_t n = 1; n <= 70; n += 23) {
            for (int64_t k = bss[i]; k <= 4 * 1024; k += 3 * bss[i]) {
                size_t b16 = mnb_packed_bytes(n, k, 4, bss[i], MNB_F16);
                size_t b32 = mnb_packed_bytes(n, k, 4, bss[i], MNB_F32);
                CHECK(b16 > 0 && b32 >= b16);
                CHECK(b16 % 256 == 0);
                CHECK(b16 >= (size_t)(n * k / 2));
            }
        }
    }
    CHECK(mnb_packed_bytes(0, 128, 4, 32, MNB_F16) == 0);
    CHECK(mnb_packed_bytes(16, 100, 4, 32, MNB_F16) == 0);
    CHECK(mnb_packed_bytes(16, 128, 8, 32, MNB_F16) == 0);
    CHECK(mnb_packed_bytes(16, 128, 4, 16, MNB_F16) == 0);
    CHECK(mnb_packed_bytes(16, 128, 4, 32, 7) == 0);
    CHECK(mnb_packed_bytes(16, MNB_MAX_K + 32, 4, 32, MNB_F16) == 0);
    CHECK(mnb_packed_bytes(INT64_MAX, 128, 4, 32, MNB_F16) == 0);
    CHECK(mnb_packed_bytes(-5, 128, 4, 32, MNB_F16) == 0);
}

static void check_invalid_calls(void) {
    void *x = dev(1), *w = dev(2), *y = dev(3), *ws = dev(4);
    int64_t *idx = (int64_t *)dev(5);
    /* each of these must be refused on the host */
    CHECK(mnb_gemm(NULL, w, y, 4, 64, 128, 4, 32, MNB_F16, NULL) == MNB_ERR_NULL);
    CHECK(mnb_gemm(x, w, y, 4, 64, 128, 3, 32, MNB_F16, NULL) == MNB_ERR_BITS);
    CHECK(mnb_gemm(x, w, y, 4, 64, 128, 4, 48, MNB_F16, NULL) == MNB_ERR_BLOCK);
    CHECK(mnb_gemm(x, w, y, 4, 64, 100, 4, 32, MNB_F16, NULL) == MNB_ERR_SHAPE);
    CHECK(mnb_gemm(x, w, y, 0, 64, 128, 4, 32, MNB_F16, NULL) == MNB_ERR_SHAPE);
    CHECK(mnb_gemm(x, w, y, -1, 64, 128, 4, 32, MNB_F16, NULL) == MNB_ERR_SHAPE);
    CHECK(mnb_gemm(x, w, y, INT64_MAX, 64, 128, 4, 32, MNB_F16, NULL) == MNB_ERR_SHAPE);
    CHECK(mnb_gemm(x, w, y, 4, 64, 128, 4, 32, 9, NULL) == MNB_ERR_DTYPE);
    CHECK(mnb_gemm((char *)x + 2, w, y, 4, 64, 128, 4, 32, MNB_F16, NULL) == MNB_ERR_ALIGN);
    CHECK(mnb_gemv(x, w, (char *)y + 8, 64, 128, 4, 32, MNB_F16, NULL) == MNB_ERR_ALIGN);
    CHECK(mnb_gemv(x, w, y, 64, MNB_MAX_K * 2, 4, 32, MNB_F16, NULL) == MNB_ERR_SHAPE);
    /* index NULL asks for the partial results only: accepted, so this fails on bits */
    CHECK(mnb_gemv_argmax(x, w, y, NULL, ws, 64, 128, 3, 32, MNB_F16, NULL) == MNB_ERR_BITS);
    CHECK(mnb_embed_gather_argmax((const int8_t *)w, (const float *)x, NULL, idx, 100, 64, MNB_F16, y, NULL) ==
          MNB_ERR_NULL);
    CHECK(mnb_embed_gather_argmax((const int8_t *)w, (const float *)x, ws, NULL, 100, 17, MNB_F16, y, NULL) ==
          MNB_ERR_SHAPE);
    CHECK(mnb_embed_gather_argmax((const int8_t *)w, (const float *)x, ws, NULL, 100, 64, 7, y, NULL) ==
          MNB_ERR_DTYPE);
    CHECK(mnb_embed_gather_argmax((const int8_t *)w, (const float *)x, (char *)ws + 8, NULL, 100, 64, MNB_F16, y,
                                  NULL) == MNB_ERR_ALIGN);
    CHECK(mnb_gemv_argmax(x, w, y, idx, NULL, 64, 128, 4, 32, MNB_F16, NULL) == MNB_ERR_NULL);
    CHECK(mnb_gemv_argmax(x, w, y, (int64_t *)((char *)idx + 4), ws, 64, 128, 4, 32, MNB_F16, NULL) ==
          MNB_ERR_ALIGN);
    CHECK(mnb_gemv_argmax(x, w, NULL, idx, ws, 64, 96, 4, 64, MNB_F16, NULL) == MNB_ERR_SHAPE);
    CHECK(mnb_quantize_rtn(NULL, 64, 128, 4, 32, MNB_F16, w, y, x, NULL) == MNB_ERR_NULL);
    CHECK(mnb_quantize_rtn((const float *)x, 64, 100, 4, 32, MNB_F16, w, y, x, NULL) == MNB_ERR_SHAPE);
    CHECK(mnb_pack(w, y, x, 64, 128, 4, 32, MNB_F16, NULL, NULL) == MNB_ERR_NULL);
    CHECK(mnb_pack(w, y, x, 64, 128, 4, 32, MNB_F16, (char *)ws + 1, NULL) == MNB_ERR_ALIGN);
    CHECK(mnb_unpack(w, 64, 128, 4, 32, MNB_F16, NULL, x, NULL) == MNB_ERR_NULL);
    CHECK(mnb_dequant(w, 64, 128, 4, 64, MNB_F32, NULL, NULL) == MNB_ERR_NULL);
    CHECK(mnb_dequant(w, 64, 96, 4, 64, MNB_F32, y, NULL) == MNB_ERR_SHAPE);
    CHECK(mnb_embed_gather((const int8_t *)w, (const float *)x, (const int64_t *)ws, 4, 100, 17, MNB_F16, y,
                           NULL) == MNB_ERR_SHAPE);
    CHECK(mnb_embed_gather((const int8_t *)w, (const float *)x, (const int64_t *)ws, -1, 100, 16, MNB_F16, y,
                           NULL) == MNB_ERR_SHAPE);
    CHECK(mnb_embed_gather((const int8_t *)w, (const float *)x, (const int64_t *)ws, 0, 100, 16, MNB_F16, y,
                           NULL) == MNB_OK);
    /* split-K */
    CHECK(mnb_gemm_split_k_workspace_bytes(1, 2048, 2048, 4, 32, MNB_F16, 0) == 0);
    CHECK(mnb_gemm_split_k_workspace_bytes(410, 2048, 2048, 4, 32, MNB_F32, 0) == 0);
    CHECK(mnb_gemm_split_k_workspace_bytes(410, 2048, 2048, 4, 32, MNB_F16, 1) == 0);
    CHECK(mnb_gemm_split_k_workspace_bytes(410, 2048, 2048, 4, 32, MNB_F16, 4) >= (size_t)4 * 410 * 2048 * 4);
    CHECK(mnb_gemm_split_k_workspace_bytes(410, 2048, 2048, 4, 32, MNB_F16, 0) > 0);
    CHECK(mnb_gemm_split_k_workspace_bytes(410, 2048, 2048, 4, 32, MNB_F16, MNB_MAX_KSPLIT + 1) == 0);
    CHECK(mnb_gemm_split_k_workspace_bytes(410, 2048, 2048, 4, 32, MNB_F16, -1) == 0);
    CHECK(mnb_gemm_split_k_workspace_bytes(410, 2048, 100, 4, 32, MNB_F16, 0) == 0);
    /* a split never exceeds the K-tiles: 2 tiles, 16 asked */
    CHECK(mnb_gemm_split_k_workspace_bytes(64, 64, 256, 4, 32, MNB_F16, 16) ==
          mnb_gemm_split_k_workspace_bytes(64, 64, 256, 4, 32, MNB_F16, 2));
    {
        const size_t need = mnb_gemm_split_k_workspace_bytes(64, 64, 2048, 4, 32, MNB_F16, 4);
        CHECK(mnb_gemm_split_k(x, w, y, NULL, need, 64, 64, 2048, 4, 32, MNB_F16, 4, NULL) == MNB_ERR_NULL);
        CHECK(mnb_gemm_split_k(x, w, y, ws, need - 1, 64, 64, 2048, 4, 32, MNB_F16, 4, NULL) == MNB_ERR_INVALID);
        CHECK(mnb_gemm_split_k(x, w, y, (char *)ws + 4, need, 64, 64, 2048, 4, 32, MNB_F16, 4, NULL) ==
              MNB_ERR_ALIGN);
        CHECK(mnb_gemm_split_k(x, w, y, ws, need, 64, 64, 2048, 4, 32, MNB_F16, 17, NULL) == MNB_ERR_INVALID);
        CHECK(mnb_gemm_split_k(x, w, y, ws, need, 64, 64, 2000, 4, 32, MNB_F16, 4, NULL) == MNB_ERR_SHAPE);
    }
    /* int8 compute mode */
    CHECK(mnb_gemm_i8_workspace_bytes(1, 4096, 32) == 0);
    {
        mnb_problem pr[3];
        memset(pr, 0, sizeof(pr));
        for (int i = 0; i < 3; ++i) {
            pr[i].x = dev(40 + 3 * (uintptr_t)i);
            pr[i].packed = dev(41 + 3 * (uintptr_t)i);
            pr[i].y = dev(42 + 3 * (uintptr_t)i);
            pr[i].M = 1;
            pr[i].N = 1000 + 77 * i;
            pr[i].K = 1024 * (i + 1);
        }
        const size_t bytes = mnb_plan_bytes(3);
        uint8_t *plan = (uint8_t *)malloc(bytes);
        CHECK(mnb_plan_grouped_i8(pr, 3, 4, 32, MNB_F16, plan, bytes) == MNB_OK);
        CHECK(mnb_plan_launches(plan) == 1);
        pr[1].M = 2;
        CHECK(mnb_plan_grouped_i8(pr, 3, 4, 32, MNB_F16, plan, bytes) == MNB_ERR_SHAPE);
        free(plan);
    }
    const size_t wsb = mnb_gemm_i8_workspace_bytes(4, 128, 32);
    CHECK(wsb >= 4 * 128 && wsb % 256 == 0);
    CHECK(mnb_gemm_i8_workspace_bytes(410, 2048, 64) >= (size_t)(410 * 2048 + 410 * 32 * 4 + 410 * 64 * 4));
    CHECK(mnb_gemm_i8_workspace_bytes(0, 128, 32) == 0);
    CHECK(mnb_gemm_i8_workspace_bytes(4, 100, 32) == 0);
    CHECK(mnb_gemm_i8_workspace_bytes(4, 128, 48) == 0);
    CHECK(mnb_gemm_i8(x, w, y, NULL, wsb, 4, 64, 128, 4, 32, MNB_F16, NULL) == MNB_ERR_NULL);
    CHECK(mnb_gemm_i8(x, w, y, ws, wsb - 1, 4, 64, 128, 4, 32, MNB_F16, NULL) == MNB_ERR_INVALID);
    CHECK(mnb_gemm_i8(x, w, y, (char *)ws + 8, wsb, 4, 64, 128, 4, 32, MNB_F16, NULL) == MNB_ERR_ALIGN);
    CHECK(mnb_gemm_i8(x, w, y, ws, wsb, 4, 64, 100, 4, 32, MNB_F16, NULL) == MNB_ERR_SHAPE);
    CHECK(mnb_gemm_i8(x, w, y, ws, wsb, 0, 64, 128, 4, 32, MNB_F16, NULL) == MNB_ERR_SHAPE);
    CHECK(mnb_gemm_i8(x, w, y, ws, wsb, 4, 64, 128, 4, 32, 5, NULL) == MNB_ERR_DTYPE);
    CHECK(mnb_quantize_act_i8(x, 4, 128, 32, MNB_F16, NULL, (float *)y, NULL) == MNB_ERR_NULL);
    CHECK(mnb_quantize_act_i8(x, 4, 100, 32, MNB_F16, (int8_t *)w, (float *)y, NULL) == MNB_ERR_SHAPE);
    CHECK(mnb_quantize_act_i8(x, 4, 128, 32, MNB_F16, (int8_t *)w + 4, (float *)y, NULL) == MNB_ERR_ALIGN);
}

/* Writes a plan for `count` products of mixed kinds and returns its status. */
static int write_plan(int count, unsigned seed, uint8_t **plan_out, size_t *bytes_out) {
    mnb_problem *pr = (mnb_problem *)calloc((size_t)count, sizeof(mnb_problem));
    if (!pr) return -1;
    unsigned s = seed;
    for (int i = 0; i < count; ++i) {
        s = s * 1103515245u + 12345u;
        const int64_t ms[6] = {1, 1, 7, 62, 410, 1500};
        pr[i].M = ms[(s >> 8) % 6];
        pr[i].N = 16 + (int64_t)((s >> 12) % 3000);
        pr[i].K = 128 * (1 + (int64_t)((s >> 20) % 48));
        pr[i].x = dev(10 + 3 * (uintptr_t)i);
        pr[i].packed = dev(11 + 3 * (uintptr_t)i);
        pr[i].y = dev(12 + 3 * (uintptr_t)i);
    }
    size_t bytes = mnb_plan_bytes(count);
    uint8_t *plan = (uint8_t *)malloc(bytes);
    int st = plan ? mnb_plan_grouped(pr, count, 4, 32, MNB_F16, plan, bytes) : -1;
    free(pr);
    *plan_out = plan;
    *bytes_out = bytes;
    return st;
}

static void check_plans(void) {
    CHECK(mnb_plan_bytes(0) == 0);
    CHECK(mnb_plan_bytes(-1) == 0);
    CHECK(mnb_plan_bytes(65537) == 0);
    CHECK(mnb_plan_bytes(1) > 0);
    const int counts[6] = {1, 2, 7, 197, 1000, 4096};
    for (int c = 0; c < 6; ++c) {
        uint8_t *plan = NULL;
        size_t bytes = 0;
        int st = write_plan(counts[c], 17u + (unsigned)c, &plan, &bytes);
        CHECK(st == MNB_OK);
        if (st == MNB_OK) {
            int n = mnb_plan_launches(plan);
            CHECK(n >= 1 && n <= 16);
            /* corrupted images are refused on the host, before any launch */
            uint8_t *bad = (uint8_t *)malloc(bytes);
            memcpy(bad, plan, bytes);
            bad[0] ^= 0xFF;
            CHECK(mnb_plan_launches(bad) == -1);
            CHECK(mnb_gemm_grouped(bad, dev(99), NULL) == MNB_ERR_PLAN);
            memcpy(bad, plan, bytes);
            memset(bad + 8, 0xFF, 4); /* count */
            CHECK(mnb_gemm_grouped(bad, dev(99), NULL) == MNB_ERR_PLAN);
            CHECK(mnb_gemm_grouped(plan, (char *)dev(99) + 4, NULL) == MNB_ERR_ALIGN);
            CHECK(mnb_gemm_grouped(NULL, dev(99), NULL) == MNB_ERR_NULL);
            free(bad);
        }
        free(plan);
    }
    /* a plan buffer one byte short, and an invalid product inside a plan */
    mnb_problem p[2];
    memset(p, 0, sizeof(p));
    p[0].x = dev(1); p[0].packed = dev(2); p[0].y = dev(3); p[0].M = 4; p[0].N = 64; p[0].K = 128;
    p[1] = p[0];
    size_t bytes = mnb_plan_bytes(2);
    uint8_t *plan = (uint8_t *)malloc(bytes);
    CHECK(mnb_plan_grouped(p, 2, 4, 32, MNB_F16, plan, bytes - 1) == MNB_ERR_PLAN);
    p[1].K = 100;
    CHECK(mnb_plan_grouped(p, 2, 4, 32, MNB_F16, plan, bytes) == MNB_ERR_SHAPE);
    p[1].K = 128;
    p[1].y = NULL;
    CHECK(mnb_plan_grouped(p, 2, 4, 32, MNB_F16, plan, bytes) == MNB_ERR_NULL);
    CHECK(mnb_plan_grouped(NULL, 2, 4, 32, MNB_F16, plan, bytes) == MNB_ERR_NULL);
    CHECK(mnb_plan_grouped(p, 0, 4, 32, MNB_F16, plan, bytes) == MNB_ERR_PLAN);
    free(plan);
}

int main(void) {
    check_status_strings();
    check_packed_bytes();
    check_invalid_calls();
    check_plans();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("abi host checks passed\n");
    return 0;
}
