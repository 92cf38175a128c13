/* Drives every function of the CPU oracle (oracle/oracle.c) on small ragged inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  It checks a few
 * identities on the way -- the blocked GEMM equals the naive one, the simulated fused schedule equals
 * gather-then-GEMM, a taller TGATHER destination keeps its extra rows -- but its purpose is that no
 * access falls outside its buffer and no arithmetic is undefined.  Prints OK and returns 0. */
#include "oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint32_t g_state = 12345u;
static uint32_t next_u32(void)
{
    g_state = g_state * 1664525u + 1013904223u;
    return g_state;
}

static uint16_t small_bf16(void)
{
    /* integers in [-3, 3] as bf16, exact */
    return oracle_f32_to_bf16_rne((float)((int)(next_u32() % 7u) - 3));
}

#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            return 1;                                                   \
        }                                                               \
    } while (0)

static int gemm_cases(void)
{
    const int64_t shapes[][3] = {{1, 1, 1}, {5, 7, 3}, {33, 17, 40}, {64, 65, 129}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
        const int64_t M = shapes[s][0], Nc = shapes[s][1], K = shapes[s][2];
        uint16_t *A = malloc(sizeof(uint16_t) * M * K), *B = malloc(sizeof(uint16_t) * Nc * K);
        float *C = malloc(sizeof(float) * M * Nc), *C2 = malloc(sizeof(float) * M * Nc);
        const uint16_t **rows = malloc(sizeof(uint16_t *) * M);
        for (int64_t i = 0; i < M * K; ++i) A[i] = small_bf16();
        for (int64_t i = 0; i < Nc * K; ++i) B[i] = small_bf16();
        for (int64_t i = 0; i < M; ++i) rows[i] = A + i * K;
        oracle_gemm_f32(A, B, M, Nc, K, C);
        oracle_gemm_f32_fast(rows, B, M, Nc, K, C2);
        CHECK(memcmp(C, C2, sizeof(float) * M * Nc) == 0);
        free(A); free(B); free(C); free(C2); free(rows);
    }
    return 0;
}

static int ag_gemm_cases(void)
{
    /* N shards of H rows; the pivoted simulation for every local shard against gather-then-GEMM */
    const int64_t cfg[][6] = {/* N, H, K, Nc, cb, BM */ {3, 10, 12, 9, 4, 8}, {4, 7, 5, 6, 3, 4}, {2, 16, 8, 5, 16, 16}};
    for (size_t s = 0; s < sizeof cfg / sizeof cfg[0]; ++s) {
        const int N = (int)cfg[s][0];
        const int64_t H = cfg[s][1], K = cfg[s][2], Nc = cfg[s][3], cb = cfg[s][4], BM = cfg[s][5];
        const int64_t M = N * H;
        uint16_t **sh = malloc(sizeof(uint16_t *) * N);
        for (int r = 0; r < N; ++r) {
            sh[r] = malloc(sizeof(uint16_t) * H * K);
            for (int64_t i = 0; i < H * K; ++i) sh[r][i] = small_bf16();
        }
        uint16_t *B = malloc(sizeof(uint16_t) * Nc * K);
        for (int64_t i = 0; i < Nc * K; ++i) B[i] = small_bf16();
        uint16_t *A = malloc(sizeof(uint16_t) * M * K), *A2 = malloc(sizeof(uint16_t) * M * K);
        float *C = malloc(sizeof(float) * M * Nc), *C2 = malloc(sizeof(float) * M * Nc);
        CHECK(oracle_ag_gemm((const uint16_t *const *)sh, N, M, K, B, Nc, A, C) == 0);
        CHECK(oracle_ag_gemm_fast((const uint16_t *const *)sh, N, M, K, B, Nc, C2) == 0);
        CHECK(memcmp(C, C2, sizeof(float) * M * Nc) == 0);
        for (int local = 0; local < N; ++local) {
            int64_t stats[6] = {0, 0, 0, 0, 0, 0};
            CHECK(oracle_ag_gemm_pivoted((const uint16_t *const *)sh, N, M, K, B, Nc, cb, BM, 4, 2,
                                         local, A2, C2, stats) == 0);
            CHECK(memcmp(A, A2, sizeof(uint16_t) * M * K) == 0);
            CHECK(memcmp(C, C2, sizeof(float) * M * Nc) == 0);
        }
        int64_t ms[3] = {0, M / 2, M - 1}, ns[3] = {Nc - 1, 0, Nc / 2};
        float at[3];
        CHECK(oracle_ag_gemm_at((const uint16_t *const *)sh, N, M, K, B, Nc, ms, ns, 3, at) == 0);
        for (int i = 0; i < 3; ++i)
            CHECK(at[i] == C[ms[i] * Nc + ns[i]]);
        for (int64_t row = 0; row < M; ++row) {
            const int64_t c = oracle_chunk_of_row(row, H, cb);
            CHECK(c >= 0 && c < N * ((H + cb - 1) / cb));
        }
        int64_t over[64];
        const int64_t n = oracle_chunks_overlapping(0, M, H, cb, over, 64);
        CHECK(n == N * ((H + cb - 1) / cb));
        for (int r = 0; r < N; ++r) free(sh[r]);
        free(sh); free(B); free(A); free(A2); free(C); free(C2);
    }
    int64_t pm, pn;
    for (int64_t t = 0; t < 7 * 5; ++t) {
        oracle_grouped_tile(t, 7, 5, 3, &pm, &pn);
        CHECK(pm >= 0 && pm < 7 && pn >= 0 && pn < 5);
    }
    return 0;
}

static int tgather_cases(void)
{
    const int N = 3;
    const int64_t D0 = 2, D1 = 1, D2 = 2, H = 5, W = 7, rows = N * H + 3;
    for (int esz = 1; esz <= 8; esz *= 2) {
        unsigned char *src[3];
        for (int r = 0; r < N; ++r) {
            src[r] = malloc((size_t)(D0 * D1 * D2 * H * W * esz));
            for (int64_t i = 0; i < D0 * D1 * D2 * H * W * esz; ++i) src[r][i] = (unsigned char)(next_u32() & 0xff);
        }
        const size_t dbytes = (size_t)(D0 * D1 * D2 * rows * W * esz);
        unsigned char *dst = malloc(dbytes);
        memset(dst, 0xab, dbytes);
        CHECK(oracle_tgather((const void *const *)src, N, dst, D0, D1, D2, H, W, rows, esz) == 0);
        /* rows past N*H of every plane are untouched */
        for (int64_t p = 0; p < D0 * D1 * D2; ++p)
            for (int64_t i = (int64_t)N * H * W * esz; i < rows * W * esz; ++i)
                CHECK(dst[p * rows * W * esz + i] == 0xab);
        CHECK(oracle_tgather((const void *const *)src, N, dst, D0, D1, D2, H, W, N * H - 1, esz) != 0);
        CHECK(oracle_tgather((const void *const *)src, N, dst, 0, D1, D2, H, W, rows, esz) == 0);
        for (int r = 0; r < N; ++r) free(src[r]);
        free(dst);
    }
    return 0;
}

static int conversion_cases(void)
{
    for (uint32_t u = 0; u < 65536; ++u) {
        const float f = oracle_bf16_to_f32((uint16_t)u);
        if (!isnan(f))
            CHECK(oracle_f32_to_bf16_rne(f) == (uint16_t)u);
    }
    float xs[1000];
    uint16_t out[1000];
    for (int i = 0; i < 1000; ++i) {
        uint32_t b = next_u32();
        memcpy(&xs[i], &b, 4);
    }
    oracle_f32_to_bf16_array(xs, 1000, out);
    uint8_t codes[256];
    uint16_t img[256];
    for (int c = 0; c < 256; ++c) {
        codes[c] = (uint8_t)c;
        const double v = oracle_e4m3fn_value((uint8_t)c);
        if (!isnan(v))
            CHECK(oracle_f32_to_e4m3fn((float)v) == (uint8_t)c);
    }
    CHECK(oracle_e4m3fn_to_bf16(codes, 256, img) == 0);
    for (int i = 0; i < 1000; ++i)
        (void)oracle_f32_to_e4m3fn(xs[i]);
    return 0;
}

static int reduce_cases(void)
{
    const int64_t H = 9, Nc = 13;
    const int nparts = 5;
    uint16_t *parts[5];
    for (int j = 0; j < nparts; ++j) {
        parts[j] = malloc(sizeof(uint16_t) * H * Nc);
        for (int64_t i = 0; i < H * Nc; ++i) parts[j][i] = small_bf16();
    }
    uint16_t *out = malloc(sizeof(uint16_t) * H * Nc);
    oracle_reduce_block((const uint16_t *const *)parts, nparts, H, Nc, out);
    for (int64_t i = 0; i < H * Nc; ++i) {
        float s = 0.f;
        for (int j = 0; j < nparts; ++j) s += oracle_bf16_to_f32(parts[j][i]);
        CHECK(oracle_bf16_to_f32(out[i]) == s);   /* small integers: exact */
    }
    for (int j = 0; j < nparts; ++j) free(parts[j]);
    free(out);
    return 0;
}

int main(void)
{
    CHECK(oracle_num_threads() >= 1);
    if (gemm_cases() || ag_gemm_cases() || tgather_cases() || conversion_cases() || reduce_cases())
        return 1;
    printf("OK\n");
    return 0;
}
