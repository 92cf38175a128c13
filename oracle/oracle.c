/*
 * oracle.c -- CPU oracle for the chunked AllGather + bf16 GEMM path and for TGATHER.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the benchmark's CPU
 * baseline, never by the GPU library.  It shares no code, header or table with the HIP path.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC oracle.c -o liboracle.so
 * (-ffp-contract=off keeps every multiply and add a separately rounded fp32 operation).
 *
 * Every function states the passage of the two pages it follows; see oracle.h for the page
 * titles.  Parity pins for each function live in tests/test_oracle.py.
 */
#include "oracle.h"

#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);           /* NaN: keep sign, force quiet */
    uint32_t lsb = (u >> 16) & 1u;                         /* ties go to the even result */
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* [TGATH] §二 数学语义 (closed form), §7.2 内存约束 (taller dst keeps its extra rows),
 * §7.4 (empty data moves nothing), §6.3 CPU_SIM (element copy semantics). */
int oracle_tgather(const void *const *src, int nranks, void *dst,
                   int64_t D0, int64_t D1, int64_t D2, int64_t H, int64_t W,
                   int64_t dst_rows, int elem_size)
{
    if (nranks <= 0 || elem_size <= 0 || D0 < 0 || D1 < 0 || D2 < 0 || H < 0 || W < 0)
        return -1;
    if (dst_rows < (int64_t)nranks * H)
        return -1;
    const size_t row_bytes = (size_t)W * (size_t)elem_size;
    for (int64_t d0 = 0; d0 < D0; ++d0)
        for (int64_t d1 = 0; d1 < D1; ++d1)
            for (int64_t d2 = 0; d2 < D2; ++d2) {
                const int64_t plane = (d0 * D1 + d1) * D2 + d2;   /* outer index, same in src and dst */
                for (int r = 0; r < nranks; ++r)
                    for (int64_t i = 0; i < H; ++i) {
                        const char *s = (const char *)src[r] + (size_t)(plane * H + i) * row_bytes;
                        char *d = (char *)dst + (size_t)(plane * dst_rows + (int64_t)r * H + i) * row_bytes;
                        memcpy(d, s, row_bytes);   /* dst row r*H + i <- src_r row i */
                    }
            }
    return 0;
}

/* One output element: ascending-k fp32 dot product of an A row and a B row (both K long). */
static float dot_ascending_f32(const uint16_t *a_row, const uint16_t *b_row, int64_t K)
{
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float prod = oracle_bf16_to_f32(a_row[k]) * oracle_bf16_to_f32(b_row[k]);
        acc = acc + prod;
    }
    return acc;
}

/* [AGMM] §对称内存如何打通GPU间访问: a is (m,k), b is materialised as (n,k), c = a @ b^T. */
void oracle_gemm_f32(const uint16_t *A, const uint16_t *B, int64_t M, int64_t Nc, int64_t K,
                     float *C)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < Nc; ++n)
            C[m * Nc + n] = dot_ascending_f32(A + m * K, B + n * K, K);
}

/* Row m of the gathered A: row m % H of shard m / H ([AGMM] §从集合通信理解数据流, AllGather
 * concatenates the shards in rank order; [TGATH] §二 with D0=D1=D2=1). */
static const uint16_t *gathered_row(const uint16_t *const *shards, int64_t H, int64_t K, int64_t m)
{
    return shards[m / H] + (m % H) * K;
}

int oracle_ag_gemm_at(const uint16_t *const *shards, int nshards, int64_t M, int64_t K,
                      const uint16_t *B, int64_t Nc, const int64_t *ms, const int64_t *ns,
                      int64_t count, float *out)
{
    if (nshards <= 0 || M % nshards != 0 || K < 0)
        return -1;
    const int64_t H = M / nshards;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= Nc)
            return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = dot_ascending_f32(gathered_row(shards, H, K, ms[i]), B + ns[i] * K, K);
    return 0;
}

/* [AGMM] §为什么要融合 AllGather 与 MatMul: the naive schedule -- finish the AllGather, then run
 * the MatMul on the concatenated tensor. */
int oracle_ag_gemm(const uint16_t *const *shards, int nshards, int64_t M, int64_t K,
                   const uint16_t *B, int64_t Nc, uint16_t *A_out, float *C)
{
    if (nshards <= 0 || M % nshards != 0)
        return -1;
    const int64_t H = M / nshards;
    const void *const *src = (const void *const *)shards;
    int rc = oracle_tgather(src, nshards, A_out, 1, 1, 1, H, K, M, (int)sizeof(uint16_t));
    if (rc != 0)
        return rc;
    oracle_gemm_f32(A_out, B, M, Nc, K, C);
    return 0;
}

/* [AGMM] §融合后的流水线 (chunks along M), §数据搬运与细粒度同步 (one flag per
 * (source rank, split) pair, index src_rank * splits_per_rank + split_id). */
int64_t oracle_chunk_of_row(int64_t row, int64_t H, int64_t cb)
{
    const int64_t S = (H + cb - 1) / cb;    /* chunks per shard */
    const int64_t r = row / H;              /* source shard */
    const int64_t s = (row % H) / cb;       /* split within the shard */
    return r * S + s;
}

int64_t oracle_chunks_overlapping(int64_t m0, int64_t m1, int64_t H, int64_t cb, int64_t *out,
                                  int64_t cap)
{
    int64_t n = 0;
    int64_t last = -1;
    for (int64_t m = m0; m < m1; ++m) {     /* row by row: plain, and obviously complete */
        int64_t c = oracle_chunk_of_row(m, H, cb);
        if (c != last) {
            if (n < cap)
                out[n] = c;
            ++n;
            last = c;
        }
    }
    return n;
}

/* Grouped ("swizzled") order of output tiles: consecutive tile ids walk down group_m tile rows
 * before moving to the next tile column, so neighbouring tiles share A rows and B rows. */
void oracle_grouped_tile(int64_t t, int64_t num_pid_m, int64_t num_pid_n, int64_t group_m,
                         int64_t *pid_m, int64_t *pid_n)
{
    const int64_t tiles_per_group = group_m * num_pid_n;
    const int64_t group = t / tiles_per_group;
    const int64_t first_m = group * group_m;
    int64_t rows_in_group = num_pid_m - first_m;
    if (rows_in_group > group_m)
        rows_in_group = group_m;
    const int64_t in_group = t % tiles_per_group;
    *pid_m = first_m + in_group % rows_in_group;
    *pid_n = in_group / rows_in_group;
}

/* Producer state of the simulation: chunks are published strictly in ready order. */
typedef struct {
    const uint16_t *const *shards;
    int nshards, local;
    int64_t H, K, cb, S;
    int64_t next;            /* position in ready order of the next chunk to publish */
    unsigned char *published;
    uint16_t *A_prime;
} sim_producer;

static int64_t ready_order_chunk(const sim_producer *p, int64_t pos)
{
    /* Remote shards in the order local+1, local+2, ... (the order the rotated tiles consume
     * them), then the local shard, whose rows no tile waits for. */
    const int64_t q = pos / p->S, s = pos % p->S;
    const int64_t r = (p->local + 1 + q) % p->nshards;
    return r * p->S + s;
}

static void publish_next(sim_producer *p)
{
    const int64_t c = ready_order_chunk(p, p->next++);
    const int64_t r = c / p->S, s = c % p->S;
    const int64_t row0 = s * p->cb;
    int64_t row1 = row0 + p->cb;
    if (row1 > p->H)
        row1 = p->H;
    /* copy first, then raise the flag: data must be visible before the signal
     * ([AGMM] §数据搬运与细粒度同步, happens-before between data and signal) */
    for (int64_t i = row0; i < row1; ++i)
        memcpy(p->A_prime + (r * p->H + i) * p->K, p->shards[r] + i * p->K,
               (size_t)p->K * sizeof(uint16_t));
    p->published[c] = 1;
}

int oracle_ag_gemm_pivoted(const uint16_t *const *shards, int nshards, int64_t M, int64_t K,
                           const uint16_t *B, int64_t Nc, int64_t cb, int64_t BM, int64_t BN,
                           int64_t group_m, int local_rank, uint16_t *A_prime, float *C,
                           int64_t *stats)
{
    if (nshards <= 0 || M <= 0 || M % nshards != 0 || cb <= 0 || BM <= 0 || BN <= 0 ||
        group_m <= 0 || local_rank < 0 || local_rank >= nshards || Nc <= 0 || K < 0)
        return -1;
    const int64_t H = M / nshards;
    const int64_t S = (H + cb - 1) / cb;
    const int64_t nchunks = (int64_t)nshards * S;
    const int64_t num_pid_m = (M + BM - 1) / BM, num_pid_n = (Nc + BN - 1) / BN;
    const int64_t pivot = ((int64_t)local_rank * H) / BM;  /* tile row holding the local start */
    const int64_t lo = (int64_t)local_rank * H, hi = lo + H;  /* local rows [lo, hi) */

    for (int64_t i = 0; i < M * K; ++i)
        A_prime[i] = 0x7fc0;                                /* bf16 quiet NaN poison */

    sim_producer p = {shards, nshards, local_rank, H, K, cb, S, 0, NULL, A_prime};
    p.published = (unsigned char *)calloc((size_t)nchunks, 1);
    int64_t *need = (int64_t *)malloc(sizeof(int64_t) * (size_t)(BM + 1));
    if (!p.published || !need) {
        free(p.published);
        free(need);
        return -1;
    }
    int64_t waited_tiles = 0, flag_checks = 0, local_tiles = 0;
    int64_t first_pid_m = -1, tiles_before_first_remote = -1;
    int rc = 0;

    for (int64_t t = 0; t < num_pid_m * num_pid_n && rc == 0; ++t) {
        int64_t pid_m, pid_n;
        oracle_grouped_tile(t, num_pid_m, num_pid_n, group_m, &pid_m, &pid_n);
        pid_m = (pid_m + pivot) % num_pid_m;                /* rotate to the local start */
        const int64_t m0 = pid_m * BM, m1 = (m0 + BM < M) ? m0 + BM : M;
        const int64_t n0 = pid_n * BN, n1 = (n0 + BN < Nc) ? n0 + BN : Nc;
        const int is_local = (m0 >= lo && m1 <= hi);
        if (t == 0)
            first_pid_m = pid_m;
        if (!is_local && tiles_before_first_remote < 0)
            tiles_before_first_remote = t;

        if (is_local) {
            ++local_tiles;
        } else {
            /* wait only on the chunks this tile reads */
            int64_t nneed = oracle_chunks_overlapping(m0, m1, H, cb, need, BM + 1);
            int waited = 0;
            for (int64_t j = 0; j < nneed; ++j) {
                ++flag_checks;
                while (!p.published[need[j]]) {
                    publish_next(&p);
                    waited = 1;
                }
            }
            waited_tiles += waited;
        }
        for (int64_t m = m0; m < m1; ++m) {
            const uint16_t *a_row;
            if (is_local) {
                a_row = shards[local_rank] + (m - lo) * K;
            } else {
                if (!p.published[oracle_chunk_of_row(m, H, cb)]) {
                    rc = -2;                                /* read before publication */
                    break;
                }
                a_row = A_prime + m * K;
            }
            for (int64_t n = n0; n < n1; ++n)
                C[m * Nc + n] = dot_ascending_f32(a_row, B + n * K, K);
        }
    }
    const int64_t published_before_drain = p.next;
    while (rc == 0 && p.next < nchunks)                     /* drain: A_prime ends as the full gather */
        publish_next(&p);

    if (stats) {
        stats[0] = waited_tiles;
        stats[1] = flag_checks;
        stats[2] = local_tiles;
        stats[3] = first_pid_m;
        stats[4] = tiles_before_first_remote < 0 ? num_pid_m * num_pid_n : tiles_before_first_remote;
        stats[5] = published_before_drain;
    }
    free(p.published);
    free(need);
    return rc;
}
