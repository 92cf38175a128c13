/*
 * oracle.c -- CPU oracle for the chunked AllGather + bf16 GEMM path and for TGATHER.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the benchmark's CPU
 * baseline, never by the GPU library.  It shares no code, header or table with the HIP path.
 *
 * Build: gcc -O3 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC oracle.c -o liboracle.so
 * (no -march: the library may run on another host; the blocked GEMM picks AVX2 at run time)
 * (-ffp-contract=off keeps every multiply and add a separately rounded fp32 operation).
 *
 * Every function states the passage of the two pages it follows; see oracle.h for the page
 * titles.  Parity pins for each function live in tests/test_oracle.py.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

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

void oracle_f32_to_bf16_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16_rne(x[i]);
}

/* [AGMM] 从集合通信理解数据流 (ReduceScatter: a rank keeps the reduction of its block). */
void oracle_reduce_block(const uint16_t *const *parts, int nparts, int64_t H, int64_t Nc, uint16_t *out)
{
    for (int64_t i = 0; i < H * Nc; ++i) {
        float s = 0.0f;
        for (int j = 0; j < nparts; ++j)
            s += oracle_bf16_to_f32(parts[j][i]);
        out[i] = oracle_f32_to_bf16_rne(s);
    }
}

/* E4M3 "fn" from the format's definition (see oracle.h).  Works in doubles: |x| divided by the
 * spacing of its binade is exact, so the rounding below is exact too. */
static double round_half_even(double v)      /* v >= 0 */
{
    double f = floor(v);
    double r = v - f;
    if (r > 0.5)
        return f + 1.0;
    if (r < 0.5)
        return f;
    return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

uint8_t oracle_f32_to_e4m3fn(float x)
{
    const uint8_t sign = signbit(x) ? 0x80u : 0u;
    if (isnan(x) || isinf(x))
        return (uint8_t)(sign | 0x7fu);
    const double a = fabs((double)x);
    const double min_normal = ldexp(1.0, -6);
    if (a < min_normal) {
        /* subnormal binade: steps of 2^-9; 8 steps is the smallest normal, code 0x08 */
        const double q = round_half_even(a / ldexp(1.0, -9));
        return (uint8_t)(sign | (uint8_t)q);
    }
    int e2;
    (void)frexp(a, &e2);                 /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                      /* a in [2^e, 2^(e+1)) */
    double q = round_half_even(a / ldexp(1.0, e - 3));   /* 8 .. 16 steps of 2^(e-3) */
    if (q == 16.0) {                     /* rounded up into the next binade */
        e += 1;
        q = 8.0;
    }
    const int field = e + 7;
    const int mant = (int)q - 8;
    if (field > 15 || (field == 15 && mant == 7))
        return (uint8_t)(sign | 0x7fu);  /* beyond 448 */
    return (uint8_t)(sign | (uint8_t)(field << 3) | (uint8_t)mant);
}

double oracle_e4m3fn_value(uint8_t code)
{
    const double s = (code & 0x80u) ? -1.0 : 1.0;
    const int field = (code >> 3) & 15, mant = code & 7;
    if (field == 15 && mant == 7)
        return NAN;
    if (field == 0)
        return s * ldexp((double)mant, -9);
    return s * ldexp(8.0 + mant, field - 10);
}

/* FP8 inputs: the bf16 bit pattern of an E4M3 "fn" code's value.  Every finite E4M3 value has a
 * 4-bit significand and an exponent in [-9, 8], so it is exactly a bf16 value (8-bit significand,
 * bf16's exponent range): the pattern is the top half of the value's float pattern, whose bottom
 * half is zero.  S.1111.111 becomes a bf16 NaN.  Returns -1 if a finite value were not exact. */
int oracle_e4m3fn_to_bf16(const uint8_t *codes, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        const float v = (float)oracle_e4m3fn_value(codes[i]);
        uint32_t u;
        memcpy(&u, &v, 4);
        if (!isnan(v) && (u & 0xFFFFu) != 0)
            return -1;
        out[i] = (uint16_t)(u >> 16);
    }
    return 0;
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

/*
 * The same C as oracle_gemm_f32, bit for bit, computed in a cache-friendly loop order so that
 * C for the full-size workloads (up to 10^12 multiply-adds) can be checked element by element.
 * Only the loop nest differs: every C[m][n] still starts at 0.0f and adds the products
 * float(A[m][k]) * float(B[n][k]) one at a time in ascending k, each product and each sum
 * rounded to fp32 on its own (no FMA: -ffp-contract=off).  The running sum of an element is
 * kept in a register across a block of k and in memory between blocks; storing an fp32 value and
 * loading it back is exact, so this is the recursive summation above with its order unchanged
 * (no partial sums, no reassociation).  The loops run over (m, n) blocks in parallel.
 */
enum { FAST_MB = 4, FAST_NB = 16, FAST_KC = 256, FAST_NP = 256, FAST_RB = 64 };

/* acc[i][j] (i < FAST_MB, j < FAST_NB) continues its ascending-k sums over k in [k0, k0 + nk).
 * a[i] points at row i of A (bf16 bits), bt at Bt[k0][j0] (row stride ldb floats). */
typedef float fast_v8 __attribute__((vector_size(32)));   /* 8 independent fp32 lanes */

#define FAST_MICRO_BODY                                                                  \
    fast_v8 r[FAST_MB][2];                                                               \
    for (int i = 0; i < FAST_MB; ++i) {                                                  \
        memcpy(&r[i][0], &acc[i][0], sizeof(fast_v8));                                   \
        memcpy(&r[i][1], &acc[i][8], sizeof(fast_v8));                                   \
    }                                                                                    \
    for (int64_t kk = 0; kk < nk; ++kk) {                                                \
        fast_v8 b0, b1;                                                                  \
        memcpy(&b0, bt + kk * ldb, sizeof b0);                                           \
        memcpy(&b1, bt + kk * ldb + 8, sizeof b1);                                       \
        for (int i = 0; i < FAST_MB; ++i) {                                              \
            const float av = oracle_bf16_to_f32(a[i][k0 + kk]);                          \
            const fast_v8 p0 = b0 * av, p1 = b1 * av;      /* products, one rounding */  \
            r[i][0] = r[i][0] + p0;                        /* then the sums */           \
            r[i][1] = r[i][1] + p1;                                                      \
        }                                                                                \
    }                                                                                    \
    for (int i = 0; i < FAST_MB; ++i) {                                                  \
        memcpy(&acc[i][0], &r[i][0], sizeof(fast_v8));                                   \
        memcpy(&acc[i][8], &r[i][1], sizeof(fast_v8));                                   \
    }

/* acc[i][j] (i < FAST_MB, j < FAST_NB = 16) continues its ascending-k sums over k in
 * [k0, k0 + nk).  a[i] points at row i of A (bf16 bits), bt at Bt[k0][j0] (row stride ldb
 * floats).  Each vector lane is one element's own sum, so lanes never mix. */
__attribute__((target("avx2"))) static void fast_micro_avx2(float acc[FAST_MB][FAST_NB],
    const uint16_t *const a[FAST_MB], const float *bt, int64_t ldb, int64_t k0, int64_t nk)
{
    FAST_MICRO_BODY
}

static void fast_micro_base(float acc[FAST_MB][FAST_NB], const uint16_t *const a[FAST_MB],
                            const float *bt, int64_t ldb, int64_t k0, int64_t nk)
{
    FAST_MICRO_BODY
}

void oracle_gemm_f32_fast(const uint16_t *const *a_rows, const uint16_t *B, int64_t M, int64_t Nc,
                          int64_t K, float *C)
{
    /* Bt[k][n] = float(B[n][k]): the k-th row of Bt holds every column's k-th weight */
    float *Bt = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1) * (size_t)(Nc > 0 ? Nc : 1));
    if (!Bt)
        abort();
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < Nc; ++n)
            Bt[k * Nc + n] = oracle_bf16_to_f32(B[n * K + k]);
    const int use_avx2 = __builtin_cpu_supports("avx2");
    const int64_t n_rb = (M + FAST_RB - 1) / FAST_RB, n_np = (Nc + FAST_NP - 1) / FAST_NP;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t blk = 0; blk < n_rb * n_np; ++blk) {
        const int64_t m0 = (blk / n_np) * FAST_RB, n0 = (blk % n_np) * FAST_NP;
        const int64_t m1 = m0 + FAST_RB < M ? m0 + FAST_RB : M;
        const int64_t n1 = n0 + FAST_NP < Nc ? n0 + FAST_NP : Nc;
        for (int64_t m = m0; m < m1; ++m)
            for (int64_t n = n0; n < n1; ++n)
                C[m * Nc + n] = 0.0f;
        for (int64_t k0 = 0; k0 < K; k0 += FAST_KC) {              /* ascending k blocks */
            const int64_t k1 = k0 + FAST_KC < K ? k0 + FAST_KC : K;
            for (int64_t mi = m0; mi < m1; mi += FAST_MB)
                for (int64_t nj = n0; nj < n1; nj += FAST_NB) {
                    const int64_t rows = m1 - mi < FAST_MB ? m1 - mi : FAST_MB;
                    const int64_t cols = n1 - nj < FAST_NB ? n1 - nj : FAST_NB;
                    float acc[FAST_MB][FAST_NB];
                    float pad[FAST_NB];
                    const uint16_t *a[FAST_MB];
                    for (int i = 0; i < FAST_MB; ++i) {
                        a[i] = a_rows[mi + (i < rows ? i : 0)];   /* short tile: repeat row 0 */
                        for (int j = 0; j < FAST_NB; ++j)
                            acc[i][j] = (i < rows && j < cols) ? C[(mi + i) * Nc + nj + j] : 0.0f;
                    }
                    if (cols < FAST_NB) {
                        /* ragged column edge: one k at a time on a zero-padded copy of the row */
                        for (int64_t k = k0; k < k1; ++k) {
                            for (int j = 0; j < FAST_NB; ++j)
                                pad[j] = j < cols ? Bt[k * Nc + nj + j] : 0.0f;
                            if (use_avx2)
                                fast_micro_avx2(acc, a, pad, FAST_NB, k, 1);
                            else
                                fast_micro_base(acc, a, pad, FAST_NB, k, 1);
                        }
                    } else if (use_avx2) {
                        fast_micro_avx2(acc, a, Bt + k0 * Nc + nj, Nc, k0, k1 - k0);
                    } else {
                        fast_micro_base(acc, a, Bt + k0 * Nc + nj, Nc, k0, k1 - k0);
                    }
                    for (int i = 0; i < rows; ++i)
                        for (int j = 0; j < cols; ++j)
                            C[(mi + i) * Nc + nj + j] = acc[i][j];
                }
        }
    }
    free(Bt);
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

/* oracle_ag_gemm's C through oracle_gemm_f32_fast (the gathered A is never materialised: row m
 * is read from its shard). */
int oracle_ag_gemm_fast(const uint16_t *const *shards, int nshards, int64_t M, int64_t K,
                        const uint16_t *B, int64_t Nc, float *C)
{
    if (nshards <= 0 || M % nshards != 0 || K < 0 || Nc < 0)
        return -1;
    const int64_t H = M / nshards;
    const uint16_t **rows = (const uint16_t **)malloc(sizeof(uint16_t *) * (size_t)(M > 0 ? M : 1));
    if (!rows)
        return -1;
    for (int64_t m = 0; m < M; ++m)
        rows[m] = gathered_row(shards, H, K, m);
    oracle_gemm_f32_fast(rows, B, M, Nc, K, C);
    free(rows);
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

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
