/*
 * oracle.h -- CPU oracle for the chunked AllGather + bf16 GEMM path and for TGATHER.
 *
 * TEST INFRASTRUCTURE ONLY.  This code is the slow, obviously-correct statement of what the
 * GPU library must compute.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load or call it; the product library never does, and the two share no code.
 *
 * Sources (the two pages this build follows):
 *   [AGMM]  "Triton第四课：基于对称内存融合 AllGather 与 MatMul，提速1.56倍"
 *   [TGATH] "CANN PTO-ISA TGATHER 指令深度解析：跨 Rank 行拼接 Gather 的实现原理与开发指南"
 *
 * Data conventions used throughout:
 *   - bf16 values travel as uint16_t bit patterns (the upper half of an IEEE fp32).
 *   - A "shard" r is a row-major (H, K) bf16 matrix; the gathered A is (M = N*H, K).
 *   - B is row-major (Nc, K) bf16; C = A * B^T is (M, Nc).
 */
#ifndef AG_ORACLE_H
#define AG_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* bf16 bit pattern -> fp32 (exact). */
float oracle_bf16_to_f32(uint16_t h);

/* fp32 -> bf16 bit pattern, round to nearest, ties to even; NaN stays a quiet NaN. */
uint16_t oracle_f32_to_bf16_rne(float f);

/* fp32 -> bf16 (round to nearest even) over n values. */
void oracle_f32_to_bf16_array(const float *x, int64_t n, uint16_t *out);

/*
 * ReduceScatter of one rank's block, [AGMM] 从集合通信理解数据流: every rank keeps the reduction,
 * over all ranks, of its own block.  parts[j] points at rank j's (H, Nc) bf16 contribution to this
 * block; out[i, n] = bf16_rne( f32(parts[0][i, n]) + f32(parts[1][i, n]) + ... ), summed in fp32 in
 * ascending j.
 */
void oracle_reduce_block(const uint16_t *const *parts, int nparts, int64_t H, int64_t Nc, uint16_t *out);

/*
 * FP8 output of the fused kernel ([AGMM] MatMul 按需等待: the MatMul is launched with FP8_OUTPUT
 * set when C's dtype is torch.float8_e4m3fn).  The conversion is that dtype's: the OCP FP8 E4M3
 * "fn" format -- 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
 * infinities, the single NaN pattern S.1111.111, largest finite 448 -- with round to nearest,
 * ties to even, onto the finite values; a value whose rounding lands beyond 448 (|x| > 464, or
 * infinite) becomes NaN, as does a NaN.  NaN results are 0x7F with the input's sign.
 */
uint8_t oracle_f32_to_e4m3fn(float x);
/* The value an E4M3 "fn" code stands for (NaN for S.1111.111). */
double oracle_e4m3fn_value(uint8_t code);
/*
 * FP8 inputs (an extension of the FP8 variant above onto the inputs): every finite E4M3 "fn" value
 * is exactly a bf16 value, so A and B in E4M3 are multiplied as the bf16 GEMM does, on the bf16
 * images of their codes: exact products, fp32 sums in ascending k.  This gives those images
 * (NaN code -> bf16 NaN); returns -1 if a finite value were not exactly representable.
 */
int oracle_e4m3fn_to_bf16(const uint8_t *codes, int64_t n, uint16_t *out);

/*
 * TGATHER closed form, [TGATH] §二 数学语义:
 *   dst[d0,d1,d2, r*H + i, j] = src_r[d0,d1,d2, i, j]  for r < nranks, i < H, j < W.
 * src[r] points at rank r's (D0,D1,D2,H,W) tensor, dst at a (D0,D1,D2,dst_rows,W) tensor, all
 * row-major with elem_size-byte elements.  Rows r*H+i >= nranks*H of a taller dst are not
 * touched ([TGATH] §7.2); an empty shape moves nothing ([TGATH] §7.4).
 * Returns 0, or -1 for invalid arguments (nranks <= 0, elem_size <= 0, dst_rows < nranks*H,
 * negative extents).
 */
int oracle_tgather(const void *const *src, int nranks, void *dst,
                   int64_t D0, int64_t D1, int64_t D2, int64_t H, int64_t W,
                   int64_t dst_rows, int elem_size);

/*
 * C[m][n] = sum over k = 0..K-1, in ascending k, of float(A[m][k]) * float(B[n][k]),
 * accumulated in fp32 with a separate multiply and add.  A is (M,K), B is (Nc,K), C is (M,Nc)
 * fp32.  [AGMM] §对称内存如何打通GPU间访问 (test tensors: a is (m,k), b is stored (n,k)).
 */
void oracle_gemm_f32(const uint16_t *A, const uint16_t *B, int64_t M, int64_t Nc, int64_t K,
                     float *C);

/*
 * The same element as oracle_gemm_f32 would produce for C = gather(shards) * B^T, evaluated
 * only at the given (ms[i], ns[i]) positions.  Row m of the gathered A is row m % H of shard
 * m / H with H = M / nshards.  Returns 0, or -1 if a position is out of range.
 */
int oracle_ag_gemm_at(const uint16_t *const *shards, int nshards, int64_t M, int64_t K,
                      const uint16_t *B, int64_t Nc, const int64_t *ms, const int64_t *ns,
                      int64_t count, float *out);

/*
 * Full "gather, then GEMM" ([AGMM] §为什么要融合: the serial schedule the fusion replaces):
 * A_out (M,K) receives the gathered rows, C (M,Nc) the fp32 product.
 */
int oracle_ag_gemm(const uint16_t *const *shards, int nshards, int64_t M, int64_t K,
                   const uint16_t *B, int64_t Nc, uint16_t *A_out, float *C);

/*
 * Bit-identical to oracle_gemm_f32 (the same ascending-k fp32 recursive sum per element, no FMA),
 * in a blocked loop order fast enough for the full-size workloads.  Row m of A is a_rows[m]
 * (K bf16 values); B is (Nc,K).  Pinned bitwise against oracle_gemm_f32 in the tests.
 */
void oracle_gemm_f32_fast(const uint16_t *const *a_rows, const uint16_t *B, int64_t M, int64_t Nc,
                          int64_t K, float *C);

/* C = gather(shards) * B^T through oracle_gemm_f32_fast.  Returns 0 or -1. */
int oracle_ag_gemm_fast(const uint16_t *const *shards, int nshards, int64_t M, int64_t K,
                        const uint16_t *B, int64_t Nc, float *C);

/* Comm-block ("chunk") map, [AGMM] §融合后的流水线 and §数据搬运与细粒度同步:
 * shard r is split along M into S = ceil(H/cb) blocks of cb rows (the last may be shorter);
 * block s of shard r has id r*S + s.  Returns the id of the chunk holding gathered row `row`. */
int64_t oracle_chunk_of_row(int64_t row, int64_t H, int64_t cb);

/* Writes the ids of all chunks that overlap gathered rows [m0, m1) into out (ascending) and
 * returns their count. */
int64_t oracle_chunks_overlapping(int64_t m0, int64_t m1, int64_t H, int64_t cb, int64_t *out,
                                  int64_t cap);

/* Grouped tile order: tile id t -> (pid_m, pid_n) with group_m tile rows per group. */
void oracle_grouped_tile(int64_t t, int64_t num_pid_m, int64_t num_pid_n, int64_t group_m,
                         int64_t *pid_m, int64_t *pid_n);

/*
 * Simulation of the fused schedule on the CPU, [AGMM] §融合后的流水线, §MatMul 按需等待:
 *  - a producer publishes chunks one at a time, in ready order: all chunks of shard
 *    local_rank+1, then local_rank+2, ... (mod N), and the local shard's chunks last;
 *    publishing copies the chunk's rows into A_prime and raises its flag;
 *  - tiles are visited in grouped order with pid_m rotated to start at the local shard:
 *    pid_m' = (pid_m + floor(local_rank*H / BM)) mod num_pid_m;
 *  - a tile whose rows all lie in the local shard reads the shard directly;
 *  - any other tile first waits for every chunk overlapping its rows (here: advances the
 *    producer until they are published) and then reads A_prime.
 * A_prime starts as bf16 NaN everywhere, so a read before publication poisons C.  Every row
 * read from A_prime is also checked against the flags.
 * Outputs: C (M,Nc) fp32, A_prime (M,K); stats (6 entries): [0] tiles that waited on at least
 * one chunk not yet published, [1] flag checks, [2] local tiles, [3] pid_m of the first tile
 * visited, [4] tiles visited before the first non-local one, [5] chunks the producer had
 * published when the last tile finished (before the final drain).
 * Returns 0, -1 for invalid arguments, -2 if a tile read a row of an unpublished chunk.
 */
int oracle_ag_gemm_pivoted(const uint16_t *const *shards, int nshards, int64_t M, int64_t K,
                           const uint16_t *B, int64_t Nc, int64_t cb, int64_t BM, int64_t BN,
                           int64_t group_m, int local_rank, uint16_t *A_prime, float *C,
                           int64_t *stats);

/* Threads the OpenMP loops above use (1 in a build without OpenMP): what a timing of the oracle
 * reports as its core count. */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
