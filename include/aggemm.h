/*
 * aggemm.h -- C ABI of libaggemm: chunked AllGather fused with a bf16 GEMM, and TGATHER, on one
 * AMD Instinct MI355X (gfx950).
 *
 * Pages this library implements:
 *   [AGMM]  "Triton第四课：基于对称内存融合 AllGather 与 MatMul，提速1.56倍" (the fused
 *           AllGather + MatMul pipeline: comm blocks, progress flags, rotated tile order)
 *   [TGATH] "CANN PTO-ISA TGATHER 指令深度解析：跨 Rank 行拼接 Gather 的实现原理与开发指南"
 *           (the root-side row-concatenating gather with 2D sliding tiles)
 *
 * On one GPU the N "ranks" are N separate device buffers ("shards"); the AllGather is an
 * HBM-to-HBM copy of their rows into one aggregate buffer.
 *
 * Conventions for every entry point:
 *   - All tensors are caller-owned DEVICE memory on the current HIP device, row-major and
 *     contiguous.  `shards` itself is a HOST array of N device pointers, read during the call only.
 *   - bf16 is IEEE binary32 truncated to its upper 16 bits (the layout of torch.bfloat16).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are enqueued on it and return
 *     before the GPU work finishes; results are valid once the stream has reached that point.
 *   - Arguments are validated before anything is enqueued; on a negative return nothing was
 *     enqueued.  Outputs must not overlap inputs.
 *   - The library keeps a per-device workspace (aggregate A buffer, progress flags, counters, a
 *     status word) that grows on demand and is released by ag_finalize().  Calls that use it are
 *     ordered with one another through an event, so at most one AG-GEMM uses it at a time.
 */
#ifndef AGGEMM_H
#define AGGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define AG_OK            0
#define AG_EINVAL       -1   /* an argument was rejected; nothing was enqueued */
#define AG_ENOMEM       -2   /* the workspace could not grow */
#define AG_EHIP         -3   /* the HIP runtime reported an error (message: ag_last_error()) */
#define AG_ETIMEOUT     -4   /* (ag_check) a tile gave up waiting on a chunk flag */
#define AG_EUNSUPPORTED -5   /* shape outside the library's limits (see each entry point) */

/* Schedules of ag_gemm_ex. */
#define AG_MODE_FUSED      0  /* chunked copy and GEMM overlapped, per-chunk flags */
#define AG_MODE_UNFUSED    1  /* full gather (tgather kernel), then the GEMM: the serial schedule */
#define AG_MODE_GEMM_ONLY  2  /* the fused GEMM with every flag already raised and no copy */
#define AG_MODE_PLAIN_GEMM 3  /* the GEMM of the serial schedule alone, on a_out (no flags at all) */

/* Who copies the chunks in AG_MODE_FUSED ([AGMM] 融合后的流水线 has the copy beside the MatMul). */
#define AG_PRODUCER_SIDE_STREAM  0  /* a copy kernel on a second stream (its first-wave part runs
                                       before the GEMM), waiting tiles help (default) */
#define AG_PRODUCER_IN_KERNEL    1  /* the GEMM's workgroups: tiles that would wait copy at once, and
                                       every running wave copies a little per K step */
#define AG_PRODUCER_COPY_ENGINE  2  /* per chunk, a device-to-device copy that uses no compute units
                                       (hipMemcpyDeviceToDeviceNoCU) then a stream write of the flag
                                       ([AGMM] 数据搬运与细粒度同步: copy, then stream_write_value32);
                                       the GEMM only waits */

/* Element type of C (ag_options.out_dtype). */
#define AG_OUT_BF16      0    /* bf16, round to nearest even (default) */
#define AG_OUT_FP8_E4M3  1    /* FP8 E4M3 "fn" (OCP; torch.float8_e4m3fn), one byte per element:
                                 C = e4m3fn(acc * out_scale), the fp32 sum times the fp32 scale,
                                 rounded to nearest even; NaN where that lands beyond +-448
                                 ([AGMM] MatMul 按需等待: the MatMul's FP8_OUTPUT variant) */

/* Element type of the shards, B and the gathered A (ag_options.in_dtype). */
#define AG_IN_BF16       0    /* bf16 (default) */
#define AG_IN_FP8_E4M3   1    /* FP8 E4M3 "fn" codes, one byte per element (K % 16 == 0).  Every
                                 product of two such values is exact in fp32 and the sums run in
                                 fp32, as for bf16; per-tensor scales of A and B fold into
                                 out_scale.  An extension of [AGMM]'s FP8 variant (there only the
                                 output is FP8) onto gfx950's FP8 matrix instructions. */

typedef struct ag_options {
    int32_t mode;          /* AG_MODE_* */
    int32_t local_rank;    /* shard whose rows the rotated tile walk starts at, 0..N-1 */
    void *a_out;           /* NULL, or an (M, K) device buffer (of the input element type) that
                              receives the gathered A.
                              Required for AG_MODE_GEMM_ONLY and AG_MODE_PLAIN_GEMM, where it must
                              already hold it. */
    int64_t timeout_us;    /* give-up time of one flag wait, microseconds (<= 0: 10 s) */
    int32_t reverse_order; /* test aid: the copy claims chunks in reverse ready order */
    int32_t skip_producer; /* test aid (AG_MODE_FUSED): copy nothing and leave the flags stale, so
                              every non-local tile's wait ends through timeout_us; ag_check then
                              reports AG_ETIMEOUT.  C is meaningless after such a call; later calls
                              are unaffected (every call starts from fresh counters, and a give-up
                              only short-cuts the waits of the call that gave up). */
    int32_t producer;      /* AG_PRODUCER_* (AG_MODE_FUSED only) */
    void *gemm_events[2];  /* measurement aid: NULL, or two hipEvent_t the call records on the GEMM
                              kernel's stream right before and right after launching it */
    int32_t out_dtype;     /* AG_OUT_*; with AG_OUT_FP8_E4M3, C is an (M, Nc) byte array */
    float out_scale;       /* AG_OUT_FP8_E4M3: factor applied to the fp32 sums before the
                              conversion; 0 means 1 (must be finite) */
    void *wait_stats;      /* measurement aid (AG_MODE_FUSED): NULL, or a device array of 4 uint64 the
                              GEMM adds to: 100 MHz clock ticks its workgroups spent waiting on chunk
                              flags (summed over workgroups), waits, pieces copied by waiting
                              workgroups, tiles that skipped their wait (flags read in advance) */
    int32_t in_dtype;      /* AG_IN_*; with AG_IN_FP8_E4M3 the shards, B and a_out hold one byte per
                              element, and C = out_scale * (A B^T) in bf16 or (out_dtype) FP8 --
                              out_scale then applies to bf16 output too (0 means 1) */
} ag_options;

/*
 * C = gather(shards) * B^T with the fused schedule ([AGMM] 融合后的流水线, MatMul 按需等待).
 *   shards[r]        (H, K) bf16, H = M / N; shard r holds rows [r*H, (r+1)*H) of A
 *   N                number of shards, 1..64
 *   M, K             rows of the gathered A and the reduction length; M % N == 0, K % 8 == 0,
 *                    K <= 2^21
 *   B                (Nc, K) bf16 (the weight stored row-major by output column)
 *   C                (M, Nc) bf16 output, written with round-to-nearest-even from fp32 sums
 *   comm_block_rows  rows per comm block (chunk) inside each shard, >= 1; the last chunk of a
 *                    shard may be shorter.  Chunk r*S + s (S = ceil(H / comm_block_rows)) has
 *                    its own uint32 progress flag ([AGMM] 数据搬运与细粒度同步).
 * Device pointers must be 16-byte aligned.  M == 0 or Nc == 0 enqueues nothing; K == 0 writes
 * zeros (shards and B may then be NULL).  The local shard is shard 0 (ag_gemm_ex chooses
 * another).
 */
int ag_gemm(const void *const *shards, int32_t N, int64_t M, int64_t K, const void *B,
            int64_t Nc, void *C, int64_t comm_block_rows, void *stream);

/* Same arguments; the serial schedule ([AGMM] 为什么要融合 AllGather 与 MatMul): the whole
 * gather into the workspace first, then the GEMM.  Bitwise equal to ag_gemm's C. */
int ag_gemm_unfused(const void *const *shards, int32_t N, int64_t M, int64_t K, const void *B,
                    int64_t Nc, void *C, int64_t comm_block_rows, void *stream);

/* ag_gemm with options (NULL = defaults: fused, side-stream producer, local_rank 0, internal buffer,
 * 10 s). */
int ag_gemm_ex(const void *const *shards, int32_t N, int64_t M, int64_t K, const void *B,
               int64_t Nc, void *C, int64_t comm_block_rows, void *stream,
               const ag_options *opt);

/*
 * TGATHER ([TGATH] 二 数学语义): dst[d0,d1,d2, r*H + i, j] = shards[r][d0,d1,d2, i, j].
 *   shards[r]            (D0, D1, D2, H, W) tensor of elem_size-byte elements, r < N (1..64)
 *   dst                  (D0, D1, D2, N*H, W) tensor
 *   valid_rows/cols      extent of the staging tile that slides over each rank's (H, W) plane
 *                        ([TGATH] 6.1, 7.4): >= 1; the last row / column tile is ragged when they
 *                        do not divide H / W; values above H / W mean one tile spans the plane.
 *                        The result does not depend on them (a copy is exact); the work split does.
 *   elem_size            1, 2, 4 or 8 bytes.
 * Any extent of 0 enqueues nothing ([TGATH] 7.4).  16-byte aligned pointers with
 * W * elem_size % 16 == 0 take the 16-byte vector path; anything else a slower element path.
 */
int tgather(const void *const *shards, int32_t N, void *dst, int64_t D0, int64_t D1, int64_t D2,
            int64_t H, int64_t W, int64_t valid_rows, int64_t valid_cols, int32_t elem_size,
            void *stream);

/* tgather into a taller dst of shape (D0, D1, D2, dst_rows, W), dst_rows >= N*H; rows at or
 * beyond N*H of every plane are left untouched ([TGATH] 7.2 内存约束).  root, 0..N-1, is the rank
 * whose buffer dst is ([TGATH] RunGatherWithRoot): on one GPU every shard is already addressable
 * from it, so it selects nothing and is only validated. */
int tgather_ex(const void *const *shards, int32_t N, void *dst, int64_t D0, int64_t D1,
               int64_t D2, int64_t H, int64_t W, int64_t dst_rows, int64_t valid_rows,
               int64_t valid_cols, int32_t elem_size, int32_t root, void *stream);

/*
 * GEMM + ReduceScatter, one rank's share ([AGMM] 从集合通信理解数据流: ReduceScatter leaves rank r
 * with the reduction, over all ranks, of block r; the mirror of the AllGather feeding the MatMul).
 * In the row-parallel form every rank multiplies its K slice, P = A * B^T, and the ranks reduce P
 * over row blocks of H = M / N rows.  On one GPU the other ranks' partials for this rank's rows
 * arrive as input buffers.
 *   A                 (M, K) bf16: this rank's K slice of the activations
 *   B                 (Nc, K) bf16: this rank's K slice of the weight
 *   recv              host array of N device pointers; recv[j], j != local_rank, is rank j's
 *                     (H, Nc) bf16 partial for rows [local_rank*H, (local_rank+1)*H);
 *                     recv[local_rank] is ignored (may be NULL)
 *   P                 (M, Nc) bf16 output: this rank's partial product, bf16 (nearest even) of the
 *                     fp32 sums -- every row block, the others being what the peers would receive
 *   out               (H, Nc) bf16 output: bf16 (nearest even) of the fp32 sum over j = 0..N-1, in
 *                     that order, of the partials (this rank's own rows of P in slot local_rank)
 *   mode              AG_RS_FUSED: a reducing kernel on a second stream starts on each GEMM tile
 *                     row of the block as soon as that row's tiles are written; AG_RS_UNFUSED: the
 *                     GEMM, then the reduction.  Both give bitwise the same P and out.
 * M % N == 0, K % 8 == 0, Nc % 8 == 0; 16-byte aligned pointers.  K > 2^21 or Nc > 2^26 returns
 * AG_EUNSUPPORTED.  A wait that gave up (10 s) is reported by ag_check.
 */
#define AG_RS_FUSED    0
#define AG_RS_UNFUSED  1
int gemm_rs(const void *A, const void *B, int32_t N, int32_t local_rank, int64_t M, int64_t Nc,
            int64_t K, const void *const *recv, void *P, void *out, int32_t mode, void *stream);

/* For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The same product as ag_gemm (C, and the gathered A in
 * a_out), by the fused schedule with the in-kernel producer on `stream` alone.  It allocates
 * nothing and creates no stream or event: its control words (one progress flag and one piece
 * count per chunk, two piece counters, a status block) live in a fixed array inside the library,
 * one per GPU, held until the process ends.
 *   a_out        (M, K) bf16 device buffer that receives the gathered A; required when K > 0
 *   local_rank   as in ag_options, 0..N-1
 *   other arguments as for ag_gemm.
 * Returns AG_EUNSUPPORTED when N * ceil((M/N) / comm_block_rows) > AG_NOALLOC_MAX_CHUNKS.
 * Every call on one GPU uses that GPU's one array: calls that overlap on one GPU (on two streams,
 * or from two host threads without ordering) race, and the caller must order them.  A flag wait
 * that gave up is reported by ag_check, as for the other entry points. */
#define AG_NOALLOC_MAX_CHUNKS 32768
int ag_gemm_noalloc(const void *const *shards, int32_t N, int64_t M, int64_t K, const void *B,
                    int64_t Nc, void *C, int64_t comm_block_rows, void *a_out, int32_t local_rank,
                    void *stream);

/* Waits for `stream`, then reads and clears the current device's status words (the workspace's,
 * then ag_gemm_noalloc's).  Returns AG_OK, or AG_ETIMEOUT with info = {code, chunk, tile, epoch}
 * for the first flag wait that gave up since the last ag_check (epoch: the failing call's flag
 * value). */
int ag_check(void *stream, int64_t info[4]);

/* Static text for a return code. */
const char *ag_status_str(int status);

/* Text of the last HIP error seen by the library on this thread's calls ("" if none). */
const char *ag_last_error(void);

/* Waits for all devices the library used and frees every workspace.  Safe to call repeatedly. */
void ag_finalize(void);

#ifdef __cplusplus
}
#endif
#endif /* AGGEMM_H */
