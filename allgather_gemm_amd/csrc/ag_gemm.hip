// ag_gemm.hip -- persistent bf16 MFMA GEMM (fp32 accumulate) for C = A * B^T on gfx950, with
// the chunked-AllGather consumer and copy logic of the fused schedule.
//
// What it computes follows the fused AllGather+MatMul article ("Triton第四课：基于对称内存融合
// AllGather 与 MatMul，提速1.56倍"):
//  * section 融合后的流水线 / MatMul 按需等待: M is split into comm blocks ("chunks"); output tiles
//    are visited with pid_m rotated to the local shard; a tile wholly inside the local shard reads
//    the shard, every other tile first waits for the flags of the chunks its rows overlap and then
//    reads the aggregate A buffer;
//  * section 数据搬运与细粒度同步: a chunk's flag is raised only after its rows have landed;
//  * section wait_signal 的实现与语义: one wave polls, then a workgroup barrier releases the block.
// The article's copy runs beside the MatMul on its own engine.  Here the copy is done by the GEMM's
// own workgroups, in pieces (contiguous byte ranges, see ag_protocol.hpp) handed out in ready order
// from counters in device memory:
//  * a workgroup whose tile finds a chunk unpublished copies pieces at full speed until the chunk is
//    ready (the pipeline fill at the start is done this way, from a counter only waiters use);
//  * every running wave also copies one piece of its own in the background, 1 KiB per K step: the
//    store of the previous step's slice and the load of the next slice go out right after the step's
//    barrier, next to the tile loads, and the piece is published once its stores have drained.
// A wave finishes its piece before its workgroup can wait on anything, and waiters only take pieces
// they copy at once, so every handed-out piece is published in bounded time: no wait can deadlock.
// Before a workgroup exits it copies whatever no one has taken yet (the gathered output needs
// every chunk, also those no tile waits for).
// Other producers (a copy kernel on a second stream, the copy engines) leave the counters alone and
// only raise the flags; the GEMM then just waits.
//
// Tiling (gfx950): 256x256 output tile per 256-thread workgroup (4 waves, 2x2, 128x128 each),
// K step 64, v_mfma_f32_32x32x16_bf16, A/B tiles staged in LDS by buffer_load ... lds (16 B per
// lane, no VGPR round trip), double-buffered (2 x 64 KiB).  LDS rows are 128 B (64 bf16) and
// their 16-byte chunks are XOR-swizzled so the ds_read_b128 fragment loads are conflict-free
// (every bank serves at most four dwords of a wave's read).  FP8 inputs keep the same 128-byte
// rows (K step 128) and use v_mfma_f32_32x32x64_f8f6f4: a lane's fragment is two 16-byte chunks.
#include "ag_device.hpp"
#include "ag_internal.hpp"
#include "ag_protocol.hpp"

#include <algorithm>

namespace ag {
namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int BM = 256, BN = 256, BK = 64;     // BK: bf16 elements per K step (128 bytes)
constexpr int NT = 256;                        // threads per workgroup
constexpr int SLOTS = BM * BK * 2 / 16;        // 16-byte slots per operand tile (2048)
constexpr int TILE_BYTES = SLOTS * 16;         // 32 KiB per operand tile
constexpr int GROUP_M = 8;                     // tile rows per group of the grouped order
constexpr int64_t PIECE_BYTES = 16 * 1024;     // bytes per copy piece
constexpr int PIECE_UNITS = (int)(PIECE_BYTES / 16 / NT);   // 16-byte units per lane per piece
static_assert(PIECE_UNITS * 16 * NT == PIECE_BYTES, "a piece is a whole number of 16-byte units per lane");
constexpr int WAIT_BATCH = 4;                  // pieces a waiting workgroup takes at a time
constexpr int SLICE = 1024;                    // bytes a wave copies per K step in the background

static_assert(BM == BN, "A and B tiles share one LDS layout");
static_assert(PIECE_BYTES % SLICE == 0, "a piece is a whole number of slices");

// Swizzle of the 16-byte chunk index inside a 128-byte LDS row: depends on row bits 0..3 so that
// any 8 (and any 16) consecutive rows reading the same logical chunk hit distinct banks.
__device__ __forceinline__ uint32_t swz(uint32_t row) { return (row & 7u) ^ ((row >> 3) & 1u); }

struct TileCoord {
    int64_t m0, n0;
    int64_t tile;
};

__host__ __device__ __forceinline__ TileCoord tile_of(int64_t t, int num_pid_m, int num_pid_n, int pivot)
{
    int64_t pid_m, pid_n;
    pm_tile_of(t, num_pid_m, num_pid_n, pivot, GROUP_M, pid_m, pid_n);
    TileCoord c;
    c.m0 = pid_m * BM;
    c.n0 = pid_n * BN;
    c.tile = t;
    return c;
}

struct KParams {
    GemmArgs a;
    int num_pid_m, num_pid_n, pivot;
    PieceMap pm;
    int64_t npieces;     // pieces of this call (0: nothing is copied by this launch's claims)
    int64_t fill_end;    // pieces [0, fill_end) come from ctl[0], only waiting workgroups take them
    int trickle;         // running waves copy pieces in the background
};

// The copy protocol's parameters (piece map, counters, flags) are read from the kernel argument
// segment where they are used, through a pointer the compiler cannot see through, instead of being
// held in scalar registers for the whole kernel: held, they stay live across the K loop, spill,
// and their reloads land in every K step.  KParams is each kernel's first argument (offset 0).
__device__ __forceinline__ const KParams& kparams()
{
    typedef const __attribute__((address_space(4))) KParams* Ptr;
    Ptr k = (Ptr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(k));
    return *(const KParams*)k;
}

// --------------------------------------------------------------------------------- copy pieces
// The single-writer steps below run on all 64 lanes of a wave (a wave-uniform branch), never on
// one lane: a one-lane branch inside a loop that also holds barriers lets the compiler's control
// flow structurizer peel that lane out of the loop while the other lanes keep iterating.  Only the
// atomics themselves are issued by lane 0 (ag_device.hpp), and their results are broadcast, so
// every decision stays wave-uniform.
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Copied bytes are stored write-through at system scope ("sc0 sc1"): when this wave's store count
// drains they have reached memory, and no L2 holds them dirty.  That is what lets a piece be
// published by a relaxed count after the drain -- no L2 write-back fence, which on this multi-XCD
// part writes back the whole L2 and would sit in the GEMM's K loop.
constexpr int kWriteThrough = 1 | 16;      // cache policy bits sc0 | sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void* base, int64_t bytes)
{
    return make_rsrc(base, (uint32_t)bytes);
}

__device__ __forceinline__ void store_wt(__amdgpu_buffer_rsrc_t r, uint32_t off, i32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kWriteThrough);
}

// Ready-order piece index -> piece (the stress mode hands pieces out back to front).
__device__ __forceinline__ PieceSpan piece_at(const KParams& p, int64_t q)
{
    return pm_piece(p.pm, p.a.reverse_order ? p.npieces - 1 - q : q);
}

// One wave: n more pieces of chunk c are complete -- their write-through stores have drained, so
// the bytes are in memory -- and the last of the chunk's pieces raises its flag.  The count is an
// atomic read-modify-write at the device's point of coherence: the wave whose count completes the
// chunk has seen every other piece's count, each made after that piece's bytes landed.
__device__ void publish(const KParams& p, int64_t c, uint32_t n)
{
    const GemmArgs& a = p.a;
    const uint32_t old = wave_fetch_add(&a.done[c], n);
    if (old + n == (uint32_t)p.pm.ppc)
        flag_publish(&a.flags[c], a.epoch);
}

// Publishes pieces [q0, q0 + n), grouping consecutive pieces of one chunk into one count.
__device__ void publish_range(const KParams& p, int64_t q0, int64_t n)
{
    int64_t q = q0;
    while (q < q0 + n) {
        const int64_t c = piece_at(p, q).chunk;
        int64_t e = q + 1;
        while (e < q0 + n && piece_at(p, e).chunk == c)
            ++e;
        publish(p, c, (uint32_t)(e - q));
        q = e;
    }
}

// One wave: takes up to `want` pieces from a counter that hands out [start, end); returns the first
// piece and sets *n (0 when the counter is spent).
__device__ __forceinline__ int64_t take(uint32_t* ctr, int64_t end, uint32_t want, int64_t* n)
{
    const uint32_t t = wave_fetch_add(ctr, want);
    const int64_t avail = end - (int64_t)t;
    *n = avail <= 0 ? 0 : (avail < (int64_t)want ? avail : (int64_t)want);
    return (int64_t)t;
}

// Copies pieces [q0, q0 + n) with the whole workgroup, then drains its stores and meets at a barrier
// (after it, one wave's release covers every byte).  A 16 KiB piece is four 16-byte units per lane,
// fewer than the unrolled loop takes, so each lane copies them one load and store at a time: a
// gentle copy.  Keeping every unit in flight copied faster, but no side-stream call got faster and
// in-kernel calls got slower (their waiting and draining workgroups then pressed harder on the
// memory system the running tiles use).
template <int U = 8>
__device__ void copy_pieces(const KParams& p, int64_t q0, int64_t n, int tid)
{
    for (int64_t q = q0; q < q0 + n; ++q) {
        const PieceSpan sp = piece_at(p, q);
        const i32x4* src = reinterpret_cast<const i32x4*>(static_cast<const char*>(p.a.shards[sp.shard]) + sp.src_off);
        const __amdgpu_buffer_rsrc_t dst =
            span_rsrc(static_cast<const char*>(p.a.A) + sp.dst_off, sp.bytes);
        const int64_t units = sp.bytes / 16;
        int64_t u = tid;
        for (; u + (U - 1) * NT < units; u += U * NT) {
            i32x4 v[U];
#pragma unroll
            for (int i = 0; i < U; ++i)
                v[i] = src[u + i * NT];
#pragma unroll
            for (int i = 0; i < U; ++i)
                store_wt(dst, (uint32_t)((u + i * NT) * 16), v[i]);
        }
        for (; u < units; u += NT)
            store_wt(dst, (uint32_t)(u * 16), src[u]);
    }
    wait_vmcnt0();
    __syncthreads();
}

constexpr int64_t kReady = -1, kIdle = -2, kFailed = -3;

// Wave 0 of a waiting workgroup: what to do next while chunk c is not ready -- kReady, kFailed, a
// batch of pieces to copy (returned as its first piece, count in *n), or kIdle (sleep, ask again).
// Gives up after spin_limit ticks of the 100 MHz clock; a failure is tagged with this call's epoch
// so only this call's other waits give up early.
__device__ int64_t decide_wait(const KParams& p, int64_t c, uint64_t t_start, int64_t tile, bool& exhausted,
                               int64_t* n)
{
    const GemmArgs& a = p.a;
    *n = 0;
    if (uniform_u32(flag_peek(&a.flags[c])) == a.epoch)
        return kReady;
    if (uniform_u32(flag_peek(&a.status[3])) == a.epoch)
        return kFailed;                                  // another workgroup of this call gave up
    if (!exhausted && p.npieces > 0) {
        int64_t q = take(a.ticket, p.fill_end, WAIT_BATCH, n);
        if (*n > 0)
            return q;
        q = take(a.ticket + 1, p.npieces, WAIT_BATCH, n);
        if (*n > 0)
            return q;
        exhausted = true;
    }
    if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t_start) > a.spin_limit) {
        report_failure(a.status, 1u, (uint32_t)c, (uint32_t)tile, a.epoch);
        return kFailed;
    }
    return kIdle;
}

// Waits until every chunk overlapping rows [m0, m1) is published, copying unclaimed pieces
// meanwhile; ends with an agent-scope acquire and a barrier.
//
// Loop shape: barrier / uniform read of the command / barrier / uniform branch / work / a
// wave-0 step that publishes and decides the next command.  Every branch is wave-uniform.  Once
// this workgroup has given up, `failed` stays set and later waits return at once, so a failed
// call ends within one timeout.
// The workgroup's flag-wait counters (measurement aid): kept in LDS by wave 0 -- in registers they
// would stay live across the K loop -- and added to the caller's counters once, when the workgroup
// ends.  Every lane of wave 0 stores the same value (no lane condition): a lane-divergent branch at
// the end of the tile's wait region keeps the compiler from proving the K loop's buffer resources
// uniform, and it then wraps every tile load in a loop over the lanes.
struct WaitStats {
    uint64_t ticks, waits, copied, skipped;
};

__device__ void wait_rows(const KParams& p, int64_t m0, int64_t m1, int64_t tile, int tid, bool wave0,
                          int64_t* s_cmd, bool& exhausted, bool& failed, WaitStats* ws)
{
    int64_t c_first, c_last;
    pm_chunks_of_rows(p.pm, m0, m1, c_first, c_last);
    const uint64_t t_wait = __builtin_amdgcn_s_memrealtime();
    uint64_t copied = 0;
    for (int64_t c = c_first; c <= c_last; ++c) {
        if (failed)
            break;
        const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
        if (wave0) {
            int64_t n;
            s_cmd[0] = decide_wait(p, c, t_start, tile, exhausted, &n);
            s_cmd[1] = n;
        }
        for (;;) {
            barrier_after_lds_write();
            const int64_t cmd = uniform_i64(s_cmd[0]);
            const int64_t cnt = uniform_i64(s_cmd[1]);
            __syncthreads();
            if (cmd == kReady)
                break;
            if (cmd == kFailed) {
                failed = true;
                break;
            }
            if (cmd >= 0) {
                copy_pieces(p, cmd, cnt, tid);
                copied += (uint64_t)cnt;
            } else {
                __builtin_amdgcn_s_sleep(4);
            }
            if (wave0) {
                if (cmd >= 0)
                    publish_range(p, cmd, cnt);
                int64_t n;
                s_cmd[0] = decide_wait(p, c, t_start, tile, exhausted, &n);
                s_cmd[1] = n;
            }
        }
    }
    // A cache line of the gathered buffer can hold bytes of two chunks only when rows are not whole
    // 128-byte lines; then an earlier read may have cached part of this chunk before it landed, and
    // the L2 is invalidated.  Otherwise no line of a chunk is cached before its flag rises.
    if (p.pm.row_bytes % 128 != 0)
        acquire_agent();
    __syncthreads();
    if (wave0) {
        ws->ticks += __builtin_amdgcn_s_memrealtime() - t_wait;
        ws->waits += 1;
        ws->copied += copied;
    }
}

// Wave 0: the flags of the chunks under gathered rows [m0, m1), one per lane (lane i: the i-th
// chunk), read in one batch -- a single round trip to the point of coherence -- while the current
// tile computes.  Returns the lane's flag; *n is the chunk count, or -1 if there are more chunks
// than lanes (that tile then waits the ordinary way).
__device__ __forceinline__ uint32_t peek_rows(const KParams& p, int64_t m0, int64_t m1, int lane, int* n)
{
    int64_t c0, c1;
    pm_chunks_of_rows(p.pm, m0, m1, c0, c1);
    const int64_t cnt = c1 - c0 + 1;
    *n = cnt > 64 ? -1 : (int)cnt;
    uint32_t v = 0;
    if (lane < *n)
        v = __hip_atomic_fetch_add(&p.a.flags[c0 + lane], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return v;
}

// ------------------------------------------------------------------------- background copy
// Per-wave state (wave-uniform): the piece being copied, how far its loads got, the slice loaded
// in the last step and not yet stored, and a piece whose last store went out in the last step.
struct Trickle {
    int32_t chunk;        // chunk of the piece being copied, -1 none
    int32_t bytes;        // its size
    int32_t off;          // next byte to load
    int32_t pend;         // byte offset of the slice held in `data`, -1 none
    int32_t publish;      // chunk of a piece to publish at the next step (its stores drained meanwhile)
    const char* src;
    __amdgpu_buffer_rsrc_t dst;
    i32x4 data;
    bool exhausted;
};

__device__ __forceinline__ void trickle_take(const KParams& p, Trickle& tr)
{
    int64_t n;
    const int64_t q = take(p.a.ticket + 1, p.npieces, 1, &n);
    if (n == 0) {
        tr.exhausted = true;
        return;
    }
    const PieceSpan sp = piece_at(p, q);
    tr.chunk = (int32_t)sp.chunk;
    tr.bytes = (int32_t)sp.bytes;
    tr.off = 0;
    tr.src = static_cast<const char*>(p.a.shards[sp.shard]) + sp.src_off;
    tr.dst = span_rsrc(static_cast<const char*>(p.a.A) + sp.dst_off, sp.bytes);
}

// One K step of the background copy; called by every lane of the wave right after the step's
// barrier, when this wave's loads and stores of the previous step have drained.  The protocol's
// parameters are fetched only on the rare steps that take or publish a piece.
__device__ void trickle_step(Trickle& tr, int lane)
{
    if (tr.publish >= 0) {
        publish(kparams(), tr.publish, 1);
        tr.publish = -1;
    }
    if (tr.pend >= 0) {
        const int32_t b = tr.pend + 16 * lane;
        if (b < tr.bytes)
            store_wt(tr.dst, (uint32_t)b, tr.data);
        if (tr.pend + SLICE >= tr.bytes) {       // that was the piece's last slice
            tr.publish = tr.chunk;
            tr.chunk = -1;
        }
        tr.pend = -1;
    }
    if (tr.chunk < 0 && !tr.exhausted)
        trickle_take(kparams(), tr);
    if (tr.chunk >= 0) {
        if (tr.bytes == 0) {                     // empty piece past a short chunk's end
            tr.publish = tr.chunk;
            tr.chunk = -1;
        } else {
            const int32_t b = tr.off + 16 * lane;
            if (b < tr.bytes)
                tr.data = *reinterpret_cast<const i32x4*>(tr.src + b);
            tr.pend = tr.off;
            tr.off += SLICE;
        }
    }
}

// Finishes this wave's piece at full speed and publishes everything it holds (per wave, no
// barrier): called before the workgroup waits on a chunk and when the kernel ends.
__device__ void trickle_flush(const KParams& p, Trickle& tr, int lane)
{
    if (tr.pend >= 0) {
        const int64_t b = tr.pend + 16 * lane;
        if (b < tr.bytes)
            store_wt(tr.dst, (uint32_t)b, tr.data);
        tr.pend = -1;
    }
    if (tr.chunk >= 0) {
        // the rest of the piece, four slices in flight per lane
        for (int32_t o = tr.off; o < tr.bytes; o += 4 * SLICE) {
            i32x4 v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t b = o + i * SLICE + 16 * lane;
                if (b < tr.bytes)
                    v[i] = *reinterpret_cast<const i32x4*>(tr.src + b);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t b = o + i * SLICE + 16 * lane;
                if (b < tr.bytes)
                    store_wt(tr.dst, (uint32_t)b, v[i]);
            }
        }
    }
    wait_vmcnt0();
    if (tr.publish >= 0) {
        publish(p, tr.publish, 1);
        tr.publish = -1;
    }
    if (tr.chunk >= 0) {
        publish(p, tr.chunk, 1);
        tr.chunk = -1;
    }
}

// Copy kernel run beside the GEMM (or before it), taking pieces from one counter: the same loop
// shape as wait_rows, never waiting on anything.
template <int U>
__device__ void drain_pieces(const KParams& p, uint32_t* ctr, int64_t end, int tid, bool wave0, int64_t* s_cmd)
{
    if (wave0) {
        int64_t n;
        s_cmd[0] = take(ctr, end, WAIT_BATCH, &n);
        s_cmd[1] = n;
    }
    for (;;) {
        barrier_after_lds_write();
        const int64_t q = uniform_i64(s_cmd[0]);
        const int64_t n = uniform_i64(s_cmd[1]);
        __syncthreads();
        if (n <= 0)
            break;
        copy_pieces<U>(p, q, n, tid);
        if (wave0) {
            publish_range(p, q, n);
            int64_t m;
            s_cmd[0] = take(ctr, end, WAIT_BATCH, &m);
            s_cmd[1] = m;
        }
    }
}

// ------------------------------------------------------------------------------------ GEMM
// The GEMM itself; MODE plain or fused.  TRICKLE: the running waves' background copy is compiled in
// (in-kernel producer only).  Idle, its bookkeeping still costs a few percent of the K loop, so
// every other schedule runs without it.
template <int MODE, bool TRICKLE, bool F8>
__device__ __forceinline__ void gemm_body(KParams p)
{
    __shared__ __attribute__((aligned(1024))) char sA0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char sB0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char sA1[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char sB1[TILE_BYTES];
    __shared__ int64_t s_cmd[2];
    __shared__ int32_t s_ready;    // wave 0's verdict on the next tile's chunks (all flags raised)
    __shared__ WaitStats s_ws;

    const GemmArgs& a = p.a;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int wm = wave >> 1, wn = wave & 1;
    const bool wave0 = (wave == 0);
    const int G = gridDim.x;
    // XCD-aware id: workgroups are dispatched round-robin over the 8 XCDs, so give each XCD a
    // contiguous run of tile ids (neighbouring tiles share A rows / B rows in that XCD's L2).
    const int vid = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int64_t num_tiles = (int64_t)p.num_pid_m * p.num_pid_n;
    // A K step is one 128-byte row segment per operand row: 64 bf16 or 128 FP8 elements.
    const int64_t K = a.K;
    const int64_t KB = F8 ? K : K * 2;             // bytes per row of A and B
    const int64_t nk = (KB + 127) / 128;
    const int64_t lo = (int64_t)a.local_rank * a.H, hi = lo + a.H;

    // per-thread constants of the global->LDS copy: slot t of every 256-slot block
    const uint32_t r_in = tid >> 3;                  // row within a 32-row block
    const uint32_t cchunk = (tid & 7) ^ swz(r_in);   // logical 16-byte chunk this slot holds
    const uint32_t row_stride32 = (uint32_t)(32 * KB);
    const uint32_t voff0 = r_in * (uint32_t)KB + cchunk * 16;
    const int32_t kval_lim = (int32_t)KB - (int32_t)cchunk * 16;   // this slot's chunk is in the row
                                                                    // in K steps kb * 128 < kval_lim
    const uint32_t lds_wave_off = wave * 1024;

    // per-lane constants of the LDS->VGPR fragment reads.  bf16: substep kk (16 k) reads chunk
    // 2 kk + fh of its row.  FP8: substep kk (64 k) reads chunks 4 kk + 2 fh and the one after it,
    // at a_off[2 kk] and a_off[2 kk + 1] (A and B fragments take the k values in the same lane
    // order, so the dot products are those of A and B's rows whatever order the instruction sums
    // them in).
    const uint32_t fr = lane & 31, fh = lane >> 5;
    const uint32_t fsw = swz(fr & 15);
    uint32_t a_off[4], b_off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t chunk = F8 ? (uint32_t)(4 * (q >> 1) + (q & 1)) + 2 * fh : (uint32_t)(2 * q) + fh;
        const uint32_t phys = chunk ^ fsw;
        a_off[q] = (wm * 128 + fr) * 128 + phys * 16;
        b_off[q] = (wn * 128 + fr) * 128 + phys * 16;
    }

    bool exhausted = false;   // (wave 0) no piece left to claim in this call
    bool failed = false;      // this workgroup gave up waiting (sticky, uniform)
    Trickle tr;               // this wave's in-loop copy (wave-uniform state)
    tr.chunk = -1;
    tr.pend = -1;
    tr.publish = -1;
    tr.exhausted = !(MODE == kGemmFused && TRICKLE && p.trickle);
    // Wave 0 reads the flags of the next tile's chunks when this tile's K loop starts and judges
    // them after its epilogue; if all were raised the next tile skips the wait (and its round
    // trips) altogether.  Any other outcome takes the ordinary wait.
    uint32_t peek = 0;
    int peek_n = -1;
    if (MODE == kGemmFused && wave0)
        s_ws = WaitStats{0, 0, 0, 0};

    for (int64_t t = vid; t < num_tiles; t += G) {
        const TileCoord tc = tile_of(t, p.num_pid_m, p.num_pid_n, p.pivot);
        const int64_t m1 = min(tc.m0 + BM, a.M);
        const char* a_base;
        int64_t a_rows;
        if (MODE == kGemmFused && tc.m0 >= lo && m1 <= hi) {
            a_base = static_cast<const char*>(a.shards[a.local_rank]) + (tc.m0 - lo) * KB;
            a_rows = m1 - tc.m0;
        } else {
            if (MODE == kGemmFused) {
                const bool ready = t != vid && __builtin_amdgcn_readfirstlane(s_ready) != 0;
                if (!ready) {
                    trickle_flush(kparams(), tr, lane);  // a piece this wave holds never waits on anything
                    wait_rows(kparams(), tc.m0, m1, t, tid, wave0, s_cmd, exhausted, failed, &s_ws);
                } else {
                    if (kparams().pm.row_bytes % 128 != 0)
                        acquire_agent();     // as at the end of an ordinary wait
                    if (wave0)
                        s_ws.skipped += 1;
                }
            }
            a_base = static_cast<const char*>(a.A) + tc.m0 * KB;
            a_rows = m1 - tc.m0;
        }
        if (MODE == kGemmFused && wave0) {
            peek_n = -1;
            const int64_t tn = t + G;
            if (tn < num_tiles) {
                const TileCoord nc = tile_of(tn, p.num_pid_m, p.num_pid_n, p.pivot);
                const int64_t nm1 = min(nc.m0 + BM, a.M);
                if (!(nc.m0 >= lo && nm1 <= hi))
                    peek = peek_rows(kparams(), nc.m0, nm1, lane, &peek_n);
            }
        }
        const int64_t b_rows = min((int64_t)BN, a.Nc - tc.n0);
        const char* b_base = static_cast<const char*>(a.B) + tc.n0 * KB;
        const uint32_t a_bytes = (uint32_t)(a_rows * KB);
        const uint32_t b_bytes = (uint32_t)(b_rows * KB);

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[i][j][v] = 0.0f;

        // Loads of K step kb into one stage: 8 + 8 DMA operations of 16 bytes per lane.  The
        // resource is re-based by the step's 128 bytes per row and shrunk by as many, so rows past
        // the tile's valid rows read zeros; a 16-byte chunk past the row's end starts its offsets at
        // the tile's full byte size, at or beyond this step's resource size, so it reads zeros (no
        // branch per lane).
        // The 16 LDS destinations and row offsets of a stage are rebuilt from the wave's LDS offset
        // and the row stride at every K step (one scalar op each): left to itself the compiler
        // keeps all of them in scalar registers for the whole kernel, and with the fused
        // schedule's state also live they spill into the K loop.
        struct Dma {
            __amdgpu_buffer_rsrc_t ra, rb;
            uint32_t va, vb;
            char *sa, *sb;
            uint32_t lw, rs;
            bool on;
        };
        auto dma_setup = [&](bool on, int64_t kb, char* sa, char* sb) {
            Dma d;
            d.lw = lds_wave_off;
            d.rs = row_stride32;
            asm volatile("" : "+s"(d.lw), "+s"(d.rs));
            const uint32_t kbyte = (uint32_t)(kb * 128);
            d.ra = make_rsrc(a_base + kbyte, a_bytes - kbyte);
            d.rb = make_rsrc(b_base + kbyte, b_bytes - kbyte);
            const bool kval = (int32_t)(kb * 128) < kval_lim;
            d.va = kval ? voff0 : a_bytes;
            d.vb = kval ? voff0 : b_bytes;
            d.sa = sa;
            d.sb = sb;
            d.on = on;
            return d;
        };
        auto dma_op = [&](const Dma& d, int q) {
            if (!d.on)
                return;
            if (q < 8)
                dma16(d.ra, d.sa + q * 4096 + d.lw, d.va + q * d.rs);
            else
                dma16(d.rb, d.sb + (q - 8) * 4096 + d.lw, d.vb + (q - 8) * d.rs);
        };
        auto issue_all = [&](int64_t kb, char* sa, char* sb) {
            const Dma d = dma_setup(true, kb, sa, sb);
#pragma unroll
            for (int q = 0; q < 16; ++q)
                dma_op(d, q);
        };

        // Fragment reads of substep kk: four A and four B fragments, one ds_read_b128 each.
        auto load_frags = [&](const char* sa, const char* sb, int kk, bf16x8* af, bf16x8* bfr) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(sa + a_off[kk] + i * 4096);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(sb + b_off[kk] + j * 4096);
        };
        // 16 MFMAs of one k-substep, and between them, one per two MFMAs: after odd ones the DMA
        // operations q0, q0+1, ... of the next stage (ndma of them, 0 or 8), after even ones the
        // fragment reads of substep `next` into (naf, nbf) (next >= 0; B's four first, which the
        // next block's first MFMAs need, then A's).  Spread out like this neither the texture
        // path nor the LDS queue backs up into this wave's MFMA issue: the same reads in one burst
        // between blocks cost the GEMM about 3 %.  sched_barrier holds every operation in its slot.
        auto mfma_block = [&](const bf16x8* af, const bf16x8* bfr, const Dma& d, int q0, int ndma,
                              const char* sa, const char* sb, int next, bf16x8* naf, bf16x8* nbf) {
#pragma unroll
            for (int g = 0; g < 16; ++g) {
                const int i = g >> 2, j = g & 3;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (ndma > 0 && (g & 1) == 1)
                    dma_op(d, q0 + (g >> 1));
                if (next >= 0 && (g & 1) == 0) {
                    const int r = g >> 1;
                    if (r < 4)
                        nbf[r] = *reinterpret_cast<const bf16x8*>(sb + b_off[next] + r * 4096);
                    else
                        naf[r - 4] = *reinterpret_cast<const bf16x8*>(sa + a_off[next] + (r - 4) * 4096);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // One K step out of stage (sa, sb) while the loads of the next step fill the other stage:
        // the first substep's fragments are read in one burst after the step's barrier (nothing
        // else is ready), each later substep's during the block before it.  All 16 DMA operations
        // go out during the first two blocks, which leaves the last two (1024 MFMA cycles) for
        // them to land before the next barrier.
        auto compute_bf16 = [&](const char* sa, const char* sb, const Dma& d) {
            bf16x8 a0[4], b0[4], a1[4], b1[4];
            load_frags(sa, sb, 0, a0, b0);
            __builtin_amdgcn_sched_barrier(0);
            mfma_block(a0, b0, d, 0, 8, sa, sb, 1, a1, b1);
            mfma_block(a1, b1, d, 8, 8, sa, sb, 2, a0, b0);
            mfma_block(a0, b0, d, 0, 0, sa, sb, 3, a1, b1);
            mfma_block(a1, b1, d, 0, 0, sa, sb, -1, nullptr, nullptr);
            __builtin_amdgcn_sched_barrier(0);
        };
        // FP8: a lane's fragment of substep kk is its row's 32 bytes at k bytes [64 kk + 32 fh, +32),
        // two chunks; a K step is two substeps of 16 v_mfma_f32_32x32x64_f8f6f4 (E4M3 operands: both
        // format fields 0; no block scales), in rows i of four MFMAs that share A fragment i.  The
        // B fragments of both substeps stay in registers (the second substep's read during the
        // first, one per row of MFMAs); the A fragments stream, each read one row of MFMAs ahead (80
        // VGPRs of fragments instead of 128, which keeps the fused kernel within the VGPR budget it
        // shares with the copy kernel beside it).  The 16 DMA operations of the
        // next stage go out one per MFMA of the first substep -- the same spacing in time as the
        // bf16 step's -- which leaves the second substep for them to land.
        auto frag8 = [&](const char* base, const uint32_t* off, int kk, int i) {
            const i32x4 x = *reinterpret_cast<const i32x4*>(base + off[2 * kk] + i * 4096);
            const i32x4 y = *reinterpret_cast<const i32x4*>(base + off[2 * kk + 1] + i * 4096);
            return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        auto compute_f8 = [&](const char* sa, const char* sb, const Dma& d) {
            i32x8 b0[4], b1[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b0[j] = frag8(sb, b_off, 0, j);
            i32x8 ac = frag8(sa, a_off, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool more = st == 0 || i < 3;
                    i32x8 an = ac;
                    if (more)
                        an = frag8(sa, a_off, i < 3 ? st : 1, i < 3 ? i + 1 : 0);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(st == 0 ? b0[j] : b1[j], ac,
                                                                                    acc[i][j], 0, 0, 0, 0, 0, 0);
                        if (st == 0) {
                            __builtin_amdgcn_sched_barrier(0);
                            dma_op(d, 4 * i + j);
                            if (j == 1)
                                b1[i] = frag8(sb, b_off, 1, i);   // the second substep's B, spread out
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    ac = an;
                }
            }
        };
        auto compute = [&](const char* sa, const char* sb, const Dma& d) {
            if constexpr (F8)
                compute_f8(sa, sb, d);
            else
                compute_bf16(sa, sb, d);
        };

        // Double-buffered K loop.  With an odd number of K steps the first one runs alone out of
        // stage 1, so the pair loop always computes twice per iteration (one accumulator PHI).
        // Every K step starts after the drain of this wave's loads and stores and a barrier; the
        // in-loop copy (fused schedule) issues its store and its next load right there, so both
        // have a whole step to land.
        int64_t kb = 0;
        if (nk & 1) {
            issue_all(0, sA1, sB1);
            wait_vmcnt0();
            __syncthreads();
            if (MODE == kGemmFused && TRICKLE)
                trickle_step(tr, lane);
            compute(sA1, sB1, dma_setup(nk > 1, 1, sA0, sB0));
            kb = 1;
        } else if (nk > 0) {
            issue_all(0, sA0, sB0);
        }
        for (; kb < nk; kb += 2) {
            wait_vmcnt0();
            __syncthreads();
            if (MODE == kGemmFused && TRICKLE)
                trickle_step(tr, lane);
            compute(sA0, sB0, dma_setup(true, kb + 1, sA1, sB1));
            wait_vmcnt0();
            __syncthreads();
            if (MODE == kGemmFused && TRICKLE)
                trickle_step(tr, lane);
            compute(sA1, sB1, dma_setup(kb + 2 < nk, kb + 2, sA0, sB0));
        }
        __syncthreads();   // all waves done with the LDS before the next tile's loads

        // Epilogue, one 32-row slab of the wave's 128x128 block at a time.  The accumulators go to
        // LDS as fp32 straight from AGPRs (a VALU use would make the register allocator carry them
        // in VGPRs through the K loop), 16 KiB per wave in stage 0; the read-back converts to bf16
        // (round to nearest even) and writes 8 consecutive columns (16 bytes) per lane, so a row
        // segment of 256 B leaves in one coalesced piece.  Slab rows are 512 B; the 16-byte unit at
        // byte b of row r sits at b ^ (r * 16), which keeps the LDS accesses (nearly) conflict-free.
        // C is never read back here, so its vector stores are non-temporal: they stream through L2
        // instead of displacing the A and B lines that neighbouring tiles (and, in the fused
        // kernel, the gathered chunks) still read; worth about 1% on the fused square and MLP-up
        // workloads, nothing elsewhere.
        // FP8 output (the FP8_OUTPUT variant of [AGMM] MatMul 按需等待): the 8 values, times
        // out_scale, go through the hardware's E4M3 "fn" conversion (round to nearest even, NaN
        // beyond 448: the conversion of torch.float8_e4m3fn) and leave as 8 bytes.
        // GEMM + ReduceScatter: this tile holds rows another kernel reduces as soon as their tile row
        // is complete, so its C goes out write-through (in memory once this wave's store count
        // drains, dirty in no L2), and the tile is counted after every wave's stores have drained.
        // Only with Nc % 8 == 0 (the caller checks).
        const bool publish = MODE == kGemmPlain && a.tile_done != nullptr && tc.m0 < a.pub_hi &&
                             tc.m0 + BM > a.pub_lo;
        {
            char* slab = (wave < 2 ? sA0 : sB0) + (wave & 1) * 16384;
            const int64_t wrow0 = tc.m0 + wm * 128, wcol0 = tc.n0 + wn * 128;
            const bool vec_ok = (a.Nc % 8) == 0;
            const bool fp8 = a.out_fp8 != 0;
            const float scale = a.out_scale;
            __bf16* C = static_cast<__bf16*>(a.C);
            uint8_t* C8 = static_cast<uint8_t*>(a.C);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // lane holds slab row lane%32, columns j*32 + g*8 + (lane/32)*4 + e, e = 0..3
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const uint32_t colb = (j * 32 + g * 8 + fh * 4) * 4;
                        const f32x4 v4 = {acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1],
                                          acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]};
                        *reinterpret_cast<f32x4*>(slab + fr * 512 + (colb ^ (fr << 4))) = v4;
                    }
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's slab is written
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int it = 0; it < 8; ++it) {
                    const uint32_t pidx = it * 64 + lane;          // row pidx/16, 8 columns
                    const uint32_t r = pidx >> 4, c8 = (pidx & 15) * 8;
                    const f32x4 x0 = *reinterpret_cast<const f32x4*>(slab + r * 512 + ((c8 * 4) ^ (r << 4)));
                    const f32x4 x1 = *reinterpret_cast<const f32x4*>(slab + r * 512 + (((c8 + 4) * 4) ^ (r << 4)));
                    const int64_t grow = wrow0 + i * 32 + r, gcol = wcol0 + c8;
                    if (fp8) {
                        // bytes 0..3 from x0, 4..7 from x1; each call fills one 16-bit half
                        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x0[0] * scale, x0[1] * scale, 0, false);
                        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x0[2] * scale, x0[3] * scale, w0, true);
                        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x1[0] * scale, x1[1] * scale, 0, false);
                        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x1[2] * scale, x1[3] * scale, w1, true);
                        if (grow < a.M) {
                            uint8_t* dstp = C8 + grow * a.Nc + gcol;
                            if (vec_ok && gcol + 8 <= a.Nc) {
                                __builtin_nontemporal_store(i32x2{w0, w1}, reinterpret_cast<i32x2*>(dstp));
                            } else {
                                for (int e = 0; e < 8; ++e)
                                    if (gcol + e < a.Nc)
                                        dstp[e] = (uint8_t)(((uint32_t)(e < 4 ? w0 : w1)) >> (8 * (e & 3)));
                            }
                        }
                        continue;
                    }
                    bf16x8 o;
                    if constexpr (F8) {
                        // FP8 inputs: the caller's per-tensor scales come in as out_scale
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            o[e] = (__bf16)(x0[e] * scale);
                            o[4 + e] = (__bf16)(x1[e] * scale);
                        }
                    } else {
                        o[0] = (__bf16)x0[0];
                        o[1] = (__bf16)x0[1];
                        o[2] = (__bf16)x0[2];
                        o[3] = (__bf16)x0[3];
                        o[4] = (__bf16)x1[0];
                        o[5] = (__bf16)x1[1];
                        o[6] = (__bf16)x1[2];
                        o[7] = (__bf16)x1[3];
                    }
                    if (publish) {
                        const __amdgpu_buffer_rsrc_t rc =
                            make_rsrc(C + (wrow0 + i * 32) * a.Nc + wcol0, (uint32_t)(32 * a.Nc * 2));
                        if (grow < a.M && gcol + 8 <= a.Nc)
                            store_wt(rc, (uint32_t)((r * a.Nc + c8) * 2), __builtin_bit_cast(i32x4, o));
                    } else if (grow < a.M) {
                        __bf16* dstp = C + grow * a.Nc + gcol;
                        if (vec_ok && gcol + 8 <= a.Nc) {
                            __builtin_nontemporal_store(o, reinterpret_cast<bf16x8*>(dstp));
                        } else {
                            for (int e = 0; e < 8; ++e)
                                if (gcol + e < a.Nc)
                                    dstp[e] = o[e];
                        }
                    }
                }
                __builtin_amdgcn_s_waitcnt(0xC07F);   // reads done before the slab is rewritten
                __builtin_amdgcn_wave_barrier();
            }
        }
        if (MODE == kGemmFused) {
            if (wave0) {
                const bool stale = peek_n >= 0 && lane < peek_n && peek != a.epoch;
                const bool ok = peek_n >= 0 && __builtin_amdgcn_ballot_w64(stale) == 0;
                if (lane == 0)
                    s_ready = ok ? 1 : 0;
            }
            barrier_after_lds_write();   // s_ready is visible; LDS is free for the next tile's loads
        } else {
            if (publish)
                wait_vmcnt0();
            __syncthreads();   // LDS is free again for the next tile's loads
            if (publish && wave0)
                (void)wave_fetch_add(&a.tile_done[tc.m0 / BM - a.pub_lo / BM], 1u);
        }
    }
    if (MODE == kGemmFused && wave0 && kparams().a.wait_stats) {
        uint64_t* st = kparams().a.wait_stats;
        const WaitStats w = s_ws;      // written by this wave only
        wave_add_u64(&st[0], w.ticks);
        wave_add_u64(&st[1], w.waits);
        wave_add_u64(&st[2], w.copied);
        wave_add_u64(&st[3], w.skipped);
    }
    if (MODE == kGemmFused) {
        // the gathered output needs every chunk, also those no tile waited for: before it exits,
        // the workgroup copies whatever is still unclaimed
        const KParams& q = kparams();
        trickle_flush(q, tr, lane);
        if (q.npieces > 0) {
            drain_pieces<8>(q, q.a.ticket, q.fill_end, tid, wave0, s_cmd);
            drain_pieces<8>(q, q.a.ticket + 1, q.npieces, tid, wave0, s_cmd);
        }
    }
}

// The kernels.  KParams is each one's first (only) argument, which kparams() relies on.
__global__ __launch_bounds__(NT, 1) void gemm_plain_kernel(KParams p)
{
    gemm_body<kGemmPlain, false, false>(p);
}

__global__ __launch_bounds__(NT, 1) void gemm_plain_f8_kernel(KParams p)
{
    gemm_body<kGemmPlain, false, true>(p);
}

// The fused kernels run beside other work on every CU -- the side-stream copy kernel, the runtime's
// small kernels that write the copy-engine producer's flags -- and must leave room for one wave of
// it per SIMD: the fused kernel's VGPRs plus the copy kernel's, each rounded up to the allocation
// granule of 8, stay within the 512 per lane (a test compiles both and checks).  Without that
// room those kernels cannot start until the GEMM ends, while the GEMM waits for them.
__global__ __launch_bounds__(NT, 1) void gemm_fused_kernel(KParams p)
{
    gemm_body<kGemmFused, false, false>(p);
}

__global__ __launch_bounds__(NT, 1) void gemm_fused_trickle_kernel(KParams p)
{
    gemm_body<kGemmFused, true, false>(p);
}

__global__ __launch_bounds__(NT, 1) void gemm_fused_f8_kernel(KParams p)
{
    gemm_body<kGemmFused, false, true>(p);
}

__global__ __launch_bounds__(NT, 1) void gemm_fused_trickle_f8_kernel(KParams p)
{
    gemm_body<kGemmFused, true, true>(p);
}

// Copy kernel of the side-stream schedule, beside the GEMM.  It is small -- no LDS tile, few VGPRs --
// so its workgroups fit next to the GEMM's.
template <int U>
__global__ __launch_bounds__(NT) void producer_kernel(KParams p, uint32_t* ctr, int64_t end)
{
    __shared__ int64_t s_cmd[2];
    const int tid = threadIdx.x;
    const bool wave0 = __builtin_amdgcn_readfirstlane(tid >> 6) == 0;
    drain_pieces<U>(p, ctr, end, tid, wave0, s_cmd);
}

// Start of a side-stream fused call, alone on the GPU before the GEMM and the copy kernel beside it:
// pieces [0, fill_end) -- every chunk the first wave of tiles reads -- are copied by the whole GPU,
// FILL_PIECES pieces per workgroup in one pass (each lane's loads all in flight, then its stores;
// units past a piece's end read zeros and store nothing, so no lane takes a branch); the flags of
// those chunks are raised, the piece counters start past them and the per-chunk piece counts at
// zero.  Nothing reads the flags, counters or copied rows before this kernel has ended.
// The kernel is short and latency-bound, so it is spread wide: one piece per workgroup copies the
// square workload's 16 MiB first wave in about 9 us, four per workgroup took 13.5 us, two 10.6 us,
// and half a piece per workgroup is no faster than one.
constexpr int FILL_PIECES = 1;

__global__ __launch_bounds__(NT) void fill_kernel(KParams p)
{
    const GemmArgs& a = p.a;
    const int tid = threadIdx.x;
    const int64_t gid = (int64_t)blockIdx.x * NT + tid, gsize = (int64_t)gridDim.x * NT;
    if (gid == 0) {
        a.ticket[0] = (uint32_t)p.fill_end;   // a waiting tile finds the fill's pieces taken
        a.ticket[1] = (uint32_t)p.fill_end;
    }
    for (int64_t i = gid; i < p.pm.nchunks; i += gsize)
        a.done[i] = 0;
    for (int64_t pos = gid; pos < p.fill_end / p.pm.ppc; pos += gsize)
        a.flags[pm_ready_chunk(p.pm, pos)] = a.epoch;
    const int64_t q0 = (int64_t)blockIdx.x * FILL_PIECES;
    __amdgpu_buffer_rsrc_t src[FILL_PIECES], dst[FILL_PIECES];
#pragma unroll
    for (int j = 0; j < FILL_PIECES; ++j) {
        int64_t bytes = 0;
        const char* from = static_cast<const char*>(a.A);
        const char* to = static_cast<const char*>(a.A);
        if (q0 + j < p.fill_end) {
            const PieceSpan sp = piece_at(p, q0 + j);
            from = static_cast<const char*>(a.shards[sp.shard]) + sp.src_off;
            to += sp.dst_off;
            bytes = sp.bytes;
        }
        // the values are the same in every lane; saying so keeps the copies free of per-lane loops
        // over the buffer resources
        src[j] = span_rsrc(reinterpret_cast<const char*>(uniform_i64(reinterpret_cast<int64_t>(from))),
                           uniform_i64(bytes));
        dst[j] = span_rsrc(reinterpret_cast<const char*>(uniform_i64(reinterpret_cast<int64_t>(to))),
                           uniform_i64(bytes));
    }
    i32x4 v[FILL_PIECES][PIECE_UNITS];
#pragma unroll
    for (int j = 0; j < FILL_PIECES; ++j)
#pragma unroll
        for (int u = 0; u < PIECE_UNITS; ++u)
            v[j][u] = __builtin_amdgcn_raw_buffer_load_b128(src[j], (uint32_t)((tid + u * NT) * 16), 0, 0);
#pragma unroll
    for (int j = 0; j < FILL_PIECES; ++j)
#pragma unroll
        for (int u = 0; u < PIECE_UNITS; ++u)
            store_wt(dst[j], (uint32_t)((tid + u * NT) * 16), v[j][u]);
}

// Start of a fused call: piece counters, per-chunk piece counts.  A call that gave up leaves its
// counters in any state; every call starts from here, so the next one is unaffected.
__global__ void reset_kernel(uint32_t* ticket, uint32_t fill_start, uint32_t main_start, uint32_t* done, int64_t n)
{
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i == 0) {
        ticket[0] = fill_start;
        ticket[1] = main_start;
    }
    for (int64_t j = i; j < n; j += (int64_t)gridDim.x * blockDim.x)
        done[j] = 0;
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

constexpr int kMaxDevices = 64;
int g_num_cus[kMaxDevices] = {};

KParams make_params(const GemmArgs& a, GemmMode mode)
{
    KParams p;
    p.a = a;
    p.num_pid_m = (int)((a.M + BM - 1) / BM);
    p.num_pid_n = (int)((a.Nc + BN - 1) / BN);
    p.pivot = 0;
    p.npieces = 0;
    p.fill_end = 0;
    p.trickle = 0;
    const int64_t row_bytes = a.in_fp8 ? a.K : a.K * 2;
    p.pm = pm_make(1, 1, 1, 0, row_bytes, BM, PIECE_BYTES);
    if (mode == kGemmFused) {
        p.pivot = (int)(((int64_t)a.local_rank * a.H) / BM % p.num_pid_m);
        p.pm = pm_make(a.H, a.cb, a.nshards, a.local_rank, row_bytes, BM, PIECE_BYTES);
        p.npieces = a.copy_pieces ? p.pm.nchunks * p.pm.ppc : 0;
        p.trickle = a.copy_pieces == 1 ? 1 : 0;
    } else if (a.tile_done) {
        p.pivot = (int)((a.pub_lo / BM) % p.num_pid_m);   // the reducing rank's rows first
    }
    return p;
}

int gemm_grid(const KParams& p, int cus)
{
    const int64_t tiles = (int64_t)p.num_pid_m * p.num_pid_n;
    return (int)std::max<int64_t>(1, std::min<int64_t>(tiles, cus));
}

hipError_t num_cus(int* out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipDeviceGetAttribute(out, hipDeviceAttributeMultiprocessorCount, dev);
    if (g_num_cus[dev] == 0) {
        e = hipDeviceGetAttribute(&g_num_cus[dev], hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
    }
    *out = g_num_cus[dev];
    return hipSuccess;
}

// Pieces [0, n) of the ready order hold every chunk that the first wave of GEMM tiles (one tile per
// workgroup of the persistent grid) reads from the aggregate buffer.
int64_t first_wave_end(const KParams& p, int cus)
{
    const GemmArgs& a = p.a;
    if (p.npieces <= 0 || a.reverse_order)
        return 0;
    const int64_t lo = (int64_t)a.local_rank * a.H, hi = lo + a.H;
    const int64_t tiles = (int64_t)p.num_pid_m * p.num_pid_n;
    const int64_t first = std::min<int64_t>(tiles, gemm_grid(p, cus));
    int64_t last_pos = -1;
    for (int64_t t = 0; t < first; ++t) {
        const TileCoord tc = tile_of(t, p.num_pid_m, p.num_pid_n, p.pivot);
        const int64_t m1 = std::min<int64_t>(tc.m0 + BM, a.M);
        if (tc.m0 >= lo && m1 <= hi)
            continue;
        int64_t c0, c1;
        pm_chunks_of_rows(p.pm, tc.m0, m1, c0, c1);
        for (int64_t c = c0; c <= c1; ++c)
            last_pos = std::max(last_pos, pm_ready_pos(p.pm, c));
    }
    return (last_pos + 1) * p.pm.ppc;
}

}  // namespace

int gemm_tile_m() { return BM; }
int gemm_tile_n() { return BN; }

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t stream)
{
    if (n <= 0)
        return hipSuccess;
    const int blocks = (int)std::min<int64_t>((n + 255) / 256, 1024);
    fill_u32_kernel<<<blocks, 256, 0, stream>>>(p, n, value);
    return hipGetLastError();
}

FusedPlan plan_fused(const GemmArgs& a)
{
    FusedPlan f;
    f.npieces = 0;
    f.fill_end = 0;
    f.nchunks = 0;
    int cus = 0;
    if (num_cus(&cus) != hipSuccess)
        return f;
    const KParams p = make_params(a, kGemmFused);
    f.npieces = p.npieces;
    f.fill_end = first_wave_end(p, cus);
    f.nchunks = p.pm.nchunks;
    return f;
}

hipError_t launch_reset(const GemmArgs& a, const FusedPlan& f, hipStream_t stream)
{
    const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((f.nchunks + 255) / 256, 256));
    reset_kernel<<<blocks, 256, 0, stream>>>(a.ticket, 0u, (uint32_t)f.fill_end, a.done, f.nchunks);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, GemmMode mode, const FusedPlan* f, hipStream_t stream)
{
    int cus = 0;
    hipError_t e = num_cus(&cus);
    if (e != hipSuccess)
        return e;
    KParams p = make_params(a, mode);
    if (f)
        p.fill_end = f->fill_end;
    const int grid = gemm_grid(p, cus);
    if (mode == kGemmFused) {
        if (p.trickle)
            (a.in_fp8 ? gemm_fused_trickle_f8_kernel : gemm_fused_trickle_kernel)<<<grid, NT, 0, stream>>>(p);
        else
            (a.in_fp8 ? gemm_fused_f8_kernel : gemm_fused_kernel)<<<grid, NT, 0, stream>>>(p);
    } else {
        (a.in_fp8 ? gemm_plain_f8_kernel : gemm_plain_kernel)<<<grid, NT, 0, stream>>>(p);
    }
    return hipGetLastError();
}

hipError_t launch_producer(const GemmArgs& a, const FusedPlan& f, hipStream_t stream)
{
    int cus = 0;
    hipError_t e = num_cus(&cus);
    if (e != hipSuccess)
        return e;
    KParams p = make_params(a, kGemmFused);
    p.fill_end = f.fill_end;
    if (p.npieces <= f.fill_end)
        return hipSuccess;
    const int64_t batches = (p.npieces - f.fill_end + WAIT_BATCH - 1) / WAIT_BATCH;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(batches, cus));
    producer_kernel<8><<<grid, NT, 0, stream>>>(p, a.ticket + 1, p.npieces);
    return hipGetLastError();
}

hipError_t launch_fill(const GemmArgs& a, const FusedPlan& f, hipStream_t stream)
{
    KParams p = make_params(a, kGemmFused);
    p.fill_end = f.fill_end;
    const int64_t grid = std::max<int64_t>(1, (f.fill_end + FILL_PIECES - 1) / FILL_PIECES);
    if (grid > INT32_MAX)
        return hipErrorInvalidValue;
    fill_kernel<<<(int)grid, NT, 0, stream>>>(p);
    return hipGetLastError();
}

hipError_t device_cus(int* out) { return num_cus(out); }

}  // namespace ag
