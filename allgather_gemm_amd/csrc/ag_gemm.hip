// ag_gemm.hip -- persistent bf16 MFMA GEMM (fp32 accumulate) for C = A * B^T on gfx950, with
// the chunked-AllGather consumer/producer logic of the fused schedule.
//
// What it computes follows the fused AllGather+MatMul article ("Triton第四课：基于对称内存融合
// AllGather 与 MatMul，提速1.56倍"):
//  * section 融合后的流水线 / MatMul 按需等待: M is split into comm blocks ("chunks"); output tiles
//    are visited with pid_m rotated to the local shard; a tile wholly inside the local shard reads
//    the shard, every other tile first waits for the flags of the chunks its rows overlap and then
//    reads the aggregate A buffer;
//  * section 数据搬运与细粒度同步: a chunk's flag is raised only after its rows have landed;
//  * section wait_signal 的实现与语义: one lane polls, then a workgroup barrier releases the block.
// The producer runs on a second stream (section 融合后的流水线 has the copy on a backend stream
// beside the MatMul): a small copy kernel whose workgroups sit next to the GEMM's on every CU.
// The chunk copies are split into pieces claimed from one counter, in ready order, by the
// producer's workgroups and also by any GEMM workgroup that would otherwise wait.  A piece is
// claimed only by a running workgroup, so no wait can deadlock whatever the two grids' residency
// or launch order: a GEMM that starts alone copies what it needs itself.
//
// Tiling (gfx950): 256x256 output tile per 256-thread workgroup (4 waves, 2x2, 128x128 each),
// K step 64, v_mfma_f32_32x32x16_bf16, A/B tiles staged in LDS by buffer_load ... lds (16 B per
// lane, no VGPR round trip), double-buffered (2 x 64 KiB).  LDS rows are 128 B (64 bf16) and
// their 16-byte chunks are XOR-swizzled so the ds_read_b128 fragment loads are conflict-free.
#include "ag_device.hpp"
#include "ag_internal.hpp"

#include <algorithm>

namespace ag {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NT = 256;                        // threads per workgroup
constexpr int SLOTS = BM * BK * 2 / 16;        // 16-byte slots per operand tile (2048)
constexpr int TILE_BYTES = SLOTS * 16;         // 32 KiB per operand tile
constexpr int GROUP_M = 8;                     // tile rows per group of the grouped order
constexpr int64_t PIECE_BYTES = 64 * 1024;     // target bytes per copy piece

static_assert(BM == BN, "A and B tiles share one LDS layout");

// Swizzle of the 16-byte chunk index inside a 128-byte LDS row: depends on row bits 0..3 so that
// any 8 (and any 16) consecutive rows reading the same logical chunk hit distinct banks.
__device__ __forceinline__ uint32_t swz(uint32_t row) { return (row & 7u) ^ ((row >> 3) & 1u); }

struct TileCoord {
    int64_t m0, n0;
    int64_t tile;
};

__host__ __device__ __forceinline__ TileCoord tile_of(int64_t t, int num_pid_m, int num_pid_n, int pivot)
{
    // grouped order, then rotation of pid_m so the walk starts at the local shard; the rotation
    // is a bijection on pid_m, so the grouping (and its L2 reuse) is kept
    const int64_t per_group = (int64_t)GROUP_M * num_pid_n;
    const int64_t group = t / per_group;
    const int64_t first_m = group * GROUP_M;
    const int64_t left = (int64_t)num_pid_m - first_m;
    const int64_t rows = left < GROUP_M ? left : (int64_t)GROUP_M;
    const int64_t in_group = t - group * per_group;
    int64_t pid_m = first_m + in_group % rows;
    const int64_t pid_n = in_group / rows;
    pid_m = (pid_m + pivot) % num_pid_m;
    TileCoord c;
    c.m0 = pid_m * BM;
    c.n0 = pid_n * BN;
    c.tile = t;
    return c;
}

struct KParams {
    GemmArgs a;
    int num_pid_m, num_pid_n, pivot;
    int64_t S, nchunks, piece_rows, ppc, npieces;
    uint32_t* claim;     // piece counter this launch claims from
    int64_t claim_end;   // pieces [counter start, claim_end) belong to this launch
};

// --------------------------------------------------------------------------------- producer
// Piece q of the copy: position q / ppc in ready order (shards local+1, local+2, ..., local),
// sub-range q % ppc of that chunk's rows.  A piece is whole rows, so it is one contiguous byte
// range in both the shard and the aggregate buffer.
struct Piece {
    const i32x4* src;
    i32x4* dst;
    int64_t units;   // 16-byte units
    int64_t chunk;
};

__device__ __forceinline__ Piece piece_of(const KParams& p, int64_t q)
{
    const GemmArgs& a = p.a;
    int64_t pos = q / p.ppc;
    const int64_t sub = q - pos * p.ppc;
    if (a.reverse_order)
        pos = p.nchunks - 1 - pos;
    const int64_t shard_step = pos / p.S, s = pos - shard_step * p.S;
    const int r = (int)((a.local_rank + 1 + shard_step) % a.nshards);
    const int64_t chunk_end = min((s + 1) * a.cb, a.H);
    const int64_t row0 = min(s * a.cb + sub * p.piece_rows, chunk_end);
    const int64_t row1 = min(row0 + p.piece_rows, chunk_end);
    Piece pc;
    pc.src = reinterpret_cast<const i32x4*>(static_cast<const char*>(a.shards[r]) + row0 * a.K * 2);
    pc.dst = reinterpret_cast<i32x4*>(static_cast<char*>(const_cast<void*>(a.A)) +
                                      ((int64_t)r * a.H + row0) * a.K * 2);
    pc.units = (row1 - row0) * a.K * 2 / 16;
    pc.chunk = (int64_t)r * p.S + s;
    return pc;
}

// All threads: copy piece q with 16-byte loads/stores (U in flight per lane), drain this wave's
// stores, then a barrier -- after it, wave 0's release covers the whole piece.
template <int U = 8>
__device__ void copy_piece_rows(const KParams& p, int64_t q, int tid)
{
    const Piece pc = piece_of(p, q);
    int64_t u = tid;
    for (; u + (U - 1) * NT < pc.units; u += U * NT) {
        i32x4 v[U];
#pragma unroll
        for (int i = 0; i < U; ++i)
            v[i] = pc.src[u + i * NT];
#pragma unroll
        for (int i = 0; i < U; ++i)
            pc.dst[u + i * NT] = v[i];
    }
    for (; u < pc.units; u += NT)
        pc.dst[u] = pc.src[u];
    wait_vmcnt0();
    __syncthreads();
}

// The single-writer steps below run on all 64 lanes of wave 0 (a wave-uniform branch), never on
// one lane: a one-lane branch inside a loop that also holds barriers lets the compiler's control
// flow structurizer peel that lane out of the loop while the other lanes keep iterating.  Counters
// take +1 from lane 0 and +0 from the others, every result is read from lane 0, and the
// remaining writes (exchange, compare-exchange, LDS store) repeat the same value.
__device__ __forceinline__ uint32_t lane0_one() { return (threadIdx.x & 63) == 0 ? 1u : 0u; }

__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Wave 0: count piece q as done; the last piece of its chunk raises the chunk's flag.
__device__ void publish_piece(const KParams& p, int64_t q)
{
    const GemmArgs& a = p.a;
    const int64_t c = piece_of(p, q).chunk;
    const uint32_t old = uniform_u32(
        __hip_atomic_fetch_add(&a.done[c], lane0_one(), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT));
    if (old + 1 == (uint32_t)p.ppc) {
        // the other pieces' releases are in this counter's release sequence: acquire them (once
        // per chunk, not per piece) so the flag's release below covers their rows too
        acquire_agent();
        (void)__hip_atomic_exchange(&a.done[c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        flag_publish(&a.flags[c], a.epoch);
    }
}

// Wave 0: next piece to copy, or -1 when none is left (then `exhausted` sticks).
__device__ int64_t claim_next(const KParams& p, bool& exhausted)
{
    if (exhausted || !p.a.copy_pieces)
        return -1;
    const uint32_t t = uniform_u32(
        __hip_atomic_fetch_add(p.claim, lane0_one(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (t < (uint32_t)p.claim_end)
        return (int64_t)t;
    exhausted = true;
    return -1;
}

constexpr int64_t kReady = -1, kIdle = -2, kFailed = -3;

// Wave 0: what the workgroup does next while it waits for chunk c: kReady, kFailed, a piece to
// copy, or kIdle (sleep and ask again).  Gives up after spin_limit ticks of the 100 MHz clock.
__device__ int64_t decide_wait(const KParams& p, int64_t c, uint64_t t_start, int64_t tile, bool& exhausted)
{
    const GemmArgs& a = p.a;
    if (uniform_u32(flag_peek(&a.flags[c])) == a.epoch)
        return kReady;
    if (uniform_u32(flag_peek(&a.status[0])) != 0)
        return kFailed;                                  // another workgroup gave up
    const int64_t q = claim_next(p, exhausted);
    if (q >= 0)
        return q;
    if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t_start) > a.spin_limit) {
        report_failure(a.status, 1u, (uint32_t)c, (uint32_t)tile);
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
__device__ void wait_rows(const KParams& p, int64_t m0, int64_t m1, int64_t tile, int tid, bool wave0,
                          int64_t* s_cmd, bool& exhausted, bool& failed)
{
    const GemmArgs& a = p.a;
    const int64_t c_first = (m0 / a.H) * p.S + (m0 % a.H) / a.cb;
    const int64_t c_last = ((m1 - 1) / a.H) * p.S + ((m1 - 1) % a.H) / a.cb;
    for (int64_t c = c_first; c <= c_last; ++c) {
        if (failed)
            break;
        const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
        if (wave0)
            *s_cmd = decide_wait(p, c, t_start, tile, exhausted);
        for (;;) {
            barrier_after_lds_write();
            const int64_t cmd = uniform_i64(*s_cmd);
            __syncthreads();
            if (cmd == kReady)
                break;
            if (cmd == kFailed) {
                failed = true;
                break;
            }
            if (cmd >= 0)
                copy_piece_rows(p, cmd, tid);
            else
                __builtin_amdgcn_s_sleep(4);
            if (wave0) {
                if (cmd >= 0)
                    publish_piece(p, cmd);
                *s_cmd = decide_wait(p, c, t_start, tile, exhausted);
            }
        }
    }
    acquire_agent();
    __syncthreads();
}

// Producer loop: claim, copy, publish until no piece is left.  Same loop shape as wait_rows.
template <int U>
__device__ void drain_pieces(const KParams& p, int tid, bool wave0, int64_t* s_cmd)
{
    bool exhausted = false;
    if (wave0)
        *s_cmd = claim_next(p, exhausted);
    for (;;) {
        barrier_after_lds_write();
        const int64_t q = uniform_i64(*s_cmd);
        __syncthreads();
        if (q < 0)
            break;
        copy_piece_rows<U>(p, q, tid);
        if (wave0) {
            publish_piece(p, q);
            *s_cmd = claim_next(p, exhausted);
        }
    }
}

// ------------------------------------------------------------------------------------ GEMM
template <int MODE>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(KParams p)
{
    __shared__ __attribute__((aligned(1024))) char sA0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char sB0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char sA1[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char sB1[TILE_BYTES];
    __shared__ int64_t s_cmd;

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
    const int64_t K = a.K;
    const int64_t nk = (K + BK - 1) / BK;
    const int64_t lo = (int64_t)a.local_rank * a.H, hi = lo + a.H;

    // per-thread constants of the global->LDS copy: slot t of every 256-slot block
    const uint32_t r_in = tid >> 3;                  // row within a 32-row block
    const uint32_t cchunk = (tid & 7) ^ swz(r_in);   // logical 16-byte chunk this slot holds
    const uint32_t row_stride32 = (uint32_t)(32 * K * 2);
    const uint32_t voff0 = r_in * (uint32_t)(K * 2) + cchunk * 16;
    const uint32_t lds_wave_off = wave * 1024;

    // per-lane constants of the LDS->VGPR fragment reads
    const uint32_t fr = lane & 31, fh = lane >> 5;
    const uint32_t fsw = swz(fr & 15);
    uint32_t a_off[4], b_off[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const uint32_t phys = ((uint32_t)(2 * kk) + fh) ^ fsw;
        a_off[kk] = (wm * 128 + fr) * 128 + phys * 16;
        b_off[kk] = (wn * 128 + fr) * 128 + phys * 16;
    }

    bool exhausted = false;   // (wave 0) no piece left to claim in this call
    bool failed = false;      // this workgroup gave up waiting (sticky, uniform)

    for (int64_t t = vid; t < num_tiles; t += G) {
        const TileCoord tc = tile_of(t, p.num_pid_m, p.num_pid_n, p.pivot);
        const int64_t m1 = min(tc.m0 + BM, a.M);
        const char* a_base;
        int64_t a_rows;
        if (MODE == kGemmFused && tc.m0 >= lo && m1 <= hi) {
            a_base = static_cast<const char*>(a.shards[a.local_rank]) + (tc.m0 - lo) * K * 2;
            a_rows = m1 - tc.m0;
        } else {
            if (MODE == kGemmFused)
                wait_rows(p, tc.m0, m1, t, tid, wave0, &s_cmd, exhausted, failed);
            a_base = static_cast<const char*>(a.A) + tc.m0 * K * 2;
            a_rows = m1 - tc.m0;
        }
        const int64_t b_rows = min((int64_t)BN, a.Nc - tc.n0);
        const char* b_base = static_cast<const char*>(a.B) + tc.n0 * K * 2;
        const uint32_t a_bytes = (uint32_t)(a_rows * K * 2);
        const uint32_t b_bytes = (uint32_t)(b_rows * K * 2);

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[i][j][v] = 0.0f;

        // Loads of K step kb into one stage.  The resource is re-based by kb*BK elements and shrunk
        // by as many bytes, so rows past the tile's valid rows read zeros; a chunk past K reads
        // zeros through an out-of-range offset.
        // Loads of K step kb into one stage: 8 + 8 DMA operations of 16 bytes per lane.  The
        // resource is re-based by kb*BK elements and shrunk by as many bytes, so rows past the
        // tile's valid rows read zeros; a 16-byte chunk past K starts its offsets at the tile's full
        // byte size, at or beyond this step's resource size, so it reads zeros (no branch per lane).
        struct Dma {
            __amdgpu_buffer_rsrc_t ra, rb;
            uint32_t va, vb;
            char *sa, *sb;
            bool on;
        };
        auto dma_setup = [&](bool on, int64_t kb, char* sa, char* sb) {
            Dma d;
            const uint32_t kbyte = (uint32_t)(kb * BK * 2);
            d.ra = make_rsrc(a_base + kbyte, a_bytes - kbyte);
            d.rb = make_rsrc(b_base + kbyte, b_bytes - kbyte);
            const bool kval = (int64_t)kb * BK + cchunk * 8 < K;
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
                dma16(d.ra, d.sa + q * 4096 + lds_wave_off, d.va + q * row_stride32);
            else
                dma16(d.rb, d.sb + (q - 8) * 4096 + lds_wave_off, d.vb + (q - 8) * row_stride32);
        };
        auto issue_all = [&](int64_t kb, char* sa, char* sb) {
            const Dma d = dma_setup(true, kb, sa, sb);
#pragma unroll
            for (int q = 0; q < 16; ++q)
                dma_op(d, q);
        };

        // Fragments of two k-substeps in flight: the reads of substep kk+1 are issued before
        // the 16 MFMAs of substep kk; sched_barrier keeps the compiler from hoisting further
        // (which would cost 128 VGPRs on top of the 256 accumulators).
        auto load_frags = [&](const char* sa, const char* sb, int kk, bf16x8* af, bf16x8* bfr) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(sa + a_off[kk] + i * 4096);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(sb + b_off[kk] + j * 4096);
        };
        // 16 MFMAs of one k-substep; with `ndma` > 0, DMA operations q0, q0+1, ... of the next
        // stage go out between them (one per 16 / ndma MFMAs) instead of in one burst, so the
        // texture path never backs up into this wave's instruction issue.
        auto mfma_block = [&](const bf16x8* af, const bf16x8* bfr, const Dma& d, int q0, int ndma) {
#pragma unroll
            for (int g = 0; g < 16; ++g) {
                const int i = g >> 2, j = g & 3;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
                if (ndma > 0 && (g + 1) % (16 / ndma) == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    dma_op(d, q0 + (g + 1) / (16 / ndma) - 1);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        // One K step out of stage (sa, sb) while the loads of the next step fill the other stage:
        // all 16 DMA operations go out during the first two substeps, which leaves the last two
        // (1024 MFMA cycles) for them to land before the next barrier.
        auto compute = [&](const char* sa, const char* sb, const Dma& d) {
            bf16x8 a0[4], b0[4], a1[4], b1[4];
            load_frags(sa, sb, 0, a0, b0);
            load_frags(sa, sb, 1, a1, b1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_block(a0, b0, d, 0, 8);
            __builtin_amdgcn_sched_barrier(0);
            load_frags(sa, sb, 2, a0, b0);
            __builtin_amdgcn_sched_barrier(0);
            mfma_block(a1, b1, d, 8, 8);
            __builtin_amdgcn_sched_barrier(0);
            load_frags(sa, sb, 3, a1, b1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_block(a0, b0, d, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            mfma_block(a1, b1, d, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        };

        // Double-buffered K loop.  With an odd number of K steps the first one runs alone out of
        // stage 1, so the pair loop always computes twice per iteration (one accumulator PHI).
        int64_t kb = 0;
        if (nk & 1) {
            issue_all(0, sA1, sB1);
            wait_vmcnt0();
            __syncthreads();
            compute(sA1, sB1, dma_setup(nk > 1, 1, sA0, sB0));
            kb = 1;
        } else if (nk > 0) {
            issue_all(0, sA0, sB0);
        }
        for (; kb < nk; kb += 2) {
            wait_vmcnt0();
            __syncthreads();
            compute(sA0, sB0, dma_setup(true, kb + 1, sA1, sB1));
            wait_vmcnt0();
            __syncthreads();
            compute(sA1, sB1, dma_setup(kb + 2 < nk, kb + 2, sA0, sB0));
        }
        __syncthreads();   // all waves done with the LDS before the next tile's loads

        // Epilogue, one 32-row slab of the wave's 128x128 block at a time.  The accumulators go to
        // LDS as fp32 straight from AGPRs (a VALU use would make the register allocator carry them
        // in VGPRs through the K loop), 16 KiB per wave in stage 0; the read-back converts to bf16
        // (round to nearest even) and writes 8 consecutive columns (16 bytes) per lane, so a row
        // segment of 256 B leaves in one coalesced piece.  Slab rows are 512 B; the 16-byte unit at
        // byte b of row r sits at b ^ (r * 16), which keeps the LDS accesses (nearly) conflict-free.
        {
            char* slab = (wave < 2 ? sA0 : sB0) + (wave & 1) * 16384;
            const int64_t wrow0 = tc.m0 + wm * 128, wcol0 = tc.n0 + wn * 128;
            const bool vec_ok = (a.Nc % 8) == 0;
            __bf16* C = static_cast<__bf16*>(a.C);
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
                    bf16x8 o;
                    o[0] = (__bf16)x0[0];
                    o[1] = (__bf16)x0[1];
                    o[2] = (__bf16)x0[2];
                    o[3] = (__bf16)x0[3];
                    o[4] = (__bf16)x1[0];
                    o[5] = (__bf16)x1[1];
                    o[6] = (__bf16)x1[2];
                    o[7] = (__bf16)x1[3];
                    const int64_t grow = wrow0 + i * 32 + r, gcol = wcol0 + c8;
                    if (grow < a.M) {
                        __bf16* dstp = C + grow * a.Nc + gcol;
                        if (vec_ok && gcol + 8 <= a.Nc) {
                            *reinterpret_cast<bf16x8*>(dstp) = o;
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
        __syncthreads();   // LDS is free again for the next tile's loads
    }

}

// Copy kernel of the fused schedule.  Beside the GEMM (U = 8) it is small -- no LDS tile, few
// VGPRs -- so its workgroups fit next to the GEMM's on every CU and the copy overlaps the MFMA work;
// it claims pieces in ready order from the same counter as the GEMM's waiting workgroups and never
// waits on anything.  Alone on the GPU, for the pipeline fill (U = 16), it keeps more loads in
// flight per lane.
template <int U>
__global__ __launch_bounds__(NT) void producer_kernel(KParams p)
{
    __shared__ int64_t s_cmd;
    const int tid = threadIdx.x;
    const bool wave0 = __builtin_amdgcn_readfirstlane(tid >> 6) == 0;
    drain_pieces<U>(p, tid, wave0, &s_cmd);
}

__global__ void set_pair_kernel(uint32_t* p, uint32_t v0, uint32_t v1)
{
    if (threadIdx.x == 0)
        p[0] = v0;
    else if (threadIdx.x == 1)
        p[1] = v1;
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
    p.S = 1;
    p.nchunks = 0;
    p.piece_rows = 1;
    p.ppc = 1;
    p.npieces = 0;
    if (mode == kGemmFused) {
        p.pivot = (int)(((int64_t)a.local_rank * a.H) / BM % p.num_pid_m);
        p.S = (a.H + a.cb - 1) / a.cb;
        p.nchunks = (int64_t)a.nshards * p.S;
        const int64_t row_bytes = a.K * 2;
        p.piece_rows = row_bytes > 0 ? std::max<int64_t>(1, PIECE_BYTES / row_bytes) : a.cb;
        p.piece_rows = std::min(p.piece_rows, a.cb);
        p.ppc = (a.cb + p.piece_rows - 1) / p.piece_rows;
        p.npieces = a.copy_pieces ? p.nchunks * p.ppc : 0;
    }
    p.claim = a.ticket;
    p.claim_end = p.npieces;
    return p;
}

int gemm_grid(const KParams& p, int cus)
{
    const int64_t tiles = (int64_t)p.num_pid_m * p.num_pid_n;
    return (int)std::max<int64_t>(1, std::min<int64_t>(tiles, cus));
}

// Ready-order position of chunk c (inverse of the mapping in piece_of).
int64_t ready_pos(const KParams& p, int64_t c)
{
    const int64_t r = c / p.S, s = c - r * p.S;
    const int64_t step = ((r - p.a.local_rank - 1) % p.a.nshards + p.a.nshards) % p.a.nshards;
    const int64_t pos = step * p.S + s;
    return p.a.reverse_order ? p.nchunks - 1 - pos : pos;
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

hipError_t launch_gemm(const GemmArgs& a, GemmMode mode, hipStream_t stream)
{
    int cus = 0;
    hipError_t e = num_cus(&cus);
    if (e != hipSuccess)
        return e;
    const KParams p = make_params(a, mode);
    const int grid = gemm_grid(p, cus);
    if (mode == kGemmFused)
        gemm_kernel<kGemmFused><<<grid, NT, 0, stream>>>(p);
    else
        gemm_kernel<kGemmPlain><<<grid, NT, 0, stream>>>(p);
    return hipGetLastError();
}

int64_t copy_pieces_total(const GemmArgs& a)
{
    return make_params(a, kGemmFused).npieces;
}

int64_t first_wave_pieces(const GemmArgs& a)
{
    int cus = 0;
    if (num_cus(&cus) != hipSuccess)
        return 0;
    const KParams p = make_params(a, kGemmFused);
    if (p.npieces <= 0)
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
        const int64_t c0 = (tc.m0 / a.H) * p.S + (tc.m0 % a.H) / a.cb;
        const int64_t c1 = ((m1 - 1) / a.H) * p.S + ((m1 - 1) % a.H) / a.cb;
        for (int64_t c = c0; c <= c1; ++c)
            last_pos = std::max(last_pos, ready_pos(p, c));
    }
    return (last_pos + 1) * p.ppc;
}

hipError_t launch_producer(const GemmArgs& a, uint32_t* counter, int64_t end, int max_grid, bool alone,
                           hipStream_t stream)
{
    KParams p = make_params(a, kGemmFused);
    p.claim = counter;
    p.claim_end = std::min(end, p.npieces);
    if (p.claim_end <= 0)
        return hipSuccess;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(p.claim_end, max_grid));
    if (alone)
        producer_kernel<16><<<grid, NT, 0, stream>>>(p);
    else
        producer_kernel<8><<<grid, NT, 0, stream>>>(p);
    return hipGetLastError();
}

hipError_t launch_set_pair(uint32_t* p, uint32_t v0, uint32_t v1, hipStream_t stream)
{
    set_pair_kernel<<<1, 64, 0, stream>>>(p, v0, v1);
    return hipGetLastError();
}

hipError_t device_cus(int* out) { return num_cus(out); }

}  // namespace ag
