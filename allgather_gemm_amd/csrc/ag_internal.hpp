// ag_internal.hpp -- host-side interface between the C ABI (ag_api.cpp) and the kernel
// translation units (tgather.hip, ag_gemm.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ag {

constexpr int kMaxShards = 64;     // shard pointers travel by value in the kernel arguments

// --------------------------------------------------------------------------------- tgather
struct GatherDesc {
    const void* src[kMaxShards];
    void* dst;
    int nranks;
    int elem_size;
    int64_t planes;        // D0 * D1 * D2
    int64_t H, W, dst_rows;
    int64_t valid_rows, valid_cols;
};

// Enqueues the gather on `stream`.  Arguments must already be validated.
hipError_t launch_tgather(const GatherDesc& d, hipStream_t stream);

// ------------------------------------------------------------------------------------ GEMM
enum GemmMode { kGemmPlain = 0, kGemmFused = 1 };

// Who copies the chunks in the fused schedule (GemmArgs::copy_pieces).
enum CopyBy {
    kCopyNone = 0,       // someone else raises the flags (copy engines, or GEMM-only with raised flags)
    kCopyInKernel = 1,   // waiting workgroups and a background copy in every running wave
    kCopyWaiters = 2,    // waiting workgroups only (a copy kernel on a second stream does the rest)
};

struct GemmArgs {
    const void* A;          // gathered A (M, K): library workspace or caller buffer
    const void* B;          // (Nc, K)
    void* C;                // (M, Nc)
    int64_t M, Nc, K;
    // fused schedule
    const void* shards[kMaxShards];
    int nshards;
    int local_rank;         // tiles wholly inside this shard read it directly
    int64_t H;              // rows per shard
    int64_t cb;             // comm block rows
    uint32_t* flags;        // progress[nshards * S]
    uint32_t* done;         // per-chunk finished-piece counters (zeroed at the start of every call)
    uint32_t* ticket;       // [0] next fill piece, [1] next piece of the rest
    uint32_t* status;       // [code, chunk, tile, epoch of the failing call]
    uint32_t epoch;         // value a published flag holds during this call
    int copy_pieces;        // CopyBy
    int reverse_order;      // stress: hand pieces out back to front
    int64_t spin_limit;     // 100 MHz ticks of one flag wait before giving up
    int out_fp8;            // C is FP8 E4M3 "fn" bytes (else bf16)
    int in_fp8;             // A, B and the shards are FP8 E4M3 "fn" codes (else bf16)
    float out_scale;        // C = convert(acc * out_scale) with FP8 output or FP8 inputs (else 1)
    // GEMM + ReduceScatter (plain mode): tiles holding rows [pub_lo, pub_hi) of C store them
    // write-through and then count themselves in tile_done[tile row - pub_lo / BM]; the tile walk
    // starts at pub_lo.  nullptr: no publishing.
    uint32_t* tile_done;
    int64_t pub_lo, pub_hi;
    // measurement aid (fused schedule): nullptr, or 4 counters the GEMM adds to -- 100 MHz ticks its
    // workgroups spent waiting on chunk flags, waits, pieces copied by waiting workgroups, tiles
    // whose prefetched flags let them skip the wait
    uint64_t* wait_stats;
};

// --------------------------------------------------------------------- GEMM + ReduceScatter
// One rank's block of the ReduceScatter: out = sum over j of parts[j], (H, Nc) bf16 each, summed in
// fp32 in ascending j and rounded to bf16.  With tile_done, block row i waits until its tile row of
// the GEMM (row lo + i of P) has `target` finished tiles.
struct RsArgs {
    const void* parts[kMaxShards];
    void* out;
    int nparts;
    int64_t H, Nc;
    int64_t lo;             // first row of the block in the GEMM's C
    int64_t bm;             // GEMM tile rows
    uint32_t* tile_done;    // nullptr: no waits (the serial schedule)
    uint32_t target;        // tiles per tile row
    uint32_t* status;       // [code, chunk, tile, epoch of the failing call]
    uint32_t epoch;
    int64_t spin_limit;     // 100 MHz ticks of one wait
};

// wgs_per_cu: 1 beside the GEMM (room for one wave per SIMD), more when it runs alone
hipError_t launch_rs_reduce(const RsArgs& r, int wgs_per_cu, hipStream_t stream);

// Piece plan of one fused call.
struct FusedPlan {
    int64_t npieces;        // pieces the GEMM's counters hand out (0 if it copies nothing)
    int64_t fill_end;       // pieces [0, fill_end): every chunk the first wave of tiles reads
    int64_t nchunks;
};

FusedPlan plan_fused(const GemmArgs& a);

// Zeroes the per-chunk piece counts and sets the piece counters to 0 and fill_end.
hipError_t launch_reset(const GemmArgs& a, const FusedPlan& f, hipStream_t stream);

hipError_t launch_gemm(const GemmArgs& a, GemmMode mode, const FusedPlan* f, hipStream_t stream);

// Start of a side-stream fused call (in place of launch_reset): copies pieces [0, fill_end) with the
// whole GPU, raises their chunks' flags, starts both piece counters at fill_end and zeroes the
// per-chunk piece counts.
hipError_t launch_fill(const GemmArgs& a, const FusedPlan& f, hipStream_t stream);

// Copy kernel of the side-stream schedule: pieces [fill_end, npieces), beside the GEMM.  It never
// waits.
hipError_t launch_producer(const GemmArgs& a, const FusedPlan& f, hipStream_t stream);

hipError_t device_cus(int* out);

// Small helper kernel: p[0..n) = value (flag epochs, GEMM-only flags).
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t stream);

int gemm_tile_m();
int gemm_tile_n();

}  // namespace ag
