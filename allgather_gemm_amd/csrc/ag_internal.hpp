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
    uint32_t* done;         // per-chunk finished-piece counters
    uint32_t* ticket;       // [0] piece claim counter (shared by producer and GEMM)
    uint32_t* status;       // [code, chunk, tile, spins]
    uint32_t epoch;         // value a published flag holds during this call
    int copy_pieces;        // 1: the grid also performs the copy; 0: flags are already set
    int reverse_order;      // stress: claim pieces in reverse ready order
    int64_t spin_limit;     // polls of one flag before giving up
};

hipError_t launch_gemm(const GemmArgs& a, GemmMode mode, hipStream_t stream);

// Copy kernel of the fused schedule (all pieces, ready order); launch it on a side stream next to
// the fused GEMM.  The piece counter (ticket[0]) must be 0 when either kernel starts.
hipError_t launch_producer(const GemmArgs& a, hipStream_t stream);

// Small helper kernel: flags[0..n) = value (used for the GEMM-only schedule and epoch wrap).
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t stream);

int gemm_tile_m();
int gemm_tile_n();

}  // namespace ag
