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
    uint32_t* ticket;       // [0] piece counter of the overlapped copy (producer and GEMM), [1] prologue's
    uint32_t* status;       // [code, chunk, tile, spins]
    uint32_t epoch;         // value a published flag holds during this call
    int copy_pieces;        // 1: the grid also performs the copy; 0: flags are already set
    int reverse_order;      // stress: claim pieces in reverse ready order
    int64_t spin_limit;     // polls of one flag before giving up
};

hipError_t launch_gemm(const GemmArgs& a, GemmMode mode, hipStream_t stream);

// Copy pieces of the fused schedule: piece q is position q / ppc in ready order, sub-range q % ppc
// of that chunk's rows.
int64_t copy_pieces_total(const GemmArgs& a);

// Pieces [0, n) hold every chunk that the first wave of GEMM tiles (one tile per workgroup of the
// persistent grid) reads from the aggregate buffer; 0 when that wave only reads the local shard.
int64_t first_wave_pieces(const GemmArgs& a);

// Copy kernel of the fused schedule: its workgroups claim pieces from `counter` until it reaches
// `end`, copy them and raise the chunk flags; at most `max_grid` workgroups.  It never waits.
// `alone`: nothing else runs meanwhile (deeper loads); otherwise it is sized to sit beside the GEMM.
hipError_t launch_producer(const GemmArgs& a, uint32_t* counter, int64_t end, int max_grid, bool alone,
                           hipStream_t stream);

// p[0] = v0, p[1] = v1 (one tiny kernel, safe to capture in a graph).
hipError_t launch_set_pair(uint32_t* p, uint32_t v0, uint32_t v1, hipStream_t stream);

hipError_t device_cus(int* out);

// Small helper kernel: flags[0..n) = value (used for the GEMM-only schedule and epoch wrap).
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t stream);

int gemm_tile_m();
int gemm_tile_n();

}  // namespace ag
