// rs.hip -- the reducing side of GEMM + ReduceScatter on gfx950: one rank's block of the
// ReduceScatter, out = sum over ranks j of parts[j], for the row block this rank keeps.
//
// "Triton第四课：基于对称内存融合 AllGather 与 MatMul，提速1.56倍", section 从集合通信理解数据流:
// ReduceScatter reduces every rank's copy of a block and leaves block r with rank r; it mirrors the
// AllGather the MatMul consumes.  Fused with the GEMM that produces this rank's own partial, the
// reduction of a block row starts as soon as the GEMM tiles of that row are complete (counted in
// tile_done by the GEMM, the same kind of per-block progress signal as the AllGather's chunk flags)
// instead of after the whole GEMM.
//
// One workgroup of 256 threads per block row (grid-strided, rows in increasing order), 8 columns
// per lane: the N parts' 16-byte vectors are loaded first (all in flight), then summed in fp32 in
// ascending rank order and rounded to bf16 (nearest even).  The kernel is small -- no LDS tile, few
// VGPRs -- so beside the GEMM one workgroup per CU fits next to the GEMM's; alone, after the GEMM,
// it runs four per CU.
#include "ag_device.hpp"
#include "ag_internal.hpp"

#include <algorithm>

namespace ag {
namespace {

constexpr int NT = 256;
constexpr int BATCH = 8;                 // parts loaded together

// Wave 0 of the workgroup: wait until tile row `chunk` of the GEMM is complete, then a barrier.
// Gives up after spin_limit ticks of the 100 MHz clock (reported in the status block; the rest of
// the call's waits then return at once).
__device__ void wait_tile_row(const RsArgs& r, int64_t chunk, bool wave0, int32_t* s_ok)
{
    if (wave0) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        int32_t ok = 1;
        for (;;) {
            if (__builtin_amdgcn_readfirstlane(flag_peek(&r.tile_done[chunk])) >= r.target)
                break;
            if (__builtin_amdgcn_readfirstlane(flag_peek(&r.status[3])) == r.epoch) {
                ok = 0;
                break;
            }
            if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > r.spin_limit) {
                report_failure(r.status, 2u, (uint32_t)chunk, 0u, r.epoch);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if ((threadIdx.x & 63) == 0)
            *s_ok = ok;
    }
    barrier_after_lds_write();
    // rows that are not whole 128-byte lines share a line with the next tile row: such a line may
    // have been cached before that row was written, so the L2 is invalidated
    if ((r.Nc * 2) % 128 != 0)
        acquire_agent();
}

// SMALL: at most BATCH parts, whose pointers are read once, before the loops (otherwise each load
// waits for a scalar load of its pointer, indexed at run time).
template <bool SMALL>
__global__ __launch_bounds__(NT) void rs_reduce_kernel(RsArgs r)
{
    __shared__ int32_t s_ok;
    const __bf16* pp[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
        pp[b] = static_cast<const __bf16*>(r.parts[SMALL && b < r.nparts ? b : 0]);
    const int tid = threadIdx.x;
    const bool wave0 = __builtin_amdgcn_readfirstlane(tid >> 6) == 0;
    const int64_t first_chunk = r.lo / r.bm;
    int64_t ready = -1;     // tile row this workgroup last saw complete (rows come in order)
    bool failed = false;
    for (int64_t i = blockIdx.x; i < r.H; i += gridDim.x) {
        if (r.tile_done && !failed) {
            const int64_t chunk = (r.lo + i) / r.bm - first_chunk;
            if (chunk != ready) {
                wait_tile_row(r, chunk, wave0, &s_ok);
                failed = __builtin_amdgcn_readfirstlane(s_ok) == 0;
                ready = chunk;
            }
        }
        const int64_t row = i * r.Nc;
        for (int64_t c = (int64_t)tid * 8; c < r.Nc; c += NT * 8) {
            float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int j0 = 0; j0 < r.nparts; j0 += BATCH) {
                bf16x8 v[BATCH];
#pragma unroll
                for (int b = 0; b < BATCH; ++b)
                    if (j0 + b < r.nparts)
                        v[b] = *reinterpret_cast<const bf16x8*>(
                            (SMALL ? pp[b] : static_cast<const __bf16*>(r.parts[j0 + b])) + row + c);
#pragma unroll
                for (int b = 0; b < BATCH; ++b)
                    if (j0 + b < r.nparts)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            s[e] += (float)v[b][e];
            }
            bf16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[e] = (__bf16)s[e];
            *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(r.out) + row + c) = o;
        }
    }
}

int g_num_cus = 0;

}  // namespace

hipError_t launch_rs_reduce(const RsArgs& r, int wgs_per_cu, hipStream_t stream)
{
    if (r.H <= 0 || r.Nc <= 0)
        return hipSuccess;
    if (g_num_cus == 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return e;
        e = hipDeviceGetAttribute(&g_num_cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
    }
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(r.H, (int64_t)g_num_cus * wgs_per_cu));
    if (r.nparts <= BATCH)
        rs_reduce_kernel<true><<<grid, NT, 0, stream>>>(r);
    else
        rs_reduce_kernel<false><<<grid, NT, 0, stream>>>(r);
    return hipGetLastError();
}

}  // namespace ag
