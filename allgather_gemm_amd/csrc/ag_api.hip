// ag_api.hip -- host runtime behind the C ABI declared in include/aggemm.h: validation,
// per-device workspace, epochs of the progress flags, stream ordering, and launches.
#include "../../include/aggemm.h"
#include "ag_internal.hpp"
#include "ag_protocol.hpp"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

namespace ag {
namespace {

struct Workspace {
    void* a_agg = nullptr;       // aggregate A (M, K) bf16
    size_t a_bytes = 0;
    uint32_t* flags = nullptr;   // progress flags, one per chunk
    uint32_t* done = nullptr;    // finished pieces per chunk
    int64_t nflags = 0;
    uint32_t* ctl = nullptr;     // [0] fill piece counter, [1] piece counter of the rest, [4..7] status
    uint32_t epoch = 0;          // value of a raised flag in the last call
    hipEvent_t last = nullptr;   // completion of the last call that used this workspace
    bool used = false;
    hipStream_t side = nullptr;  // the fused schedule's copy stream (default priority)
    hipEvent_t fork = nullptr, join = nullptr;
};

std::mutex g_mu;
std::vector<Workspace> g_ws;
thread_local std::string t_err;

int hip_fail(hipError_t e, const char* what)
{
    t_err = std::string(what) + ": " + hipGetErrorString(e);
    return AG_EHIP;
}

#define AG_HIP(call, what)                     \
    do {                                       \
        hipError_t e_ = (call);                \
        if (e_ != hipSuccess)                  \
            return hip_fail(e_, what);         \
    } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int current_ws(Workspace** out)
{
    int dev = 0;
    AG_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0)
        return AG_EINVAL;
    if ((size_t)dev >= g_ws.size())
        g_ws.resize(dev + 1);
    Workspace& w = g_ws[dev];
    if (!w.ctl) {
        AG_HIP(hipMalloc(&w.ctl, 8 * sizeof(uint32_t)), "hipMalloc(control)");
        AG_HIP(hipMemset(w.ctl, 0, 8 * sizeof(uint32_t)), "hipMemset(control)");
        // The workspace's events only order this library's kernels against each other on this
        // device (every kernel's own end-of-kernel release makes its writes visible to later
        // kernels); nothing on the host waits on them.  Without the system-scope fences each of
        // their markers idles the GPU about 1 us less between kernels (about 5 instead of 6).
        const unsigned ev_flags = hipEventDisableTiming | hipEventDisableSystemFence;
        AG_HIP(hipEventCreateWithFlags(&w.last, ev_flags), "hipEventCreate");
        AG_HIP(hipEventCreateWithFlags(&w.fork, ev_flags), "hipEventCreate");
        AG_HIP(hipEventCreateWithFlags(&w.join, ev_flags), "hipEventCreate");
        AG_HIP(hipStreamCreateWithFlags(&w.side, hipStreamNonBlocking), "hipStreamCreate");
    }
    *out = &w;
    return AG_OK;
}

// Grows are rare; they wait for the device so no in-flight kernel still uses the old buffers.
int ensure_flags(Workspace& w, int64_t n)
{
    if (n <= w.nflags)
        return AG_OK;
    AG_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize(grow flags)");
    if (w.flags)
        AG_HIP(hipFree(w.flags), "hipFree(flags)");
    if (w.done)
        AG_HIP(hipFree(w.done), "hipFree(done)");
    w.flags = w.done = nullptr;
    w.nflags = 0;
    const int64_t cap = n < 1024 ? 1024 : n;
    if (hipMalloc(&w.flags, cap * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc(&w.done, cap * sizeof(uint32_t)) != hipSuccess)
        return AG_ENOMEM;
    AG_HIP(hipMemset(w.flags, 0, cap * sizeof(uint32_t)), "hipMemset(flags)");
    AG_HIP(hipMemset(w.done, 0, cap * sizeof(uint32_t)), "hipMemset(done)");
    w.nflags = cap;
    w.epoch = 0;   // fresh flags are all 0, so any epoch >= 1 is new
    return AG_OK;
}

int ensure_a(Workspace& w, size_t bytes)
{
    if (bytes <= w.a_bytes)
        return AG_OK;
    AG_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize(grow A)");
    if (w.a_agg)
        AG_HIP(hipFree(w.a_agg), "hipFree(A)");
    w.a_agg = nullptr;
    w.a_bytes = 0;
    if (hipMalloc(&w.a_agg, bytes) != hipSuccess)
        return AG_ENOMEM;
    w.a_bytes = bytes;
    return AG_OK;
}

// Next flag value; on wrap-around the flags and the give-up word are cleared so an old value cannot
// match.
int next_epoch(Workspace& w, hipStream_t s)
{
    if (++w.epoch == 0) {
        AG_HIP(launch_fill_u32(w.flags, w.nflags, 0u, s), "fill flags");
        AG_HIP(launch_fill_u32(w.ctl + 7, 1, 0u, s), "clear give-up epoch");
        w.epoch = 1;
    }
    return AG_OK;
}

int begin_use(Workspace& w, hipStream_t s)
{
    if (w.used)
        AG_HIP(hipStreamWaitEvent(s, w.last, 0), "hipStreamWaitEvent");
    return AG_OK;
}

int end_use(Workspace& w, hipStream_t s)
{
    AG_HIP(hipEventRecord(w.last, s), "hipEventRecord");
    w.used = true;
    return AG_OK;
}

int validate_gemm(const void* const* shards, int32_t N, int64_t M, int64_t K, const void* B,
                  int64_t Nc, void* C, int64_t cb, const ag_options* opt)
{
    if (!shards || N < 1 || N > kMaxShards || M < 0 || K < 0 || Nc < 0 || cb < 1)
        return AG_EINVAL;
    if (M % N != 0 || K % 8 != 0)
        return AG_EINVAL;
    if (K > (int64_t(1) << 21))
        return AG_EUNSUPPORTED;
    if (opt) {
        if (opt->mode < AG_MODE_FUSED || opt->mode > AG_MODE_PLAIN_GEMM || opt->local_rank < 0 ||
            opt->local_rank >= N || opt->skip_producer < 0 || opt->skip_producer > 1 ||
            opt->producer < AG_PRODUCER_SIDE_STREAM || opt->producer > AG_PRODUCER_COPY_ENGINE)
            return AG_EINVAL;
        if ((opt->mode == AG_MODE_GEMM_ONLY || opt->mode == AG_MODE_PLAIN_GEMM) && !opt->a_out)
            return AG_EINVAL;
        if (opt->out_dtype != AG_OUT_BF16 && opt->out_dtype != AG_OUT_FP8_E4M3)
            return AG_EINVAL;
        if (opt->in_dtype != AG_IN_BF16 && opt->in_dtype != AG_IN_FP8_E4M3)
            return AG_EINVAL;
        if (opt->in_dtype == AG_IN_FP8_E4M3 && K % 16 != 0)
            return AG_EINVAL;   // rows of whole 16-byte chunks
        if (!std::isfinite(opt->out_scale))
            return AG_EINVAL;
        if (opt->a_out && !aligned16(opt->a_out))
            return AG_EINVAL;
    }
    if (M == 0 || Nc == 0)
        return AG_OK;
    if (!C || !aligned16(C))
        return AG_EINVAL;
    if (K > 0) {   // with K == 0 nothing is read, so empty inputs may have null pointers
        if (!B || !aligned16(B))
            return AG_EINVAL;
        for (int r = 0; r < N; ++r)
            if (!shards[r] || !aligned16(shards[r]))
                return AG_EINVAL;
    }
    const int64_t H = M / N;
    const int64_t chunks = (int64_t)N * ((H + cb - 1) / cb);
    if (chunks > (int64_t(1) << 30))
        return AG_EUNSUPPORTED;
    return AG_OK;
}

// ----------------------------------------------------------------- ag_gemm_noalloc's control words
// One fixed array per GPU: [0] fill piece counter, [1] piece counter of the rest, [4..7] status,
// [8, 8 + max) progress flags, [8 + max, 8 + 2 max) piece counts.  Zero when the code object is
// loaded.  Host code never uses the symbol itself (on the host it is only a stand-in): the device
// address comes from hipGetSymbolAddress, once per device, on that device's first call.
constexpr int64_t kNoAllocChunks = AG_NOALLOC_MAX_CHUNKS;
constexpr int64_t kScratchWords = 8 + 2 * kNoAllocChunks;
static __device__ __align__(256) uint32_t scratch[kScratchWords];

constexpr int kMaxDevicesNoAlloc = 64;
struct NoAllocState {
    uint32_t* words = nullptr;   // device address of `scratch` on this device
    uint32_t epoch = 0;          // value of a raised flag in the last call on this device
};
NoAllocState g_na[kMaxDevicesNoAlloc];

int noalloc_state(NoAllocState** out)
{
    int dev = 0;
    AG_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevicesNoAlloc) {
        t_err = "ag_gemm_noalloc: device index beyond the library's table";
        return AG_EUNSUPPORTED;
    }
    NoAllocState& st = g_na[dev];
    if (!st.words) {
        void* p = nullptr;
        AG_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        st.words = static_cast<uint32_t*>(p);
    }
    *out = &st;
    return AG_OK;
}

// Launches the GEMM kernel, bracketed by the caller's measurement events when it asked for them.
int gemm_timed(const GemmArgs& g, GemmMode mode, const FusedPlan* f, hipStream_t s, const ag_options* opt)
{
    if (opt && opt->gemm_events[0])
        AG_HIP(hipEventRecord(static_cast<hipEvent_t>(opt->gemm_events[0]), s), "hipEventRecord(gemm start)");
    AG_HIP(launch_gemm(g, mode, f, s), "launch gemm");
    if (opt && opt->gemm_events[1])
        AG_HIP(hipEventRecord(static_cast<hipEvent_t>(opt->gemm_events[1]), s), "hipEventRecord(gemm end)");
    return AG_OK;
}

}  // namespace
}  // namespace ag

using namespace ag;

extern "C" int ag_gemm_ex(const void* const* shards, int32_t N, int64_t M, int64_t K, const void* B,
                          int64_t Nc, void* C, int64_t comm_block_rows, void* stream,
                          const ag_options* opt)
{
    int rc = validate_gemm(shards, N, M, K, B, Nc, C, comm_block_rows, opt);
    if (rc != AG_OK || M == 0 || Nc == 0)
        return rc;
    const int mode = opt ? opt->mode : AG_MODE_FUSED;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_mu);
    Workspace* w = nullptr;
    if ((rc = current_ws(&w)) != AG_OK)
        return rc;
    const int64_t H = M / N;
    const int64_t S = (H + comm_block_rows - 1) / comm_block_rows;
    const int64_t nchunks = (int64_t)N * S;
    const bool in_fp8 = opt && opt->in_dtype == AG_IN_FP8_E4M3;
    const int64_t esize = in_fp8 ? 1 : 2;   // bytes per element of the shards, B and A
    void* a_buf = opt ? opt->a_out : nullptr;
    if (!a_buf && K > 0) {
        if ((rc = ensure_a(*w, (size_t)(M * K * esize))) != AG_OK)
            return rc;
        a_buf = w->a_agg;
    }
    if ((rc = ensure_flags(*w, nchunks)) != AG_OK)
        return rc;
    if ((rc = begin_use(*w, s)) != AG_OK)
        return rc;

    GemmArgs g;
    std::memset(&g, 0, sizeof g);
    g.A = a_buf;
    g.B = B;
    g.C = C;
    g.M = M;
    g.Nc = Nc;
    g.K = K;
    for (int r = 0; r < N; ++r)
        g.shards[r] = shards[r];
    g.nshards = N;
    g.local_rank = opt ? opt->local_rank : 0;
    g.H = H;
    g.cb = comm_block_rows;
    g.flags = w->flags;
    g.done = w->done;
    g.ticket = w->ctl;
    g.status = w->ctl + 4;
    const int64_t timeout_us = (opt && opt->timeout_us > 0) ? opt->timeout_us : 10000000;
    g.spin_limit = timeout_us * 100;   // s_memrealtime runs at 100 MHz
    g.reverse_order = opt ? opt->reverse_order : 0;
    g.wait_stats = opt ? static_cast<uint64_t*>(opt->wait_stats) : nullptr;
    g.out_fp8 = (opt && opt->out_dtype == AG_OUT_FP8_E4M3) ? 1 : 0;
    g.in_fp8 = in_fp8 ? 1 : 0;
    g.out_scale = ((g.out_fp8 || g.in_fp8) && opt->out_scale != 0.0f) ? opt->out_scale : 1.0f;

    if (K == 0) {
        // empty reduction: C = 0, nothing to gather
        if ((rc = gemm_timed(g, kGemmPlain, nullptr, s, opt)) != AG_OK)
            return rc;
        return end_use(*w, s);
    }
    if (mode == AG_MODE_PLAIN_GEMM) {
        if ((rc = gemm_timed(g, kGemmPlain, nullptr, s, opt)) != AG_OK)
            return rc;
        return end_use(*w, s);
    }
    if (mode == AG_MODE_UNFUSED) {
        GatherDesc d;
        std::memset(&d, 0, sizeof d);
        for (int r = 0; r < N; ++r)
            d.src[r] = shards[r];
        d.dst = a_buf;
        d.nranks = N;
        d.elem_size = (int)esize;
        d.planes = 1;
        d.H = H;
        d.W = K;
        d.dst_rows = M;
        d.valid_rows = H;
        d.valid_cols = K;
        AG_HIP(launch_tgather(d, s), "launch tgather");
        if ((rc = gemm_timed(g, kGemmPlain, nullptr, s, opt)) != AG_OK)
            return rc;
        return end_use(*w, s);
    }
    if ((rc = next_epoch(*w, s)) != AG_OK)
        return rc;
    g.epoch = w->epoch;
    const int producer = opt ? opt->producer : AG_PRODUCER_SIDE_STREAM;
    if (mode == AG_MODE_GEMM_ONLY || (opt && opt->skip_producer)) {
        // every flag raised beforehand (GEMM-only), or none ever (test of the give-up path)
        if (mode == AG_MODE_GEMM_ONLY)
            AG_HIP(launch_fill_u32(w->flags, nchunks, g.epoch, s), "fill flags");
        g.copy_pieces = kCopyNone;
        if ((rc = gemm_timed(g, kGemmFused, nullptr, s, opt)) != AG_OK)
            return rc;
    } else if (producer == AG_PRODUCER_IN_KERNEL) {
        g.copy_pieces = kCopyInKernel;
        const FusedPlan f = plan_fused(g);
        AG_HIP(launch_reset(g, f, s), "reset piece counters");
        if ((rc = gemm_timed(g, kGemmFused, &f, s, opt)) != AG_OK)
            return rc;
    } else if (producer == AG_PRODUCER_SIDE_STREAM) {
        // the first wave's chunks are copied by the whole GPU before the GEMM starts (the same
        // kernel resets the call's counters); the rest by a copy kernel on the side stream while
        // the GEMM runs (waiting tiles help); the call ends when both kernels have
        g.copy_pieces = kCopyWaiters;
        const FusedPlan f = plan_fused(g);
        AG_HIP(launch_fill(g, f, s), "launch fill copy");
        AG_HIP(hipEventRecord(w->fork, s), "hipEventRecord(fork)");
        AG_HIP(hipStreamWaitEvent(w->side, w->fork, 0), "hipStreamWaitEvent(side)");
        AG_HIP(launch_producer(g, f, w->side), "launch producer");
        if ((rc = gemm_timed(g, kGemmFused, &f, s, opt)) != AG_OK)
            return rc;
        AG_HIP(hipEventRecord(w->join, w->side), "hipEventRecord(join)");
        AG_HIP(hipStreamWaitEvent(s, w->join, 0), "hipStreamWaitEvent(join)");
    } else {
        // copy engines: per chunk in ready order, a copy that uses no compute units, then the
        // chunk's flag written by the stream once the copy has completed
        g.copy_pieces = kCopyNone;
        AG_HIP(hipEventRecord(w->fork, s), "hipEventRecord(fork)");
        AG_HIP(hipStreamWaitEvent(w->side, w->fork, 0), "hipStreamWaitEvent(side)");
        if ((rc = gemm_timed(g, kGemmFused, nullptr, s, opt)) != AG_OK)
            return rc;
        const PieceMap pm = pm_make(H, comm_block_rows, N, g.local_rank, K * esize, gemm_tile_m(), 1);
        for (int64_t pos = 0; pos < pm.nchunks; ++pos) {
            const int64_t c = pm_ready_chunk(pm, pos);
            int64_t first = 0, last = 0;
            pm_chunk_rows(pm, c, first, last);
            const int64_t r = c / pm.S;
            const char* src = static_cast<const char*>(shards[r]) + (first - r * H) * K * esize;
            char* dst = static_cast<char*>(a_buf) + first * K * esize;
            AG_HIP(hipMemcpyAsync(dst, src, (size_t)((last - first) * K * esize), hipMemcpyDeviceToDeviceNoCU,
                                  w->side), "hipMemcpyAsync(copy engine)");
            AG_HIP(hipStreamWriteValue32(w->side, w->flags + c, g.epoch, 0), "hipStreamWriteValue32(flag)");
        }
        AG_HIP(hipEventRecord(w->join, w->side), "hipEventRecord(join)");
        AG_HIP(hipStreamWaitEvent(s, w->join, 0), "hipStreamWaitEvent(join)");
    }
    return end_use(*w, s);
}

extern "C" int ag_gemm(const void* const* shards, int32_t N, int64_t M, int64_t K, const void* B,
                       int64_t Nc, void* C, int64_t comm_block_rows, void* stream)
{
    return ag_gemm_ex(shards, N, M, K, B, Nc, C, comm_block_rows, stream, nullptr);
}

extern "C" int ag_gemm_unfused(const void* const* shards, int32_t N, int64_t M, int64_t K,
                               const void* B, int64_t Nc, void* C, int64_t comm_block_rows,
                               void* stream)
{
    ag_options o;
    std::memset(&o, 0, sizeof o);
    o.mode = AG_MODE_UNFUSED;
    return ag_gemm_ex(shards, N, M, K, B, Nc, C, comm_block_rows, stream, &o);
}

extern "C" int tgather_ex(const void* const* shards, int32_t N, void* dst, int64_t D0, int64_t D1,
                          int64_t D2, int64_t H, int64_t W, int64_t dst_rows, int64_t valid_rows,
                          int64_t valid_cols, int32_t elem_size, int32_t root, void* stream)
{
    if (!shards || N < 1 || N > kMaxShards || D0 < 0 || D1 < 0 || D2 < 0 || H < 0 || W < 0)
        return AG_EINVAL;
    if (root < 0 || root >= N)
        return AG_EINVAL;
    if (valid_rows < 1 || valid_cols < 1)
        return AG_EINVAL;
    if (!(elem_size == 1 || elem_size == 2 || elem_size == 4 || elem_size == 8))
        return AG_EINVAL;
    if (dst_rows < (int64_t)N * H)
        return AG_EINVAL;
    if (D0 == 0 || D1 == 0 || D2 == 0 || H == 0 || W == 0)
        return AG_OK;                                   // nothing moves
    if (!dst)
        return AG_EINVAL;
    for (int r = 0; r < N; ++r)
        if (!shards[r])
            return AG_EINVAL;
    GatherDesc d;
    std::memset(&d, 0, sizeof d);
    for (int r = 0; r < N; ++r)
        d.src[r] = shards[r];
    d.dst = dst;
    d.nranks = N;
    d.elem_size = elem_size;
    d.planes = D0 * D1 * D2;
    d.H = H;
    d.W = W;
    d.dst_rows = dst_rows;
    d.valid_rows = valid_rows;
    d.valid_cols = valid_cols;
    AG_HIP(launch_tgather(d, static_cast<hipStream_t>(stream)), "launch tgather");
    return AG_OK;
}

extern "C" int tgather(const void* const* shards, int32_t N, void* dst, int64_t D0, int64_t D1,
                       int64_t D2, int64_t H, int64_t W, int64_t valid_rows, int64_t valid_cols,
                       int32_t elem_size, void* stream)
{
    return tgather_ex(shards, N, dst, D0, D1, D2, H, W, (int64_t)N * H, valid_rows, valid_cols,
                      elem_size, 0, stream);
}

extern "C" int gemm_rs(const void* A, const void* B, int32_t N, int32_t local_rank, int64_t M, int64_t Nc,
                       int64_t K, const void* const* recv, void* P, void* out, int32_t mode, void* stream)
{
    if (N < 1 || N > kMaxShards || local_rank < 0 || local_rank >= N || M < 0 || Nc < 0 || K < 0)
        return AG_EINVAL;
    if (M % N != 0 || K % 8 != 0 || Nc % 8 != 0 || (mode != AG_RS_FUSED && mode != AG_RS_UNFUSED))
        return AG_EINVAL;
    if (K > (int64_t(1) << 21) || Nc * 32 * 2 > (int64_t(1) << 32))
        return AG_EUNSUPPORTED;
    if (M == 0 || Nc == 0)
        return AG_OK;
    const int64_t H = M / N;
    if (!recv || !P || !out || !aligned16(P) || !aligned16(out))
        return AG_EINVAL;
    if (K > 0 && (!A || !B || !aligned16(A) || !aligned16(B)))
        return AG_EINVAL;
    for (int j = 0; j < N; ++j)
        if (j != local_rank && (!recv[j] || !aligned16(recv[j])))
            return AG_EINVAL;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_mu);
    Workspace* w = nullptr;
    int rc;
    if ((rc = current_ws(&w)) != AG_OK)
        return rc;
    const int64_t bm = gemm_tile_m();
    const int64_t lo = (int64_t)local_rank * H, hi = lo + H;
    const int64_t nrows = H > 0 ? (hi - 1) / bm - lo / bm + 1 : 0;   // GEMM tile rows meeting the block
    if ((rc = ensure_flags(*w, nrows)) != AG_OK)
        return rc;
    if ((rc = begin_use(*w, s)) != AG_OK)
        return rc;
    if ((rc = next_epoch(*w, s)) != AG_OK)
        return rc;

    GemmArgs g;
    std::memset(&g, 0, sizeof g);
    g.A = A;
    g.B = B;
    g.C = P;
    g.M = M;
    g.Nc = Nc;
    g.K = K;
    g.nshards = 1;
    g.H = M;
    g.cb = M > 0 ? M : 1;
    g.status = w->ctl + 4;
    g.out_scale = 1.0f;

    RsArgs r;
    std::memset(&r, 0, sizeof r);
    for (int j = 0; j < N; ++j)
        r.parts[j] = j == local_rank ? static_cast<const void*>(static_cast<const char*>(P) + lo * Nc * 2) : recv[j];
    r.out = out;
    r.nparts = N;
    r.H = H;
    r.Nc = Nc;
    r.lo = lo;
    r.bm = bm;
    r.target = (uint32_t)((Nc + gemm_tile_n() - 1) / gemm_tile_n());
    r.status = w->ctl + 4;
    r.epoch = w->epoch;
    r.spin_limit = (int64_t)10000000 * 100;   // 10 s of the 100 MHz clock

    if (mode == AG_RS_UNFUSED || H == 0) {
        AG_HIP(launch_gemm(g, kGemmPlain, nullptr, s), "launch gemm");
        AG_HIP(launch_rs_reduce(r, 4, s), "launch reduce");
        return end_use(*w, s);
    }
    // fused: tile-row counts start at zero; the reduction waits on them from a second stream.  They
    // live in the piece-count array, which every call that uses it zeroes first (the progress
    // flags hold epochs and must never hold a count).
    g.tile_done = w->done;
    g.pub_lo = lo;
    g.pub_hi = hi;
    r.tile_done = w->done;
    AG_HIP(launch_fill_u32(w->done, nrows, 0u, s), "clear tile counts");
    AG_HIP(hipEventRecord(w->fork, s), "hipEventRecord(fork)");
    AG_HIP(hipStreamWaitEvent(w->side, w->fork, 0), "hipStreamWaitEvent(side)");
    AG_HIP(launch_rs_reduce(r, 1, w->side), "launch reduce");
    AG_HIP(launch_gemm(g, kGemmPlain, nullptr, s), "launch gemm");
    AG_HIP(hipEventRecord(w->join, w->side), "hipEventRecord(join)");
    AG_HIP(hipStreamWaitEvent(s, w->join, 0), "hipStreamWaitEvent(join)");
    return end_use(*w, s);
}

extern "C" int ag_gemm_noalloc(const void* const* shards, int32_t N, int64_t M, int64_t K, const void* B,
                               int64_t Nc, void* C, int64_t comm_block_rows, void* a_out, int32_t local_rank,
                               void* stream)
{
    ag_options o;
    std::memset(&o, 0, sizeof o);
    o.mode = AG_MODE_FUSED;
    o.local_rank = local_rank;
    o.a_out = a_out;
    o.producer = AG_PRODUCER_IN_KERNEL;
    int rc = validate_gemm(shards, N, M, K, B, Nc, C, comm_block_rows, &o);
    if (rc != AG_OK || M == 0 || Nc == 0)
        return rc;
    if (K > 0 && !a_out)
        return AG_EINVAL;
    const int64_t H = M / N;
    const int64_t nchunks = (int64_t)N * ((H + comm_block_rows - 1) / comm_block_rows);
    if (nchunks > kNoAllocChunks) {
        t_err = "ag_gemm_noalloc: " + std::to_string(nchunks) + " chunks, at most " +
                std::to_string(kNoAllocChunks);
        return AG_EUNSUPPORTED;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_mu);
    NoAllocState* st = nullptr;
    if ((rc = noalloc_state(&st)) != AG_OK)
        return rc;

    GemmArgs g;
    std::memset(&g, 0, sizeof g);
    g.A = a_out;
    g.B = B;
    g.C = C;
    g.M = M;
    g.Nc = Nc;
    g.K = K;
    for (int r = 0; r < N; ++r)
        g.shards[r] = shards[r];
    g.nshards = N;
    g.local_rank = local_rank;
    g.H = H;
    g.cb = comm_block_rows;
    g.ticket = st->words;
    g.status = st->words + 4;
    g.flags = st->words + 8;
    g.done = st->words + 8 + kNoAllocChunks;
    g.spin_limit = (int64_t)10000000 * 100;   // 10 s of the 100 MHz clock
    g.out_fp8 = 0;
    g.out_scale = 1.0f;
    if (K == 0) {
        AG_HIP(launch_gemm(g, kGemmPlain, nullptr, s), "launch gemm");   // C = 0
        return AG_OK;
    }
    // A new flag value per call; on wrap-around the flags and the give-up word are cleared (by a
    // kernel: no memset node if the caller captures this into a graph).
    if (++st->epoch == 0) {
        AG_HIP(launch_fill_u32(g.flags, kNoAllocChunks, 0u, s), "clear flags");
        AG_HIP(launch_fill_u32(g.status + 3, 1, 0u, s), "clear give-up epoch");
        st->epoch = 1;
    }
    g.epoch = st->epoch;
    g.copy_pieces = kCopyInKernel;
    const FusedPlan f = plan_fused(g);
    AG_HIP(launch_reset(g, f, s), "reset piece counters");   // piece counts and counters start at 0
    AG_HIP(launch_gemm(g, kGemmFused, &f, s), "launch gemm");
    return AG_OK;
}

// Reads one status block; if it holds a failure, reports it and clears it.
static int take_status(uint32_t* block, int64_t info[4], bool* failed)
{
    uint32_t st[4] = {0, 0, 0, 0};
    AG_HIP(hipMemcpy(st, block, sizeof st, hipMemcpyDeviceToHost), "hipMemcpy(status)");
    *failed = st[0] != 0;
    if (!*failed)
        return AG_OK;
    if (info)
        for (int i = 0; i < 4; ++i)
            info[i] = st[i];
    // the reported failure is consumed; counters need no repair (every call resets its own)
    AG_HIP(hipMemset(block, 0, 3 * sizeof(uint32_t)), "hipMemset(status)");
    return AG_OK;
}

extern "C" int ag_check(void* stream, int64_t info[4])
{
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    AG_HIP(hipGetDevice(&dev), "hipGetDevice");
    AG_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "hipStreamSynchronize");
    if (info)
        for (int i = 0; i < 4; ++i)
            info[i] = 0;
    bool failed = false;
    int rc;
    if (dev >= 0 && (size_t)dev < g_ws.size() && g_ws[dev].ctl) {
        if ((rc = take_status(g_ws[dev].ctl + 4, info, &failed)) != AG_OK)
            return rc;
        if (failed)
            return AG_ETIMEOUT;
    }
    if (dev >= 0 && dev < kMaxDevicesNoAlloc && g_na[dev].words) {
        if ((rc = take_status(g_na[dev].words + 4, info, &failed)) != AG_OK)
            return rc;
        if (failed)
            return AG_ETIMEOUT;
    }
    return AG_OK;
}

extern "C" const char* ag_status_str(int status)
{
    switch (status) {
    case AG_OK: return "ok";
    case AG_EINVAL: return "invalid argument";
    case AG_ENOMEM: return "out of device memory";
    case AG_EHIP: return "HIP runtime error";
    case AG_ETIMEOUT: return "timed out waiting on a chunk flag";
    case AG_EUNSUPPORTED: return "unsupported shape";
    default: return "unknown status";
    }
}

extern "C" const char* ag_last_error(void) { return t_err.c_str(); }

extern "C" void ag_finalize(void)
{
    std::lock_guard<std::mutex> lock(g_mu);
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess)
        return;
    for (size_t dev = 0; dev < g_ws.size(); ++dev) {
        Workspace& w = g_ws[dev];
        if (!w.ctl)
            continue;
        if (hipSetDevice((int)dev) != hipSuccess)
            continue;
        (void)hipDeviceSynchronize();
        (void)hipFree(w.a_agg);
        (void)hipFree(w.flags);
        (void)hipFree(w.done);
        (void)hipFree(w.ctl);
        (void)hipEventDestroy(w.last);
        (void)hipEventDestroy(w.fork);
        (void)hipEventDestroy(w.join);
        (void)hipStreamDestroy(w.side);
        w = Workspace();
    }
    (void)hipSetDevice(prev);
}
