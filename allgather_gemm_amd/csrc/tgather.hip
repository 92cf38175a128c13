// tgather.hip -- TGATHER on gfx950: the root concatenates N ranks' (D0,D1,D2,H,W) tensors along
// DIM_3 into dst (D0,D1,D2,dst_rows,W).
//
// Follows "CANN PTO-ISA TGATHER 指令深度解析：跨 Rank 行拼接 Gather 的实现原理与开发指南":
//  * section 二 数学语义: dst[d0,d1,d2, r*H + i, j] = src_r[d0,d1,d2, i, j];
//  * section 三 数据路径: data moves global -> on-chip staging tile -> global;
//  * section 6.1: the outer dims D0..D2 are walked explicitly, and each rank's (H, W) plane is cut
//    into logical tiles of valid_rows x valid_cols that slide over rows and columns, the last row
//    and column tiles being ragged (the DYNAMIC valid-extent case); the ping/pong path overlaps the
//    load of the next staging tile with the store of the current one;
//  * section 7.2: rows of dst at or beyond N*H are never written; section 7.4: empty shapes move
//    nothing.
// On gfx950 the staging tile is a workgroup's registers: each logical tile is moved as a sequence
// of sub-tiles of NT * UPT * 16 bytes, a sub-tile being loaded whole into VGPRs (16 bytes per load,
// UPT loads per lane in flight) and then stored.  UPT is 8 (32 KiB sub-tiles), or 12 (48 KiB) when
// that packs the rows fuller -- a row of 0.6 of the smaller sub-tile leaves 40 % of every lane's
// loads idle.  The sub-tiles of all tiles of all ranks and
// planes form one index space that the grid walks with a stride; the load/store overlap of the
// ping/pong scheme comes from the many workgroups resident on each CU, whose loads run while
// others store.  An LDS hop would add traffic and buy nothing for a copy.  The copy is byte-exact
// for every element size.
#include "ag_device.hpp"
#include "ag_internal.hpp"

#include <algorithm>

namespace ag {
namespace {

constexpr int NT = 256;
constexpr int UPT_SMALL = 8, UPT_LARGE = 12;  // 16-byte units per lane per sub-tile (32 / 48 KiB)
constexpr int WG_PER_CU = 16;

// A rectangular family of identical logical tiles inside one (rank, plane) region: the full
// tiles, the ragged last column, the ragged last row, and the ragged corner.
struct TileClass {
    int64_t count;     // tiles in the class
    int64_t ncols;     // tiles per row of the class's grid
    int64_t row0, col0;
    int64_t th, tw;    // tile height (rows) and width (elements)
    int64_t sr;        // rows per sub-tile
    int64_t scn;       // column pieces per tile row
    int64_t scw;       // elements per column piece (last may be shorter)
    int64_t subs;      // sub-tiles per tile
    int64_t first;     // first sub-tile of the class inside the region
};

struct Plan {
    GatherDesc d;
    int64_t sub_bytes;  // bytes per sub-tile, NT * UPT * 16
    TileClass cls[4];
    int ncls;
    int64_t subs_per_region;
    int64_t total;
    int vec;           // 1: 16-byte path; 0: element path
};

struct SubTile {
    const char* src;   // first byte of row 0 of the sub-tile (column start included)
    char* dst;
    int64_t rows;
    int64_t bytes;     // bytes per row
    int64_t pitch;     // row pitch (W * elem_size), same in src and dst
};

__device__ __forceinline__ SubTile locate(const Plan& P, int64_t q)
{
    const GatherDesc& d = P.d;
    const int64_t region = q / P.subs_per_region;
    int64_t rem = q - region * P.subs_per_region;
    const int r = (int)(region / d.planes);
    const int64_t plane = region - (int64_t)r * d.planes;
    int ci = 0;
#pragma unroll
    for (int k = 1; k < 4; ++k)
        if (k < P.ncls && rem >= P.cls[k].first)
            ci = k;
    const TileClass& c = P.cls[ci];
    rem -= c.first;
    const int64_t ti = rem / c.subs;
    const int64_t st = rem - ti * c.subs;
    const int64_t tr = ti / c.ncols, tc = ti - tr * c.ncols;
    const int64_t rs = st / c.scn, cs = st - rs * c.scn;
    const int64_t tile_r0 = c.row0 + tr * c.th, tile_c0 = c.col0 + tc * c.tw;
    const int64_t r0 = tile_r0 + rs * c.sr;
    const int64_t rows = min(c.sr, tile_r0 + c.th - r0);
    const int64_t c0 = tile_c0 + cs * c.scw;
    const int64_t cols = min(c.scw, tile_c0 + c.tw - c0);
    const int64_t esz = d.elem_size;
    SubTile s;
    s.pitch = d.W * esz;
    s.src = static_cast<const char*>(d.src[r]) + ((plane * d.H + r0) * d.W + c0) * esz;
    s.dst = static_cast<char*>(d.dst) + ((plane * d.dst_rows + (int64_t)r * d.H + r0) * d.W + c0) * esz;
    s.rows = rows;
    s.bytes = cols * esz;
    return s;
}

// Interior of a row segment that is 16-byte aligned in absolute address (the same offset in src
// and dst, because both bases are 16-byte aligned and the pitch is a multiple of 16).
struct Interior {
    int64_t head;      // bytes before the first full unit
    int64_t nu;        // full 16-byte units per row
};

__device__ __forceinline__ Interior interior_of(const SubTile& s)
{
    const int64_t mis = (int64_t)((uintptr_t)s.src & 15);
    int64_t head = mis ? 16 - mis : 0;
    if (head > s.bytes)
        head = s.bytes;
    const int64_t nu = (s.bytes - head) / 16;
    Interior in{head, nu};
    return in;
}

// u / nu for u < 2^16, nu >= 1 (single-precision reciprocal plus one correction step); a sub-tile
// has at most NT * UPT_LARGE = 3072 units.
__device__ __forceinline__ uint32_t div_small(uint32_t u, uint32_t nu, float rcp)
{
    uint32_t q = (uint32_t)((float)u * rcp);
    if (q * nu > u)
        --q;
    else if ((q + 1) * nu <= u)
        ++q;
    return q;
}

// The sub-tile's aligned interior: all UPT loads of a lane first (all in flight at once), then the
// stores.  Loads and stores are raw buffer operations over the sub-tile's span (under 2 GiB, which
// the plan guarantees); a lane past the interior's end gets an offset beyond the span, where a load
// returns zeros and a store is dropped without touching memory.  So no operation sits under a lane
// condition, which would make the compiler wait for each load right behind it.
constexpr int kStream = 2;            // cache policy "nt": the copy's lines are used once
constexpr uint32_t kNowhere = 0xFFFFFFF0u;

template <int UPT>
__device__ __forceinline__ void copy_interior(const SubTile& s, const Interior& in, int tid)
{
    const uint32_t U = (uint32_t)(s.rows * in.nu);
    if (U == 0)
        return;
    const uint32_t span = (uint32_t)((s.rows - 1) * s.pitch + in.head + in.nu * 16);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(s.src, span);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(s.dst, span);
    const uint32_t pitch = (uint32_t)s.pitch, head = (uint32_t)in.head, nu = (uint32_t)in.nu;
    const float rcp = 1.0f / (float)nu;
    i32x4 v[UPT];
    uint32_t off[UPT];
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
        const uint32_t u = j * NT + tid;
        const uint32_t row = div_small(u, nu, rcp);
        off[j] = u < U ? row * pitch + head + (u - row * nu) * 16 : kNowhere;
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[j], 0, kStream);
    }
#pragma unroll
    for (int j = 0; j < UPT; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(v[j], rd, off[j], 0, kStream);
}

// Bytes outside the aligned interior -- at most 15 at each end of a row, a whole number of elements
// -- one element per lane: element e of the sub-tile is element e % per_row of row e / per_row,
// counting the head's elements first.  EPT elements per lane are loaded before any is stored, so
// the loads' latencies overlap (a narrow ragged column tile is all edge).
template <typename T>
__device__ __forceinline__ void copy_edges_t(const SubTile& s, const Interior& in, int tid)
{
    constexpr int EPT = 4;
    const int64_t esz = sizeof(T);
    const int64_t nh = in.head / esz;
    const int64_t tail0 = in.head + in.nu * 16;
    const int64_t per_row = nh + (s.bytes - tail0) / esz;
    if (per_row == 0)
        return;
    const int64_t E = s.rows * per_row;
    for (int64_t e0 = 0; e0 < E; e0 += (int64_t)EPT * NT) {
        T v[EPT];
        int64_t off[EPT];
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int64_t e = min(e0 + j * NT + tid, E - 1);    // past the end: re-read the last one
            const int64_t row = e / per_row, k = e - row * per_row;
            off[j] = row * s.pitch + (k < nh ? k * esz : tail0 + (k - nh) * esz);
            v[j] = *reinterpret_cast<const T*>(s.src + off[j]);
        }
#pragma unroll
        for (int j = 0; j < EPT; ++j)
            if (e0 + j * NT + tid < E)
                *reinterpret_cast<T*>(s.dst + off[j]) = v[j];
    }
}

__device__ __forceinline__ void copy_edges(const SubTile& s, const Interior& in, int tid, int elem_size)
{
    if (in.head == 0 && in.head + in.nu * 16 >= s.bytes)
        return;
    switch (elem_size) {
    case 1: copy_edges_t<uint8_t>(s, in, tid); break;
    case 2: copy_edges_t<uint16_t>(s, in, tid); break;
    case 4: copy_edges_t<uint32_t>(s, in, tid); break;
    default: copy_edges_t<uint64_t>(s, in, tid); break;
    }
}

template <int UPT>
__global__ __launch_bounds__(NT) void tgather_vec_kernel(Plan P)
{
    const int tid = threadIdx.x;
    for (int64_t q = blockIdx.x; q < P.total; q += gridDim.x) {
        const SubTile s = locate(P, q);
        const Interior in = interior_of(s);
        copy_interior<UPT>(s, in, tid);
        copy_edges(s, in, tid, P.d.elem_size);
    }
}

// Fallback when rows are not 16-byte aligned (pitch not a multiple of 16 or unaligned bases):
// same sub-tile walk, element-wise copies.
__global__ __launch_bounds__(NT) void tgather_elem_kernel(Plan P)
{
    const int tid = threadIdx.x;
    const int esz = P.d.elem_size;
    for (int64_t q = blockIdx.x; q < P.total; q += gridDim.x) {
        const SubTile s = locate(P, q);
        const int64_t n = s.bytes / esz;
        for (int64_t row = 0; row < s.rows; ++row) {
            const char* sp = s.src + row * s.pitch;
            char* dp = s.dst + row * s.pitch;
            for (int64_t e = tid; e < n; e += NT) {
                const int64_t b = e * esz;
                switch (esz) {
                case 1: dp[b] = sp[b]; break;
                case 2: *reinterpret_cast<uint16_t*>(dp + b) = *reinterpret_cast<const uint16_t*>(sp + b); break;
                case 4: *reinterpret_cast<uint32_t*>(dp + b) = *reinterpret_cast<const uint32_t*>(sp + b); break;
                default: *reinterpret_cast<uint64_t*>(dp + b) = *reinterpret_cast<const uint64_t*>(sp + b); break;
                }
            }
        }
    }
}

void add_class(Plan& P, int64_t count, int64_t ncols, int64_t row0, int64_t col0, int64_t th, int64_t tw)
{
    if (count <= 0 || th <= 0 || tw <= 0)
        return;
    const int64_t esz = P.d.elem_size;
    TileClass c{};
    c.count = count;
    c.ncols = ncols;
    c.row0 = row0;
    c.col0 = col0;
    c.th = th;
    c.tw = tw;
    const int64_t twb = tw * esz;
    const int64_t SUB_BYTES = P.sub_bytes;
    if (twb <= SUB_BYTES) {
        c.scn = 1;
        c.scw = tw;
        c.sr = std::max<int64_t>(1, std::min<int64_t>(th, SUB_BYTES / twb));
        // a sub-tile's span, (sr - 1) * pitch + row bytes, stays under 2 GiB (32-bit buffer offsets)
        const int64_t pitch = P.d.W * esz;
        c.sr = std::max<int64_t>(1, std::min<int64_t>(c.sr, ((int64_t(1) << 31) - 1 - twb) / pitch + 1));
    } else {
        c.sr = 1;
        const int64_t pieces = (twb + SUB_BYTES - 1) / SUB_BYTES;
        c.scw = std::min<int64_t>((tw + pieces - 1) / pieces, SUB_BYTES / esz);
        c.scn = (tw + c.scw - 1) / c.scw;
    }
    c.subs = ((th + c.sr - 1) / c.sr) * c.scn;
    c.first = P.subs_per_region;
    P.subs_per_region += count * c.subs;
    P.cls[P.ncls++] = c;
}

int g_num_cus = 0;

}  // namespace

hipError_t launch_tgather(const GatherDesc& d, hipStream_t stream)
{
    if (d.nranks <= 0 || d.planes <= 0 || d.H <= 0 || d.W <= 0)
        return hipSuccess;                       // nothing to move
    if (g_num_cus == 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return e;
        e = hipDeviceGetAttribute(&g_num_cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
    }
    // the plan for either sub-tile size; the larger one only if it packs the rows at least 10 %
    // fuller (it holds 50 % more VGPRs per lane, so fewer workgroups fit on a CU)
    auto make_plan = [&](int upt) {
        Plan P{};
        P.d = d;
        P.sub_bytes = (int64_t)NT * upt * 16;
        const int64_t vr = std::min(d.valid_rows, d.H), vc = std::min(d.valid_cols, d.W);
        const int64_t nrf = d.H / vr, hr = d.H - nrf * vr;        // full row tiles, ragged height
        const int64_t ncf = d.W / vc, wr = d.W - ncf * vc;        // full column tiles, ragged width
        add_class(P, nrf * ncf, ncf, 0, 0, vr, vc);
        add_class(P, wr > 0 ? nrf : 0, 1, 0, ncf * vc, vr, wr);
        add_class(P, hr > 0 ? ncf : 0, ncf, nrf * vr, 0, hr, vc);
        add_class(P, (hr > 0 && wr > 0) ? 1 : 0, 1, nrf * vr, ncf * vc, hr, wr);
        P.total = (int64_t)d.nranks * d.planes * P.subs_per_region;
        return P;
    };
    Plan P = make_plan(UPT_SMALL);
    bool aligned = ((d.W * d.elem_size) % 16) == 0 && ((uintptr_t)d.dst % 16) == 0;
    for (int r = 0; r < d.nranks; ++r)
        aligned = aligned && ((uintptr_t)d.src[r] % 16) == 0;
    P.vec = aligned ? 1 : 0;
    int upt = UPT_SMALL;
    if (P.vec) {
        const Plan L = make_plan(UPT_LARGE);
        // fill = payload / (sub-tiles * sub-tile bytes): the payload is common to both plans
        if (11 * L.total * L.sub_bytes <= 10 * P.total * P.sub_bytes) {
            P = L;
            P.vec = 1;
            upt = UPT_LARGE;
        }
    }
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(P.total, (int64_t)g_num_cus * WG_PER_CU));
    if (!P.vec)
        tgather_elem_kernel<<<grid, NT, 0, stream>>>(P);
    else if (upt == UPT_LARGE)
        tgather_vec_kernel<UPT_LARGE><<<grid, NT, 0, stream>>>(P);
    else
        tgather_vec_kernel<UPT_SMALL><<<grid, NT, 0, stream>>>(P);
    return hipGetLastError();
}

}  // namespace ag
