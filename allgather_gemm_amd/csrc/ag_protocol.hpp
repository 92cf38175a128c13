// ag_protocol.hpp -- chunk and piece map of the fused AllGather + MatMul schedule, shared by the
// gfx950 kernels and by the host (launch planning and the CPU model of the copy protocol).
//
// Fused AllGather+MatMul article ("Triton第四课：基于对称内存融合 AllGather 与 MatMul，提速1.56倍"):
//  * section 融合后的流水线: every shard's rows are cut into comm blocks ("chunks") of cb rows; chunk
//    id r*S + s (S = ceil(H / cb)) covers rows [r*H + s*cb, r*H + min((s+1)*cb, H)) of the
//    gathered A;
//  * section 数据搬运与细粒度同步: one progress flag per chunk, raised once the chunk's rows have
//    landed.
// A chunk is moved as "pieces": contiguous byte ranges of at most piece_bytes (a chunk's rows are
// contiguous in the shard and in the gathered buffer, so any byte range of it is one copy).  Every
// chunk has the same number of pieces, ppc; the pieces past a short chunk's end are empty.
//
// Ready order (the order pieces are handed out): the local shard's edge chunks (those a tile that
// straddles the local shard's boundary reads from the gathered buffer), then the other shards in
// the rotation local+1, local+2, ... (the order the rotated tile walk reaches them), then the rest
// of the local shard, which only the gathered output needs.
//
// Everything here is integer arithmetic on plain values, compiled both for the device and the host.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define AG_HD __host__ __device__ __forceinline__
#else
#define AG_HD inline
#endif

namespace ag {

struct PieceMap {
    int64_t H;            // rows per shard
    int64_t cb;           // rows per chunk
    int64_t S;            // chunks per shard
    int64_t row_bytes;    // K * element size
    int64_t piece_bytes;  // bytes per piece (multiple of 16)
    int64_t ppc;          // pieces per chunk
    int64_t nchunks;      // nshards * S
    int32_t nshards;
    int32_t local;        // local shard
    int64_t edge_lo[2];   // local chunks [edge_lo[i], edge_hi[i]) are copied first
    int64_t edge_hi[2];
    int64_t nedge;        // chunks in the two edge ranges together
};

AG_HD int64_t pm_min(int64_t a, int64_t b) { return a < b ? a : b; }
AG_HD int64_t pm_max(int64_t a, int64_t b) { return a > b ? a : b; }

// Local chunk index range [s0, s1) whose rows meet gathered rows [r0, r1) (empty if none).
AG_HD void pm_local_chunks_meeting(const PieceMap& p, int64_t r0, int64_t r1, int64_t& s0, int64_t& s1)
{
    const int64_t lo = (int64_t)p.local * p.H, hi = lo + p.H;
    const int64_t a = pm_max(r0, lo), b = pm_min(r1, hi);
    if (a >= b) {
        s0 = s1 = 0;
        return;
    }
    s0 = (a - lo) / p.cb;
    s1 = (b - 1 - lo) / p.cb + 1;
}

// Fills the map.  bm: GEMM tile rows (the edge chunks are those meeting the tile rows that hold the
// local shard's first and last row, when those tiles also hold rows of another shard).
AG_HD PieceMap pm_make(int64_t H, int64_t cb, int32_t nshards, int32_t local, int64_t row_bytes,
                       int64_t bm, int64_t piece_bytes)
{
    PieceMap p;
    p.H = H;
    p.cb = cb;
    p.S = (H + cb - 1) / cb;
    p.row_bytes = row_bytes;
    p.piece_bytes = piece_bytes;
    const int64_t chunk_bytes = cb * p.row_bytes;
    p.ppc = chunk_bytes > 0 ? (chunk_bytes + piece_bytes - 1) / piece_bytes : 1;
    p.nchunks = (int64_t)nshards * p.S;
    p.nshards = nshards;
    p.local = local;
    const int64_t M = (int64_t)nshards * H, lo = (int64_t)local * H, hi = lo + H;
    int64_t n = 0;
    for (int e = 0; e < 2; ++e) {
        const int64_t row = e == 0 ? lo : hi - 1;
        const int64_t t0 = (row / bm) * bm, t1 = pm_min(t0 + bm, M);
        int64_t s0 = 0, s1 = 0;
        if (H > 0 && (t0 < lo || t1 > hi))       // the tile straddles the local shard's boundary
            pm_local_chunks_meeting(p, t0, t1, s0, s1);
        if (e == 1 && s0 < p.edge_hi[0]) {       // overlaps the first range: keep the ranges disjoint
            s0 = pm_max(s0, p.edge_hi[0]);
            if (s1 < s0)
                s1 = s0;
        }
        p.edge_lo[e] = s0;
        p.edge_hi[e] = s1;
        n += s1 - s0;
    }
    p.nedge = n;
    return p;
}

// Chunk id at position pos of the ready order.
AG_HD int64_t pm_ready_chunk(const PieceMap& p, int64_t pos)
{
    const int64_t lbase = (int64_t)p.local * p.S;
    const int64_t n0 = p.edge_hi[0] - p.edge_lo[0];
    if (pos < n0)
        return lbase + p.edge_lo[0] + pos;
    if (pos < p.nedge)
        return lbase + p.edge_lo[1] + (pos - n0);
    pos -= p.nedge;
    const int64_t remote = (int64_t)(p.nshards - 1) * p.S;
    if (pos < remote) {
        const int64_t step = pos / p.S, s = pos - step * p.S;
        const int64_t r = (p.local + 1 + step) % p.nshards;
        return r * p.S + s;
    }
    // rest of the local shard, skipping the edge ranges
    int64_t s = pos - remote;
    for (int e = 0; e < 2; ++e)
        if (s >= p.edge_lo[e])
            s += p.edge_hi[e] - p.edge_lo[e];
    return lbase + s;
}

// Inverse of pm_ready_chunk.
AG_HD int64_t pm_ready_pos(const PieceMap& p, int64_t c)
{
    const int64_t r = c / p.S, s = c - r * p.S;
    if (r == p.local) {
        if (s >= p.edge_lo[0] && s < p.edge_hi[0])
            return s - p.edge_lo[0];
        if (s >= p.edge_lo[1] && s < p.edge_hi[1])
            return (p.edge_hi[0] - p.edge_lo[0]) + (s - p.edge_lo[1]);
        int64_t before = s;        // local non-edge chunks before s
        for (int e = 0; e < 2; ++e)
            if (s >= p.edge_hi[e])
                before -= p.edge_hi[e] - p.edge_lo[e];
        return p.nedge + (int64_t)(p.nshards - 1) * p.S + before;
    }
    const int64_t step = ((r - p.local - 1) % p.nshards + p.nshards) % p.nshards;
    return p.nedge + step * p.S + s;
}

// Rows [first, last) of chunk c in the gathered A.
AG_HD void pm_chunk_rows(const PieceMap& p, int64_t c, int64_t& first, int64_t& last)
{
    const int64_t r = c / p.S, s = c - r * p.S;
    first = r * p.H + s * p.cb;
    last = r * p.H + pm_min((s + 1) * p.cb, p.H);
}

// Chunks overlapping gathered rows [m0, m1): ids c_first .. c_last (consecutive ids).
AG_HD void pm_chunks_of_rows(const PieceMap& p, int64_t m0, int64_t m1, int64_t& c_first, int64_t& c_last)
{
    c_first = (m0 / p.H) * p.S + (m0 % p.H) / p.cb;
    c_last = ((m1 - 1) / p.H) * p.S + ((m1 - 1) % p.H) / p.cb;
}

struct PieceSpan {
    int32_t shard;        // source shard
    int64_t src_off;      // byte offset inside the shard
    int64_t dst_off;      // byte offset inside the gathered buffer
    int64_t bytes;        // 0 for a piece past a short chunk's end
    int64_t chunk;
};

// Piece q: position q / ppc of the ready order, bytes [(q % ppc) * piece_bytes, ...) of that chunk.
AG_HD PieceSpan pm_piece(const PieceMap& p, int64_t q)
{
    const int64_t pos = q / p.ppc, sub = q - pos * p.ppc;
    const int64_t c = pm_ready_chunk(p, pos);
    int64_t first, last;
    pm_chunk_rows(p, c, first, last);
    const int64_t cbytes = (last - first) * p.row_bytes;
    const int64_t b0 = pm_min(sub * p.piece_bytes, cbytes), b1 = pm_min(b0 + p.piece_bytes, cbytes);
    PieceSpan sp;
    sp.shard = (int32_t)(c / p.S);
    sp.src_off = (first - (int64_t)sp.shard * p.H) * p.row_bytes + b0;
    sp.dst_off = first * p.row_bytes + b0;
    sp.bytes = b1 - b0;
    sp.chunk = c;
    return sp;
}

// Output tile t of the persistent walk: grouped order (group_m tile rows per group, so
// neighbouring tile ids share A and B rows in L2), then pid_m rotated by `pivot` so the walk starts
// at the local shard's first tile row ([AGMM] 融合后的流水线); the rotation is a bijection on pid_m.
AG_HD void pm_tile_of(int64_t t, int64_t num_pid_m, int64_t num_pid_n, int64_t pivot, int64_t group_m,
                      int64_t& pid_m, int64_t& pid_n)
{
    const int64_t per_group = group_m * num_pid_n;
    const int64_t group = t / per_group;
    const int64_t first_m = group * group_m;
    const int64_t left = num_pid_m - first_m;
    const int64_t rows = left < group_m ? left : group_m;
    const int64_t in_group = t - group * per_group;
    pid_m = (first_m + in_group % rows + pivot) % num_pid_m;
    pid_n = in_group / rows;
}

}  // namespace ag
