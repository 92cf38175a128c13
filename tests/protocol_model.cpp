// CPU model of the fused schedule's copy protocol, built from the library's own chunk / piece map
// and tile walk (allgather_gemm_amd/csrc/ag_protocol.hpp).  Workgroups are threads; the rules are
// the kernel's:
//   * a tile wholly inside the local shard reads the shard; any other tile first waits for every
//     chunk its rows overlap;
//   * while it waits, a workgroup takes batches of pieces -- from the fill counter (pieces of the
//     first wave's chunks) first, then from the main counter -- copies them at once and publishes
//     them: per-chunk piece count, and the chunk's flag when the count reaches pieces-per-chunk;
//   * every running "wave" (4 per workgroup) also holds one piece from the main counter and copies
//     one slice of it per K step (store of the previous slice, load of the next), publishing it one
//     step after its last store; it finishes its piece before its workgroup waits on anything.
// Checks: every piece is copied exactly once; when a flag rises, every byte of its chunk has
// landed; the gathered buffer equals the concatenation of the shards; no wait exceeds a deadline
// (a deadlock shows up as a timeout).  Prints "OK ..." or "FAIL ...".
//
// Usage: protocol_model N H K cb local grid bm bn Nc trickle(0|1) piece_bytes slice_bytes seed
#include "ag_protocol.hpp"

#include <algorithm>
#include <atomic>
#include <mutex>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <thread>
#include <vector>

using namespace ag;

struct Model {
    int N, local, grid, trickle;
    int64_t H, K, cb, bm, bn, Nc, M, slice;
    PieceMap pm;
    int64_t npieces, fill_end;
    int64_t num_pid_m, num_pid_n, pivot, nk;
    std::vector<std::vector<uint8_t>> shards;
    std::vector<uint8_t> A;                              // gathered buffer
    std::vector<std::atomic<uint32_t>> done, flag, copied;
    std::vector<std::atomic<int64_t>> landed;            // bytes landed per chunk
    std::atomic<uint32_t> fill_ctr{0}, main_ctr{0};
    std::atomic<int> failures{0};
    std::string why;
    std::mutex why_mu;

    void fail(const std::string& w)
    {
        std::lock_guard<std::mutex> g(why_mu);
        if (failures++ == 0)
            why = w;
    }
};

static int64_t take(std::atomic<uint32_t>& ctr, int64_t end, uint32_t want, int64_t* n)
{
    const uint32_t t = ctr.fetch_add(want);
    const int64_t avail = end - (int64_t)t;
    *n = avail <= 0 ? 0 : (avail < (int64_t)want ? avail : (int64_t)want);
    return t;
}

static void publish(Model& m, int64_t c, uint32_t n)
{
    const uint32_t old = m.done[c].fetch_add(n);
    if (old + n == (uint32_t)m.pm.ppc) {
        int64_t first, last;
        pm_chunk_rows(m.pm, c, first, last);
        if (m.landed[c].load() != (last - first) * m.pm.row_bytes)
            m.fail("flag of chunk " + std::to_string(c) + " raised before all its bytes landed");
        m.flag[c].store(1);
    } else if (old + n > (uint32_t)m.pm.ppc) {
        m.fail("chunk " + std::to_string(c) + " counted more pieces than it has");
    }
}

static void copy_bytes(Model& m, const PieceSpan& sp, int64_t off, int64_t len)
{
    std::memcpy(&m.A[sp.dst_off + off], &m.shards[sp.shard][sp.src_off + off], (size_t)len);
    m.landed[sp.chunk].fetch_add(len);
}

static void copy_piece(Model& m, int64_t q)
{
    const PieceSpan sp = pm_piece(m.pm, q);
    if (m.copied[q].fetch_add(1) != 0)
        m.fail("piece " + std::to_string(q) + " copied twice");
    copy_bytes(m, sp, 0, sp.bytes);
}

struct Trickle {
    int64_t q = -1, off = 0, pend = -1, publish_q = -1;
    bool exhausted = false;
};

static void trickle_step(Model& m, Trickle& t)
{
    if (t.publish_q >= 0) {
        publish(m, pm_piece(m.pm, t.publish_q).chunk, 1);
        t.publish_q = -1;
    }
    if (t.pend >= 0) {
        const PieceSpan sp = pm_piece(m.pm, t.q);
        copy_bytes(m, sp, t.pend, std::min<int64_t>(m.slice, sp.bytes - t.pend));
        if (t.pend + m.slice >= sp.bytes) {
            t.publish_q = t.q;
            t.q = -1;
        }
        t.pend = -1;
    }
    if (t.q < 0 && !t.exhausted) {
        int64_t n;
        const int64_t q = take(m.main_ctr, m.npieces, 1, &n);
        if (n == 0) {
            t.exhausted = true;
        } else {
            t.q = q;
            t.off = 0;
            if (m.copied[q].fetch_add(1) != 0)
                m.fail("piece " + std::to_string(q) + " taken twice");
        }
    }
    if (t.q >= 0) {
        const PieceSpan sp = pm_piece(m.pm, t.q);
        if (sp.bytes == 0) {
            t.publish_q = t.q;
            t.q = -1;
        } else {
            t.pend = t.off;
            t.off += m.slice;
        }
    }
}

static void trickle_flush(Model& m, Trickle& t)
{
    if (t.pend >= 0) {
        const PieceSpan sp = pm_piece(m.pm, t.q);
        copy_bytes(m, sp, t.pend, std::min<int64_t>(m.slice, sp.bytes - t.pend));
        t.pend = -1;
    }
    if (t.q >= 0) {
        const PieceSpan sp = pm_piece(m.pm, t.q);
        if (t.off < sp.bytes)
            copy_bytes(m, sp, t.off, sp.bytes - t.off);
    }
    if (t.publish_q >= 0) {
        publish(m, pm_piece(m.pm, t.publish_q).chunk, 1);
        t.publish_q = -1;
    }
    if (t.q >= 0) {
        publish(m, pm_piece(m.pm, t.q).chunk, 1);
        t.q = -1;
    }
}

static void workgroup(Model& m, int wg, unsigned seed)
{
    std::mt19937 rng(seed * 7919u + (unsigned)wg);
    Trickle waves[4];
    for (auto& w : waves)
        w.exhausted = !m.trickle;
    const int64_t lo = (int64_t)m.local * m.H, hi = lo + m.H;
    const int64_t tiles = m.num_pid_m * m.num_pid_n;
    for (int64_t t = wg; t < tiles; t += m.grid) {
        int64_t pid_m, pid_n;
        pm_tile_of(t, m.num_pid_m, m.num_pid_n, m.pivot, 8, pid_m, pid_n);
        const int64_t m0 = pid_m * m.bm, m1 = std::min(m0 + m.bm, m.M);
        if (!(m0 >= lo && m1 <= hi)) {
            for (auto& w : waves)
                trickle_flush(m, w);
            int64_t c0, c1;
            pm_chunks_of_rows(m.pm, m0, m1, c0, c1);
            bool exhausted = false;
            for (int64_t c = c0; c <= c1; ++c) {
                const auto deadline = std::chrono::steady_clock::now() + std::chrono::seconds(20);
                while (!m.flag[c].load()) {
                    int64_t n = 0, q = -1;
                    if (!exhausted) {
                        q = take(m.fill_ctr, m.fill_end, 4, &n);
                        if (n == 0)
                            q = take(m.main_ctr, m.npieces, 4, &n);
                        if (n == 0)
                            exhausted = true;
                    }
                    if (n > 0) {
                        for (int64_t i = 0; i < n; ++i)
                            copy_piece(m, q + i);
                        for (int64_t i = 0; i < n; ++i)
                            publish(m, pm_piece(m.pm, q + i).chunk, 1);
                    } else {
                        std::this_thread::yield();
                    }
                    if (std::chrono::steady_clock::now() > deadline) {
                        m.fail("wait on chunk " + std::to_string(c) + " by tile " + std::to_string(t) +
                               " never ended (deadlock)");
                        return;
                    }
                }
            }
            // every row this tile reads has landed
            for (int64_t r = m0; r < m1; ++r)
                for (int64_t b = 0; b < m.pm.row_bytes; ++b)
                    if (m.A[r * m.pm.row_bytes + b] != m.shards[r / m.H][(r % m.H) * m.pm.row_bytes + b]) {
                        m.fail("tile " + std::to_string(t) + " would read row " + std::to_string(r) +
                               " before it landed");
                        return;
                    }
        }
        for (int64_t k = 0; k < m.nk; ++k) {
            for (auto& w : waves)
                trickle_step(m, w);
            if (rng() % 4 == 0)
                std::this_thread::yield();
        }
    }
    for (auto& w : waves)
        trickle_flush(m, w);
    // before it exits the workgroup copies whatever no one has taken (fill counter, then the rest)
    for (std::atomic<uint32_t>* ctr : {&m.fill_ctr, &m.main_ctr}) {
        const int64_t end = ctr == &m.fill_ctr ? m.fill_end : m.npieces;
        for (;;) {
            int64_t n;
            const int64_t q = take(*ctr, end, 4, &n);
            if (n == 0)
                break;
            for (int64_t i = 0; i < n; ++i)
                copy_piece(m, q + i);
            for (int64_t i = 0; i < n; ++i)
                publish(m, pm_piece(m.pm, q + i).chunk, 1);
        }
    }
}

int main(int argc, char** argv)
{
    if (argc != 14) {
        std::fprintf(stderr, "usage: %s N H K cb local grid bm bn Nc trickle piece_bytes slice seed\n", argv[0]);
        return 2;
    }
    Model m;
    m.N = std::atoi(argv[1]);
    m.H = std::atoll(argv[2]);
    m.K = std::atoll(argv[3]);
    m.cb = std::atoll(argv[4]);
    m.local = std::atoi(argv[5]);
    m.grid = std::atoi(argv[6]);
    m.bm = std::atoll(argv[7]);
    m.bn = std::atoll(argv[8]);
    m.Nc = std::atoll(argv[9]);
    m.trickle = std::atoi(argv[10]);
    const int64_t piece_bytes = std::atoll(argv[11]);
    m.slice = std::atoll(argv[12]);
    const unsigned seed = (unsigned)std::atoi(argv[13]);
    m.M = m.N * m.H;
    m.pm = pm_make(m.H, m.cb, m.N, m.local, m.K * 2, m.bm, piece_bytes);   // K bf16 elements per row
    m.npieces = m.pm.nchunks * m.pm.ppc;
    m.num_pid_m = (m.M + m.bm - 1) / m.bm;
    m.num_pid_n = (m.Nc + m.bn - 1) / m.bn;
    m.pivot = (m.local * m.H) / m.bm % m.num_pid_m;
    m.nk = (m.K + 63) / 64;

    // ready order is a permutation of the chunks, and pm_ready_pos its inverse
    std::vector<int> seen(m.pm.nchunks, 0);
    for (int64_t pos = 0; pos < m.pm.nchunks; ++pos) {
        const int64_t c = pm_ready_chunk(m.pm, pos);
        if (c < 0 || c >= m.pm.nchunks || seen[c]++ || pm_ready_pos(m.pm, c) != pos) {
            std::printf("FAIL ready order is not a permutation at position %lld\n", (long long)pos);
            return 1;
        }
    }
    // the pieces of every chunk tile its bytes exactly
    for (int64_t c = 0; c < m.pm.nchunks; ++c) {
        int64_t first, last;
        pm_chunk_rows(m.pm, c, first, last);
        const int64_t pos = pm_ready_pos(m.pm, c);
        int64_t at = first * m.pm.row_bytes;
        for (int64_t sub = 0; sub < m.pm.ppc; ++sub) {
            const PieceSpan sp = pm_piece(m.pm, pos * m.pm.ppc + sub);
            if (sp.chunk != c || (sp.bytes > 0 && sp.dst_off != at) || sp.bytes < 0 || sp.bytes > piece_bytes) {
                std::printf("FAIL piece %lld of chunk %lld misplaced\n", (long long)sub, (long long)c);
                return 1;
            }
            at += sp.bytes;
        }
        if (at != last * m.pm.row_bytes) {
            std::printf("FAIL pieces of chunk %lld do not cover it\n", (long long)c);
            return 1;
        }
    }
    // first-wave fill end: every chunk a non-local tile of the first wave reads
    const int64_t lo = (int64_t)m.local * m.H, hi = lo + m.H;
    int64_t last_pos = -1;
    for (int64_t t = 0; t < std::min<int64_t>(m.grid, m.num_pid_m * m.num_pid_n); ++t) {
        int64_t pid_m, pid_n;
        pm_tile_of(t, m.num_pid_m, m.num_pid_n, m.pivot, 8, pid_m, pid_n);
        const int64_t m0 = pid_m * m.bm, m1 = std::min(m0 + m.bm, m.M);
        if (m0 >= lo && m1 <= hi)
            continue;
        int64_t c0, c1;
        pm_chunks_of_rows(m.pm, m0, m1, c0, c1);
        for (int64_t c = c0; c <= c1; ++c)
            last_pos = std::max(last_pos, pm_ready_pos(m.pm, c));
    }
    m.fill_end = (last_pos + 1) * m.pm.ppc;
    m.main_ctr.store((uint32_t)m.fill_end);

    std::mt19937 rng(seed);
    m.shards.resize(m.N);
    for (auto& s : m.shards) {
        s.resize((size_t)(m.H * m.pm.row_bytes));
        for (auto& b : s)
            b = (uint8_t)(rng() & 0xff);
    }
    m.A.assign((size_t)(m.M * m.pm.row_bytes), 0);
    for (size_t i = 0; i < m.A.size(); ++i)      // poison: a byte differing from the shard's
        m.A[i] = (uint8_t)(m.shards[(i / m.pm.row_bytes) / m.H][(((i / m.pm.row_bytes) % m.H) * m.pm.row_bytes) + i % m.pm.row_bytes] ^ 0x5a);
    m.done = std::vector<std::atomic<uint32_t>>(m.pm.nchunks);
    m.flag = std::vector<std::atomic<uint32_t>>(m.pm.nchunks);
    m.landed = std::vector<std::atomic<int64_t>>(m.pm.nchunks);
    m.copied = std::vector<std::atomic<uint32_t>>(m.npieces);

    std::vector<std::thread> th;
    for (int wg = 0; wg < m.grid; ++wg)
        th.emplace_back(workgroup, std::ref(m), wg, seed);
    for (auto& t : th)
        t.join();
    if (m.failures.load() == 0) {
        // the copy drains completely: every piece exactly once, every flag up, A == concatenation
        for (int64_t q = 0; q < m.npieces; ++q)
            if (m.copied[q].load() != 1) {
                m.fail("piece " + std::to_string(q) + " copied " + std::to_string(m.copied[q].load()) + " times");
                break;
            }
        for (int64_t c = 0; c < m.pm.nchunks && m.failures.load() == 0; ++c)
            if (!m.flag[c].load())
                m.fail("flag of chunk " + std::to_string(c) + " never raised");
        for (int64_t r = 0; r < m.M && m.failures.load() == 0; ++r)
            if (std::memcmp(&m.A[r * m.pm.row_bytes], &m.shards[r / m.H][(r % m.H) * m.pm.row_bytes],
                            (size_t)m.pm.row_bytes) != 0)
                m.fail("gathered row " + std::to_string(r) + " differs from its shard");
    }
    if (m.failures.load()) {
        std::printf("FAIL %s\n", m.why.c_str());
        return 1;
    }
    std::printf("OK chunks=%lld pieces=%lld fill_end=%lld edge=%lld\n", (long long)m.pm.nchunks,
                (long long)m.npieces, (long long)m.fill_end, (long long)m.pm.nedge);
    return 0;
}
