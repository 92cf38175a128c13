"""Pins for the CPU oracle: each test checks it against something other than itself.

The pins are values the pages print or state for a worked example (tests/golden/), closed
forms, library routines the method reduces to in a special case (torch.cat, float64 matmul),
brute force with an error bound, and invariants of the fused schedule.  A plausible mistake in
the oracle -- a dropped term, a swapped index, a transposed operand, a wrong accumulation
order -- fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import read_golden


def np_of(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> numpy array with the same element size (bf16 as uint16 bits)."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def bytes_of(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint8).reshape(-1)


# ---------------------------------------------------------------------------------- gather
@pytest.mark.parametrize("N,D,H,W,dtype,bits", [
    (4, (1, 1, 1), 3, 5, torch.float32, False),
    (8, (2, 1, 1), 16, 24, torch.float16, False),       # small version of the fp16 gather config
    (3, (2, 3, 2), 5, 7, torch.int32, False),           # every outer dim > 1
    (5, (1, 2, 1), 4, 9, torch.uint8, False),
    (2, (3, 1, 2), 6, 3, torch.float64, False),
    (8, (1, 1, 1), 10, 50, torch.float32, True),        # raw bit patterns: NaN payloads, subnormals
    (1, (1, 1, 1), 7, 4, torch.int16, False),           # a single rank
])
def test_gather_matches_torch_cat(N, D, H, W, dtype, bits):
    """TGATHER deep dive §二: dst is the concatenation along DIM_3 (rows) of the ranks' tensors,
    every other dim unchanged -- exactly torch.cat(dim=3) on (D0,D1,D2,H,W) views."""
    shards = workloads.make_tgather(N, D, H, W, dtype, seed=1, bits=bits)
    expect = torch.cat(shards, dim=3)
    dst = np.zeros(expect.numel() * expect.element_size(), dtype=np.uint8)
    dst = dst.view(np_of(shards[0]).dtype)
    oracle.tgather([np_of(s) for s in shards], dst, *D, H, W)
    assert np.array_equal(bytes_of(dst), bytes_of(np_of(expect)))


def test_gather_outer_dims_interleave():
    """With D0 > 1 the destination is per outer index: dst[d0] = concat_r src_r[d0], not the
    concatenation of flattened shards (the closed form keeps d0 outside the row index)."""
    N, H, W = 3, 2, 4
    shards = [(np.full((2, 1, 1, H, W), 10 * r) + np.arange(2).reshape(2, 1, 1, 1, 1)).astype(np.int32)
              for r in range(N)]
    dst = np.zeros((2, 1, 1, N * H, W), dtype=np.int32)
    oracle.tgather(shards, dst, 2, 1, 1, H, W)
    for d0 in range(2):
        for r in range(N):
            assert (dst[d0, 0, 0, r * H:(r + 1) * H] == 10 * r + d0).all()


def test_gather_golden_rank_pattern():
    g = read_golden("tgather_rank_pattern.txt")
    nr, count = int(g["nranks"][0]), int(g["count"][0])
    shards = [np.arange(count, dtype=np.float32) + r * 10000 for r in range(nr)]
    dst = np.zeros(nr * count, dtype=np.float32)
    oracle.tgather(shards, dst, 1, 1, 1, 1, count)
    assert dst.tolist() == [float(x) for x in g["dst"]]


@pytest.mark.parametrize("dtype,count", [(np.float32, 256), (np.int32, 4096), (np.uint8, 512)])
def test_gather_page_test_matrix_basic(dtype, count):
    """TGATHER deep dive §九: basic cases float 256 / int32 4096 / uint8 512 elements per rank,
    shape [1,1,1,1,count], value i + rank*10000 (wrapping in uint8), 8 ranks."""
    nr = 8
    shards = [(np.arange(count, dtype=np.int64) + r * 10000).astype(dtype) for r in range(nr)]
    dst = np.zeros(nr * count, dtype=dtype)
    oracle.tgather(shards, dst, 1, 1, 1, 1, count)
    for r in range(nr):
        expect = (np.arange(count, dtype=np.int64) + r * 10000).astype(dtype)
        assert np.array_equal(dst[r * count:(r + 1) * count], expect)


def test_gather_golden_empty():
    g = read_golden("tgather_empty.txt")
    nr, H, W, dst_rows = (int(g[k][0]) for k in ("nranks", "H", "W", "dst_rows"))
    init = float(g["initial"][0])
    shards = [np.zeros((0, W), dtype=np.float32) for _ in range(nr)]
    dst = np.full(dst_rows * W, init, dtype=np.float32)
    oracle.tgather(shards, dst, 1, 1, 1, H, W, dst_rows=dst_rows)
    assert (dst == init).all()
    # zero columns: nothing moves either
    shards = [np.zeros((3, 0), dtype=np.float32) for _ in range(nr)]
    dst = np.full(0, init, dtype=np.float32)
    oracle.tgather(shards, dst, 1, 1, 1, 3, 0)


def test_gather_taller_dst_keeps_extra_rows():
    """TGATHER deep dive §7.2: a dst taller than N*H receives only the first N*H rows."""
    N, H, W, extra = 4, 3, 6, 5
    shards = [np.full((H, W), r + 1, dtype=np.int32) for r in range(N)]
    dst = np.full(((N * H + extra) * W,), -7, dtype=np.int32)
    oracle.tgather(shards, dst, 1, 1, 1, H, W, dst_rows=N * H + extra)
    d = dst.reshape(N * H + extra, W)
    for r in range(N):
        assert (d[r * H:(r + 1) * H] == r + 1).all()
    assert (d[N * H:] == -7).all()
    # with an outer dim the untouched rows sit at the end of every plane
    shards = [np.full((2, 1, 1, H, W), r + 1, dtype=np.int32) for r in range(N)]
    dst = np.full((2, 1, 1, N * H + extra, W), -7, dtype=np.int32)
    oracle.tgather(shards, dst, 2, 1, 1, H, W, dst_rows=N * H + extra)
    assert (dst[:, :, :, N * H:] == -7).all() and (dst[:, :, :, :N * H] > 0).all()


def test_gather_rejects_invalid():
    """TGATHER deep dive §7.2 (dst DIM_3 must hold N*H rows) and §7.3 (at least one rank)."""
    shards = [np.zeros((2, 2), dtype=np.float32)] * 2
    with pytest.raises(ValueError):
        oracle.tgather(shards, np.zeros(6, dtype=np.float32), 1, 1, 1, 2, 2, dst_rows=3)
    with pytest.raises(ValueError):
        oracle.tgather([], np.zeros(0, dtype=np.float32), 1, 1, 1, 2, 2, dst_rows=0)


# ---------------------------------------------------------------------------------- bf16
def test_bf16_conversions():
    # exact round trip for every finite bf16 pattern's value through fp32
    bits = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    for b, f in zip(bits[:400], t[:400].tolist()):
        got = oracle.bf16_to_f32(int(b))
        assert (math.isnan(got) and math.isnan(f)) or got == f
    # RNE against torch's fp32 -> bf16 cast (a library routine), including exact ties
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.standard_normal(2000).astype(np.float32) * 100,
                         np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 3.0e38],
                                  dtype=np.float32)])
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for x, r in zip(xs.tolist(), ref.tolist()):
        assert oracle.f32_to_bf16_rne(x) == r
    assert oracle.f32_to_bf16_rne(1 + 2 ** -8) == 0x3F80            # tie -> even (1.0)
    assert oracle.f32_to_bf16_rne(1 + 3 * 2 ** -8) == 0x3F82        # tie -> even (1 + 2^-6)


# ---------------------------------------------------------------------------------- GEMM
def to_bf16_bits(vals) -> np.ndarray:
    return np_of(torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16))


def test_gemm_golden_2x2_transposed_operand():
    g = read_golden("gemm_2x2.txt")
    A = to_bf16_bits([float(x) for x in g["A"]]).reshape(2, 2)
    B = to_bf16_bits([float(x) for x in g["B"]]).reshape(2, 2)
    C = oracle.gemm_f32(A, B)
    assert C.reshape(-1).tolist() == [float(x) for x in g["C"]]


def test_gemm_golden_fp32_ascending_accumulation():
    g = read_golden("fp32_ascending.txt")
    a = to_bf16_bits([float(x) for x in g["a"]]).reshape(1, -1)
    b = to_bf16_bits([float(x) for x in g["b"]]).reshape(1, -1)
    C = oracle.gemm_f32(a, b)
    assert C[0, 0] == float(g["c_fp32_ascending"][0])
    assert C[0, 0] != float(g["c_exact"][0])


def higham_bound(a_rows: np.ndarray, b_rows: np.ndarray, K: int) -> np.ndarray:
    """gamma_K * sum |a_k b_k| with gamma_K = K u / (1 - K u), u = 2^-24 (recursive fp32 summation
    of exact products)."""
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    return gamma * np.sum(np.abs(a_rows * b_rows), axis=-1)


@pytest.mark.parametrize("M,Nc,K,seed", [(17, 13, 300, 0), (8, 40, 1024, 1), (33, 9, 4096, 2)])
def test_gemm_brute_force_exact_sum(M, Nc, K, seed):
    """Every product of two bf16 values is exact in fp64; math.fsum gives the correctly rounded
    sum.  The oracle's fp32 result must sit within the recursive-summation bound of it, for
    every element (a dropped term or a wrong index breaks this by orders of magnitude)."""
    A_t, _, B_t = workloads.make_ag_gemm_shapes(1, M, K, Nc, seed=seed)
    A, B = np_of(A_t), np_of(B_t)
    C = oracle.gemm_f32(A, B)
    Af, Bf = A_t.double().numpy(), B_t.double().numpy()
    for m in range(M):
        for n in range(Nc):
            exact = math.fsum((Af[m] * Bf[n]).tolist())
            bound = higham_bound(Af[m], Bf[n], K)
            assert abs(float(C[m, n]) - exact) <= bound, (m, n)


@pytest.mark.parametrize("M,Nc,K,seed", [(7, 5, 3, 0), (33, 17, 300, 1), (65, 259, 257, 2), (130, 40, 1000, 3),
                                        (1, 1, 1, 4), (5, 16, 0, 5), (300, 300, 70, 6), (64, 512, 2048, 7)])
def test_gemm_fast_is_bitwise_the_naive_order(M, Nc, K, seed):
    """The blocked loop order used for the full-size checks computes every element with the same
    ascending-k fp32 recursive sum as the naive triple loop, so the two agree bit for bit on shapes
    that leave ragged row, column and k blocks."""
    A_t, _, B_t = workloads.make_ag_gemm_shapes(1, M, K, Nc, seed=seed)
    naive = oracle.gemm_f32(np_of(A_t), np_of(B_t))
    fast = oracle.gemm_f32_fast(np_of(A_t), np_of(B_t))
    assert np.array_equal(naive.view(np.uint32), fast.view(np.uint32))


def test_ag_gemm_fast_matches_gather_then_gemm():
    """oracle.ag_gemm_fast reads A's rows from the shards without gathering them; bitwise equal to
    the gather-then-GEMM C on a ragged multi-shard shape, including signed zeros and exact ties."""
    A_t, shards, B_t = workloads.make_ag_gemm_shapes(5, 37, 136, 70, seed=12)
    _, C = oracle.ag_gemm([np_of(s) for s in shards], np_of(B_t))
    Cf = oracle.ag_gemm_fast([np_of(s) for s in shards], np_of(B_t))
    assert np.array_equal(C.view(np.uint32), Cf.view(np.uint32))


def test_gemm_identity_b_returns_a():
    """Special case B = I (K = Nc): every sum has one non-zero term, so C == A exactly."""
    M, K = 24, 40
    A_t, _, _ = workloads.make_ag_gemm_shapes(1, M, K, 1, seed=5)
    I = torch.eye(K, dtype=torch.bfloat16)
    C = oracle.gemm_f32(np_of(A_t), np_of(I))
    assert np.array_equal(C, A_t.float().numpy())


def test_gemm_tiny_config_vs_float64_matmul():
    """The tiny AG-GEMM workload against torch.matmul in float64 (a library routine) within the
    recursive-summation bound."""
    cfg = workloads.AG_TINY
    A_t, shards, B_t = workloads.make_ag_gemm(cfg)
    C = oracle.gemm_f32(np_of(A_t), np_of(B_t))
    ref = torch.matmul(A_t.double(), B_t.double().t()).numpy()
    Af, Bf = A_t.double().numpy(), B_t.double().numpy()
    bound = np.array([[higham_bound(Af[m], Bf[n], cfg.K) for n in range(cfg.Nc)] for m in range(cfg.M)])
    assert (np.abs(C.astype(np.float64) - ref) <= bound + 1e-12).all()


# ---------------------------------------------------------------------------------- AG-GEMM
def test_ag_gemm_is_gather_then_gemm():
    cfg = workloads.AG_TINY
    A_t, shards, B_t = workloads.make_ag_gemm(cfg)
    A_out, C = oracle.ag_gemm([np_of(s) for s in shards], np_of(B_t))
    assert np.array_equal(A_out, np_of(A_t))                  # gathered A == torch.cat(shards)
    ref = torch.matmul(A_t.double(), B_t.double().t()).numpy()
    assert np.max(np.abs(C - ref)) < 1e-3
    ms = np.array([0, 1, 63, 64, 100, 255, 255, 128])
    ns = np.array([0, 127, 5, 64, 0, 127, 0, 77])
    at = oracle.ag_gemm_at([np_of(s) for s in shards], np_of(B_t), ms, ns)
    assert np.array_equal(at, C[ms, ns])


def test_chunk_map_partition():
    """Comm blocks split every shard along M into cb-row blocks (last one shorter); block s of
    shard r carries flag index r * splits_per_rank + s (fused AG-MatMul article, progress
    array section)."""
    for N, H, cb in [(4, 64, 32), (8, 500, 100), (3, 10, 4), (2, 7, 7), (5, 9, 1), (2, 5, 8)]:
        S = -(-H // cb)
        rows_of = {}
        for m in range(N * H):
            rows_of.setdefault(oracle.chunk_of_row(m, H, cb), []).append(m)
        assert sorted(rows_of) == list(range(N * S))
        for c, rows in rows_of.items():
            r, s = divmod(c, S)
            assert rows == list(range(r * H + s * cb, r * H + min((s + 1) * cb, H)))
        # overlap query on a few ranges, against the row-wise definition
        for m0, m1 in [(0, N * H), (1, 2), (H - 1, H + 1), (max(0, H - 3), min(N * H, 2 * H + 3))]:
            expect = sorted({oracle.chunk_of_row(m, H, cb) for m in range(m0, m1)})
            assert oracle.chunks_overlapping(m0, m1, H, cb) == expect


def test_grouped_order_is_a_bijection():
    for pm, pn, g in [(4, 2, 8), (32, 32, 8), (16, 112, 4), (7, 5, 3), (1, 9, 2)]:
        seen = {oracle.grouped_tile(t, pm, pn, g) for t in range(pm * pn)}
        assert seen == {(i, j) for i in range(pm) for j in range(pn)}


# ---------------------------------------------------------------------------------- pivot
@pytest.mark.parametrize("N,H,K,Nc,cb,BM,BN,group,local", [
    (4, 64, 128, 128, 32, 64, 64, 8, 0),     # the tiny AG-GEMM workload
    (4, 64, 128, 128, 32, 64, 64, 8, 3),
    (4, 64, 32, 48, 32, 128, 32, 2, 2),      # BM > H: every tile spans several shards
    (8, 50, 16, 40, 10, 32, 16, 4, 5),       # ragged: cb | H but BM straddles chunks and shards
    (3, 37, 24, 20, 8, 16, 8, 3, 1),         # H % cb != 0 (short last chunk), H % BM != 0
    (2, 9, 8, 8, 9, 4, 8, 1, 1),             # cb == H: one chunk per shard
    (1, 40, 16, 16, 7, 16, 16, 2, 0),        # one shard: every tile local
    (5, 20, 12, 30, 3, 64, 64, 8, 4),        # one tile row covers all of M
])
def test_pivoted_schedule_equals_gather_then_gemm(N, H, K, Nc, cb, BM, BN, group, local):
    """Fused AG-MatMul article, section 融合后的流水线: once every chunk is consumed the result
    equals a full AllGather followed by the MatMul.  The simulation reads a poisoned (NaN)
    buffer for unpublished chunks, so a missed wait shows up in C and in rc."""
    A_t, shards, B_t = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=7)
    sh = [np_of(s) for s in shards]
    A_ref, C_ref = oracle.ag_gemm(sh, np_of(B_t))
    rc, A_p, C_p, st = oracle.ag_gemm_pivoted(sh, np_of(B_t), cb, BM, BN, group, local)
    assert rc == 0
    assert np.array_equal(C_p.view(np.uint32), C_ref.view(np.uint32))   # bitwise
    assert np.array_equal(A_p, A_ref)
    num_pid_n = -(-Nc // BN)
    if H % BM == 0:
        assert st["local_tiles"] == (H // BM) * num_pid_n
    if N == 1:
        assert st["waited_tiles"] == 0


def test_pivot_matches_page_formula_when_one_block_per_rank():
    """With one comm block per rank (cb = H) and BM | H, rotating pid_m by floor(local*H/BM)
    is the article's literal offset NUM_PID_M_PER_COMM_BLOCK * RANK: the first visited tile row
    is the first tile row of the local shard, so the first tiles need no wait."""
    N, H, K, Nc, BM, BN = 4, 64, 16, 32, 32, 32
    A_t, shards, B_t = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=9)
    sh = [np_of(s) for s in shards]
    for local in range(N):
        # group_m = 1 makes tile order row-major in pid_m, so the local tile rows come first
        rc, _, _, st = oracle.ag_gemm_pivoted(sh, np_of(B_t), H, BM, BN, 1, local)
        assert rc == 0
        assert st["local_tiles"] == (H // BM) * (Nc // BN)
        # one chunk per remote shard: only the first tile reading each shard waits, and every
        # remote tile checks exactly one flag
        assert st["waited_tiles"] == N - 1
        assert st["flag_checks"] == (N - 1) * (H // BM) * (Nc // BN)
        # the page's rotation: the first visited tile row is NUM_PID_M_PER_COMM_BLOCK * RANK
        # (here H // BM tile rows per comm block), and all local tiles come before any remote one
        assert st["first_pid_m"] == (H // BM) * local
        assert st["tiles_before_first_remote"] == (H // BM) * (Nc // BN)
        # no tile reads the local shard's copy, so the producer's ready order leaves it for last:
        # only the remote chunks were needed while tiles ran
        assert st["published_before_drain"] == N - 1


def test_pivot_poison_catches_missing_wait():
    """Sanity check of the detector itself: reading A_prime without publishing (simulated by
    asking for a result before any chunk is published) yields NaN, i.e. the poison is live."""
    N, H, K, Nc = 2, 8, 8, 8
    A_t, shards, B_t = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=11)
    poison = np.full((N * H, K), 0x7FC0, dtype=np.uint16)
    C = oracle.gemm_f32(poison, np_of(B_t))
    assert np.isnan(C).all()


# ------------------------------------------------------------------- FP8 (E4M3 "fn") output
def test_e4m3fn_hand_cases_from_the_format_definition():
    """Values fixed by the format itself: bias 7, 3 mantissa bits, subnormal steps of 2^-9, largest
    finite 448 (S.1111.110), S.1111.111 is NaN; round to nearest, ties to even."""
    cases = [
        (0.0, 0x00), (-0.0, 0x80), (1.0, 0x38), (-2.0, 0xC0), (448.0, 0x7E), (-448.0, 0xFE),
        (2.0 ** -6, 0x08),          # smallest normal
        (2.0 ** -9, 0x01),          # smallest subnormal
        (7 * 2.0 ** -9, 0x07),      # largest subnormal
        (2.0 ** -10, 0x00),         # halfway 0 .. 2^-9: tie to the even code 0
        (3 * 2.0 ** -10, 0x02),     # halfway 2^-9 .. 2^-8: tie to mantissa 2 (even)
        (1.0625, 0x38),             # halfway 1 .. 1.125: tie to 1.0 (mantissa 0)
        (1.1875, 0x3A),             # halfway 1.125 .. 1.25: tie to 1.25 (mantissa 2)
        (1.07, 0x39),               # nearer 1.125
        (15.0 * 2.0 ** -10, 0x08),  # halfway 7*2^-9 .. 2^-6: tie to the even code 0x08
        (464.0, 0x7E),              # halfway 448 .. 480: tie to mantissa 110 (448)
        (464.5, 0x7F), (1e9, 0x7F), (-465.0, 0xFF),   # rounding beyond 448: NaN
    ]
    for x, code in cases:
        assert oracle.f32_to_e4m3fn(np.float32(x)) == code, (x, hex(int(oracle.f32_to_e4m3fn(np.float32(x)))))
    assert oracle.f32_to_e4m3fn(np.float32(np.inf)) == 0x7F
    assert oracle.f32_to_e4m3fn(np.float32(-np.inf)) == 0xFF
    assert np.isnan(oracle.e4m3fn_value(0x7F)) and np.isnan(oracle.e4m3fn_value(0xFF))
    assert oracle.e4m3fn_value(0x7E) == 448.0 and oracle.e4m3fn_value(0x01) == 2.0 ** -9


def test_e4m3fn_every_code_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3fn_value(codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254
    back = oracle.f32_to_e4m3fn(vals[finite].astype(np.float32))
    assert np.array_equal(back, codes[finite])
    # values are strictly increasing over the non-negative codes 0x00 .. 0x7E
    assert np.all(np.diff(vals[:0x7F]) > 0)


def test_e4m3fn_matches_torch_float8_conversion():
    """torch's float8_e4m3fn conversion is an independent implementation of the same rounding."""
    rng = np.random.default_rng(5)
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3fn_value(codes)
    fin = np.unique(vals[~np.isnan(vals)])
    mids = (fin[1:] + fin[:-1]) / 2
    xs = np.concatenate([
        fin, mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
        np.nextafter(mids.astype(np.float32), np.float32(-np.inf)),
        rng.standard_normal(4000) * 50, np.exp(rng.uniform(-25, 6.3, 4000)) * rng.choice([-1, 1], 4000),
        [463.99, 464.0, 464.01, 479.0, 480.0, 1e6, -1e6, np.inf, -np.inf],
    ]).astype(np.float32)
    ours = oracle.f32_to_e4m3fn(xs)
    theirs = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs), xs[ours != theirs][:10]


# ------------------------------------------------------------------ FP8 inputs
def test_e4m3fn_to_bf16_is_exact_for_every_code():
    """Every E4M3 value's bf16 image is the same number: checked against torch's own float8_e4m3fn
    decoding (an independent implementation), with the NaN code mapping to NaN."""
    codes = np.arange(256, dtype=np.uint8)
    bits = oracle.e4m3fn_to_bf16(codes)
    as_f32 = (bits.astype(np.uint32) << 16).view(np.float32)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(theirs)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.isnan(as_f32[nan]).all()
    assert np.array_equal(as_f32[~nan], theirs[~nan])
    assert np.array_equal(as_f32[~nan], oracle.e4m3fn_value(codes)[~nan].astype(np.float32))


@pytest.mark.parametrize("M,Nc,K,seed", [(5, 7, 48, 1), (33, 17, 160, 2)])
def test_fp8_input_gemm_exact_integers_against_int64(M, Nc, K, seed):
    """FP8 integer inputs: the product through the bf16 images equals the int64 product."""
    rng = np.random.default_rng(seed)
    a = rng.integers(-4, 5, (M, K))
    b = rng.integers(-4, 5, (Nc, K))
    ca = torch.from_numpy(a.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    cb = torch.from_numpy(b.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    C = oracle.gemm_f32(oracle.e4m3fn_to_bf16(ca), oracle.e4m3fn_to_bf16(cb))
    assert np.array_equal(C.astype(np.int64), a @ b.T)


def test_fp8_input_gemm_within_fp32_bound_of_float64():
    """Random E4M3 inputs: products are exact, so the fp32 ascending sum is within K * 2^-24 *
    sum |a b| of the float64 product of the decoded values."""
    rng = np.random.default_rng(7)
    M, Nc, K = 9, 11, 320
    ca = workloads.to_e4m3fn_codes(torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))).numpy()
    cb = workloads.to_e4m3fn_codes(torch.from_numpy(rng.standard_normal((Nc, K)).astype(np.float32))).numpy()
    va, vb = oracle.e4m3fn_value(ca), oracle.e4m3fn_value(cb)
    C = oracle.gemm_f32(oracle.e4m3fn_to_bf16(ca), oracle.e4m3fn_to_bf16(cb)).astype(np.float64)
    ref = va @ vb.T
    bound = K * 2.0 ** -24 * (np.abs(va) @ np.abs(vb).T)
    assert (np.abs(C - ref) <= bound).all()


# ------------------------------------------------------------------ GEMM + ReduceScatter (one rank)
def _int_bf16(rng, shape, lim):
    """Small integers as bf16 bit patterns (exact)."""
    v = rng.integers(-lim, lim + 1, shape).astype(np.float32)
    return oracle.f32_to_bf16(v), v.astype(np.int64)


def test_reduce_scatter_then_allgather_is_allreduce():
    """[AGMM] 从集合通信理解数据流: ReduceScatter followed by AllGather equals AllReduce.  With
    integer-valued partials every fp32 sum is exact, so the AllReduce is computed independently in
    int64 and the identity must hold bit for bit."""
    rng = np.random.default_rng(11)
    N, H, Nc = 4, 6, 40
    parts_bits, parts_int = zip(*[_int_bf16(rng, (N * H, Nc), 50) for _ in range(N)])
    gathered = np.concatenate([oracle.reduce_block([p[r * H:(r + 1) * H] for p in parts_bits]) for r in range(N)])
    allreduce = oracle.f32_to_bf16(np.sum(np.stack(parts_int), axis=0).astype(np.float32))
    assert np.array_equal(gathered, allreduce)


def test_reduce_block_sums_in_fp32_in_ascending_rank_order():
    """Where the fp32 order matters: 2^24 + 1 rounds back to 2^24 (a tie, to even), so in ascending
    order 2^24, 1, 1, -2^24 sums to 0; in the reverse order the partial sums stay exact and give 2."""
    vals = [2.0 ** 24, 1.0, 1.0, -(2.0 ** 24)]
    parts = [oracle.f32_to_bf16(np.full((1, 8), v, dtype=np.float32)) for v in vals]
    assert np.all(oracle.reduce_block(parts) == 0)
    rev = oracle.reduce_block(parts[::-1])
    assert np.all(rev == oracle.f32_to_bf16(np.float32(2.0)))


def test_gemm_rs_exact_integers_against_int64():
    rng = np.random.default_rng(12)
    N, H, K, Nc = 3, 5, 24, 16
    A_bits, A_int = _int_bf16(rng, (N * H, K), 2)
    B_bits, B_int = _int_bf16(rng, (Nc, K), 2)
    recv = [_int_bf16(rng, (H, Nc), 30) for _ in range(N)]
    for local in range(N):
        P, out = oracle.gemm_rs(A_bits, B_bits, [r[0] for r in recv], local)
        P_int = A_int @ B_int.T
        assert np.array_equal(P, oracle.f32_to_bf16(P_int.astype(np.float32)))
        want = P_int[local * H:(local + 1) * H] + sum(recv[j][1] for j in range(N) if j != local)
        assert np.array_equal(out, oracle.f32_to_bf16(want.astype(np.float32)))


def test_reduce_block_within_rounding_of_the_exact_sum():
    rng = np.random.default_rng(13)
    parts = [oracle.f32_to_bf16(rng.standard_normal((7, 33)).astype(np.float32)) for _ in range(8)]
    vals = [np.array([oracle.bf16_to_f32(int(b)) for b in p.ravel()]).reshape(p.shape) for p in parts]
    exact = np.sum(vals, axis=0)
    out = np.array([oracle.bf16_to_f32(int(b)) for b in oracle.reduce_block(parts).ravel()]).reshape(exact.shape)
    # fp32 sum of 8 terms (7 roundings, each within 2^-24 relative of a partial sum), then one bf16
    # rounding (8 significant bits: within 2^-8 relative)
    bound = 2.0 ** -8 * np.abs(exact) + 8 * 2.0 ** -24 * np.sum(np.abs(vals), axis=0) * 1.01
    assert np.all(np.abs(out - exact) <= bound)
