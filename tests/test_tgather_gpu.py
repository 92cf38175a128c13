"""TGATHER on the GPU against the CPU oracle, bit-exact (the gather is a copy).

Cases follow the TGATHER deep dive: the fp16 gather workload and the ragged fp32 workload,
section 九's test matrix (basic / root / empty / large chunked / ping-pong), 2D sliding with
ragged tiles, outer dims, a taller destination, and the element path for unaligned rows.
"""
import numpy as np
import pytest
import torch

import allgather_gemm_amd as ag
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


def np_bytes(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    return t.view(torch.uint8).numpy().reshape(-1) if t.dtype != torch.uint8 else t.numpy().reshape(-1)


def oracle_gather(shards_cpu, D, H, W, dst_rows=None, init=None):
    N = len(shards_cpu)
    dst_rows = N * H if dst_rows is None else dst_rows
    esz = shards_cpu[0].element_size()
    n = D[0] * D[1] * D[2] * dst_rows * W
    dst = np.zeros(n * esz, dtype=np.uint8) if init is None else np_bytes(init).copy()
    dst = dst.view({1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[esz])
    srcs = [np_bytes(s).view(dst.dtype) for s in shards_cpu]
    oracle.tgather(srcs, dst, D[0], D[1], D[2], H, W, dst_rows=dst_rows)
    return dst.view(np.uint8)


def run_and_compare(shards_cpu, D, H, W, vr, vc, dst_rows=None, fill=None):
    print("tgather N=%d D=%s H=%d W=%d esz=%d valid=%dx%d dst_rows=%s" % (
        len(shards_cpu), D, H, W, shards_cpu[0].element_size(), vr, vc, dst_rows), flush=True)
    shards = [s.to(DEV) for s in shards_cpu]
    N = len(shards)
    rows = N * H if dst_rows is None else dst_rows
    dst = torch.empty((D[0], D[1], D[2], rows, W), dtype=shards_cpu[0].dtype, device=DEV)
    if fill is not None:
        dst.view(torch.uint8).fill_(fill)
    init = dst.cpu()
    ag.tgather(shards, vr, vc, dst=dst, dst_rows=rows)
    torch.cuda.synchronize()
    got = np_bytes(dst)
    expect = oracle_gather(shards_cpu, D, H, W, dst_rows=rows, init=init)
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("vr,vc", [(512, 2048),        # a whole (H, W) plane per tile
                                   (64, 512),          # 2D sliding, tiles divide the plane
                                   (100, 300),         # ragged last row and column tiles
                                   (1, 2048),          # one row per tile
                                   (10 ** 6, 10 ** 6)])  # larger than the plane
def test_fp16_gather_workload(vr, vc):
    cfg = workloads.TG_FP16
    shards = workloads.make_tgather(cfg.N, cfg.D, cfg.H, cfg.W, cfg.dtype, seed=cfg.seed)
    run_and_compare(shards, cfg.D, cfg.H, cfg.W, vr, vc)


@pytest.mark.parametrize("bits", [False, True])
def test_ragged_fp32_gather_workload(bits):
    """valid extents 997 x 4999 over 1000 x 5000: row chunks [0,997)+[997,1000), column chunks
    [0,4999)+[4999,5000); raw 32-bit patterns too (NaN payloads, subnormals)."""
    cfg = workloads.TG_RAGGED
    shards = workloads.make_tgather(cfg.N, cfg.D, cfg.H, cfg.W, cfg.dtype, seed=cfg.seed, bits=bits)
    run_and_compare(shards, cfg.D, cfg.H, cfg.W, cfg.valid_rows, cfg.valid_cols)


@pytest.mark.parametrize("dtype,W", [(torch.float16, 64),    # 128-byte rows: 16-byte vector path
                                     (torch.float16, 70),    # 140-byte rows: element path
                                     (torch.uint8, 70)])
def test_largest_supported_rank_count(dtype, W):
    """64 source ranks, the most the library carries; two planes, ragged tiles."""
    N, D, H = 64, (2, 1, 1), 9
    shards = workloads.make_tgather(N, D, H, W, dtype, seed=64)
    run_and_compare(shards, D, H, W, 4, 33)


@pytest.mark.parametrize("dtype,count", [(torch.float32, 256), (torch.int32, 4096), (torch.uint8, 512)])
def test_page_matrix_basic(dtype, count):
    """§九 basic: per-rank [1,1,1,1,count], value i + rank*10000 (wrapping for uint8)."""
    N = 8
    shards = [((torch.arange(count, dtype=torch.int64) + r * 10000) % (256 if dtype == torch.uint8 else 2 ** 31))
              .to(dtype).reshape(1, 1, 1, 1, count) for r in range(N)]
    run_and_compare(shards, (1, 1, 1), 1, count, 1, count)


@pytest.mark.parametrize("dtype,rows,cols,tile_rows", [(torch.int32, 128, 32, 16),
                                                       (torch.float32, 256, 64, 32),
                                                       (torch.int32, 512, 32, 64)])
def test_page_matrix_large_chunked(dtype, rows, cols, tile_rows):
    """§九 large-shape chunked cases (static tiles with rows % tile_rows == 0)."""
    shards = workloads.make_tgather(4, (1, 1, 1), rows, cols, dtype, seed=3)
    run_and_compare(shards, (1, 1, 1), rows, cols, tile_rows, cols)


def test_page_matrix_empty_keeps_destination():
    """§九 empty case: DIM_3 = 0 moves nothing, the destination keeps its initial bytes."""
    dst = torch.full((1, 1, 1, 4, 8), -1.0, device=DEV)
    shards = [torch.empty((1, 1, 1, 0, 8), device=DEV) for _ in range(4)]
    ag.tgather(shards, 1, 1, dst=dst, dst_rows=4)
    torch.cuda.synchronize()
    assert (dst == -1).all()


def test_outer_dims_and_taller_destination():
    """Outer dims interleave per plane; rows >= N*H of a taller dst stay untouched (§7.2)."""
    shards = workloads.make_tgather(3, (2, 3, 2), 5, 96, torch.float16, seed=4)
    run_and_compare(shards, (2, 3, 2), 5, 96, 2, 40, dst_rows=3 * 5 + 7, fill=0xAB)


@pytest.mark.parametrize("dtype,W,vr,vc", [(torch.uint8, 5, 3, 2),       # rows not 16-byte multiples
                                           (torch.int16, 37, 4, 10),
                                           (torch.float64, 30, 7, 11),   # 8-byte elements
                                           (torch.int32, 12, 1, 5)])
def test_element_path_and_sizes(dtype, W, vr, vc):
    shards = workloads.make_tgather(5, (1, 2, 1), 9, W, dtype, seed=5)
    run_and_compare(shards, (1, 2, 1), 9, W, vr, vc)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_random_tiles(seed):
    """Random valid extents (1, primes, > extent) and shapes; result independent of them."""
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 9))
    D = (int(rng.integers(1, 3)), 1, int(rng.integers(1, 3)))
    H = int(rng.integers(1, 200))
    W = int(rng.choice([8, 64, 100, 256, 1000, 4100]))
    dtype = [torch.float16, torch.float32, torch.uint8, torch.float64][int(rng.integers(0, 4))]
    vr = int(rng.choice([1, 7, 31, H, H + 5]))
    vc = int(rng.choice([1, 13, 127, W, W + 3]))
    shards = workloads.make_tgather(N, D, H, W, dtype, seed=seed, bits=dtype != torch.uint8)
    run_and_compare(shards, D, H, W, vr, vc)


def test_unaligned_base_pointers_take_element_path():
    base = torch.zeros(4 * 64 * 32 + 3, dtype=torch.float16, device=DEV)
    src_cpu = workloads.make_tgather(2, (1, 1, 1), 32, 64, torch.float16, seed=8)
    shards = [base[1 + r * 2048: 1 + (r + 1) * 2048].view(1, 1, 1, 32, 64) for r in range(2)]
    for s, c in zip(shards, src_cpu):
        s.copy_(c.to(DEV))
    dst = torch.empty((1, 1, 1, 64, 64), dtype=torch.float16, device=DEV)
    ag.tgather(shards, 5, 9, dst=dst)
    torch.cuda.synchronize()
    assert np.array_equal(np_bytes(dst), oracle_gather(src_cpu, (1, 1, 1), 32, 64))


@pytest.mark.slow
def test_sub_tile_spans_capped_and_destination_beyond_4_gib():
    """Rows 2 MiB apart and 16-byte-wide tiles 1100 rows tall: a sub-tile of up to 2048 such rows
    would span more than the 2 GiB its 32-bit buffer offsets reach, so the plan cuts it at 1024 rows.
    Two 2.2 GiB ranks fill a 4.4 GiB destination, so the second rank's rows lie beyond 4 GiB."""
    N, D, H, W = 2, (1, 1, 1), 1100, 2 << 20
    print("tgather large: N=%d H=%d W=%d uint8" % (N, H, W), flush=True)
    shards = workloads.make_tgather(N, D, H, W, torch.uint8, seed=77, bits=True)
    expect = oracle_gather(shards, D, H, W)
    sd = [s.to(DEV) for s in shards]
    del shards
    dst = torch.empty((1, 1, 1, N * H, W), dtype=torch.uint8, device=DEV)
    ag.tgather(sd, H, 16, dst=dst)
    torch.cuda.synchronize()
    del sd
    assert np.array_equal(np_bytes(dst), expect)
