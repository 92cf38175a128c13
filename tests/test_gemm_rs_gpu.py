"""GEMM + ReduceScatter, one rank's share ("Triton第四课：基于对称内存融合 AllGather 与 MatMul",
section 从集合通信理解数据流), through the library against the oracle.

* Exact: with small integer inputs the partial product and the reduction are exact in fp32 in any
  order, so P and out must equal the oracle's bit for bit, fused and unfused, for every local rank;
  the blocks (H = 200 rows) straddle GEMM tile rows (256).
* Random data: P within the GEMM tolerance of the oracle's fp32 sums; out exactly the oracle's
  reduction of the GPU's own P block and the peers' partials (the reduction itself has one
  correct result); fused and unfused bitwise equal.
* Full size (the square workload split over 8 ranks): P at sampled elements, out on the whole block.
"""
import numpy as np
import pytest
import torch

import allgather_gemm_amd as ag
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
RTOL, ATOL = 1.6e-2, 1e-2


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def run(A, B, recv, local, fused):
    Ad, Bd = A.to(DEV), B.to(DEV)
    rd = [None if r is None else r.to(DEV) for r in recv]
    M, Nc = A.shape[0], B.shape[0]
    H = M // len(recv)
    P = torch.full((M, Nc), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = torch.full((H, Nc), float("nan"), dtype=torch.bfloat16, device=DEV)
    ag.gemm_rs(Ad, Bd, rd, local, P=P, out=out, fused=fused)
    torch.cuda.synchronize()
    rc, info = ag.check()
    assert rc == ag.AG_OK, info
    return u16(P), u16(out)


def test_gemm_rs_exact_integers_every_rank_fused_and_unfused():
    N, H, K, Nc = 3, 200, 64, 264
    print("gemm_rs exact N=%d H=%d K=%d Nc=%d" % (N, H, K, Nc), flush=True)
    shards, B = workloads.make_ag_gemm_integers(1, N * H, K, Nc, seed=91, lim=2)
    A = shards[0]
    peers, _ = workloads.make_ag_gemm_integers(N, H, Nc, 8, seed=92, lim=30)   # (H, Nc) integer blocks
    for local in range(N):
        recv = [None if j == local else peers[j] for j in range(N)]
        P_ref, out_ref = oracle.gemm_rs(u16(A), u16(B), [None if r is None else u16(r) for r in recv], local)
        for fused in (True, False):
            P, out = run(A, B, recv, local, fused)
            assert np.array_equal(P, P_ref), (local, fused)
            assert np.array_equal(out, out_ref), (local, fused)


@pytest.mark.parametrize("N,H,local", [(1, 300, 0),     # one rank: the reduction is its own block
                                       (64, 8, 0),      # the most ranks the library carries
                                       (64, 8, 63)])
def test_gemm_rs_exact_integers_rank_count_extremes(N, H, local):
    K, Nc = 48, 40
    print("gemm_rs exact N=%d H=%d local=%d" % (N, H, local), flush=True)
    shards, B = workloads.make_ag_gemm_integers(1, N * H, K, Nc, seed=94, lim=2)
    A = shards[0]
    peers, _ = workloads.make_ag_gemm_integers(N, H, Nc, 8, seed=95, lim=30)
    recv = [None if j == local else peers[j] for j in range(N)]
    P_ref, out_ref = oracle.gemm_rs(u16(A), u16(B), [None if r is None else u16(r) for r in recv], local)
    for fused in (True, False):
        P, out = run(A, B, recv, local, fused)
        assert np.array_equal(P, P_ref), fused
        assert np.array_equal(out, out_ref), fused


def check_random(cfg, sample=None):
    A, B, recv = workloads.make_gemm_rs(cfg)
    H = cfg.H
    recv_bits = [None if r is None else u16(r) for r in recv]
    P_f, out_f = run(A, B, recv, cfg.local, True)
    P_u, out_u = run(A, B, recv, cfg.local, False)
    assert np.array_equal(P_f, P_u) and np.array_equal(out_f, out_u)
    # the reduction: exactly the oracle's, given this P block
    parts = [P_f[cfg.local * H:(cfg.local + 1) * H] if j == cfg.local else recv_bits[j] for j in range(cfg.N)]
    assert np.array_equal(out_f, oracle.reduce_block(parts))
    # the partial product against the oracle's fp32 sums
    P = bits_to_bf16(P_f).float().numpy().astype(np.float64)
    if sample is None:
        C32 = oracle.gemm_f32(u16(A), u16(B)).astype(np.float64)
        err = np.abs(P - C32) - (ATOL + RTOL * np.abs(C32))
    else:
        rng = np.random.default_rng(93)
        ms = rng.integers(0, cfg.M, sample)
        ns = rng.integers(0, cfg.Nc, sample)
        c32 = oracle.ag_gemm_at([u16(A)], u16(B), ms, ns).astype(np.float64)
        err = np.abs(P[ms, ns] - c32) - (ATOL + RTOL * np.abs(c32))
    assert (err <= 0).all(), float(err.max())


def test_gemm_rs_random_tiny():
    print("gemm_rs %s" % workloads.RS_TINY.name, flush=True)
    check_random(workloads.RS_TINY)


@pytest.mark.parametrize("local", [0, 3])
def test_gemm_rs_random_ragged(local):
    cfg = workloads.GemmRsConfig("gemm_rs_ragged", N=4, M=4 * 300, K=520, Nc=392, local=local, b_std=0.1)
    print("gemm_rs ragged local=%d" % local, flush=True)
    check_random(cfg)


@pytest.mark.slow
def test_gemm_rs_full_size_square_workload():
    print("gemm_rs %s" % workloads.RS_SQUARE.name, flush=True)
    check_random(workloads.RS_SQUARE, sample=4000)
