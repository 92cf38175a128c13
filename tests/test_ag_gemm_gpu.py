"""AG-GEMM on the GPU against the CPU oracle.

C must be within |gpu - C32| <= 1e-2 + 1.6e-2 * |C32| of the oracle's fp32-accumulated result
(element by element at small sizes; at the full workload sizes on sampled elements, the tile,
chunk and shard boundaries included).  The gathered A must equal the oracle's gather bit for bit.
The fused, unfused and GEMM-only schedules share the tile code and k order, so their C must agree
bit for bit with each other.
"""
import numpy as np
import pytest
import torch

import allgather_gemm_amd as ag
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"
RTOL, ATOL = 1.6e-2, 1e-2


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def assert_close_to_oracle(C_gpu: torch.Tensor, C32: np.ndarray, where=""):
    got = C_gpu.float().cpu().numpy()
    err = np.abs(got.astype(np.float64) - C32.astype(np.float64))
    bound = ATOL + RTOL * np.abs(C32.astype(np.float64))
    bad = err > bound
    assert not np.isnan(got).any(), "NaN in C " + where
    assert not bad.any(), "%d elements out of tolerance %s, worst %g at %s" % (
        bad.sum(), where, float(err.max()), np.unravel_index(np.argmax(err - bound), err.shape))


def to_dev(A, shards, B):
    return [s.to(DEV) for s in shards], B.to(DEV)


def run(shards_d, B_d, cb, **kw):
    C = ag.ag_gemm(shards_d, B_d, cb, **kw)
    torch.cuda.synchronize()
    return C


# ------------------------------------------------------------------------------ small, full check
@pytest.mark.parametrize("local_rank", [0, 1, 2, 3])
def test_tiny_workload_all_schedules(local_rank):
    cfg = workloads.AG_TINY
    print("tiny AG-GEMM local_rank=%d" % local_rank, flush=True)
    A, shards, B = workloads.make_ag_gemm(cfg)
    A_ref, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
    sd, Bd = to_dev(A, shards, B)
    a_out = torch.full((cfg.M, cfg.K), float("nan"), dtype=torch.bfloat16, device=DEV)
    C_f = run(sd, Bd, cfg.cb, local_rank=local_rank, a_out=a_out)
    assert np.array_equal(u16(a_out), A_ref)
    assert_close_to_oracle(C_f, C32, "fused")
    C_u = run(sd, Bd, cfg.cb, mode="unfused")
    C_g = run(sd, Bd, cfg.cb, mode="gemm_only", local_rank=local_rank, a_out=a_out)
    assert torch.equal(C_f.view(torch.int16), C_u.view(torch.int16))
    assert torch.equal(C_f.view(torch.int16), C_g.view(torch.int16))
    rc, info = ag.check()
    assert rc == ag.AG_OK, info


@pytest.mark.parametrize("N,H,K,Nc,cb,local", [
    (4, 64, 128, 128, 1, 1),        # one row per comm block
    (4, 64, 128, 128, 24, 2),       # comm block does not divide H (short last chunk)
    (4, 64, 128, 128, 64, 3),       # one comm block per shard
    (3, 100, 200, 72, 7, 1),        # M, Nc, K all ragged against the 256x256x64 tile
    (8, 50, 64, 300, 10, 5),        # tiles straddle chunks and shards, Nc not a multiple of 8
    (1, 300, 40, 260, 33, 0),       # one shard: every tile local
    (5, 200, 136, 514, 64, 4),      # odd number of K steps, Nc % 8 == 2
    (2, 512, 1024, 512, 128, 1),    # several tiles in both dims, 16 K steps
])
def test_edge_shapes_full_check(N, H, K, Nc, cb, local):
    print("AG-GEMM N=%d H=%d K=%d Nc=%d cb=%d local=%d" % (N, H, K, Nc, cb, local), flush=True)
    A, shards, B = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=N * 1000 + H)
    A_ref, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
    sd, Bd = to_dev(A, shards, B)
    a_out = torch.full((N * H, K), float("nan"), dtype=torch.bfloat16, device=DEV)
    C_f = run(sd, Bd, cb, local_rank=local, a_out=a_out)
    assert np.array_equal(u16(a_out), A_ref)
    assert_close_to_oracle(C_f, C32)
    C_u = run(sd, Bd, cb, mode="unfused")
    assert torch.equal(C_f.view(torch.int16), C_u.view(torch.int16))


def test_zero_k_gives_zero():
    shards = [torch.empty((16, 0), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    B = torch.empty((24, 0), dtype=torch.bfloat16, device=DEV)
    C = torch.full((32, 24), 7.0, dtype=torch.bfloat16, device=DEV)
    ag.ag_gemm(shards, B, 4, C=C)
    torch.cuda.synchronize()
    assert (C == 0).all()


def test_reverse_claim_order_and_poison():
    """Stress: the copy claims chunks in reverse ready order, so early tiles find their chunks
    last; the aggregate buffer starts as NaN, so any early read would poison C.  C must equal
    the normal fused result bit for bit."""
    N, H, K, Nc, cb = 8, 256, 512, 512, 32
    A, shards, B = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=21)
    sd, Bd = to_dev(A, shards, B)
    ref = run(sd, Bd, cb, local_rank=2).clone()
    for rep in range(3):
        a_out = torch.full((N * H, K), float("nan"), dtype=torch.bfloat16, device=DEV)
        C = run(sd, Bd, cb, local_rank=2, a_out=a_out, reverse_order=True)
        assert torch.equal(C.view(torch.int16), ref.view(torch.int16)), rep
        assert torch.equal(a_out.view(torch.int16), A.to(DEV).view(torch.int16))
    A_ref, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
    assert_close_to_oracle(ref, C32)


def test_wait_times_out_instead_of_hanging():
    """With no producer and stale flags every non-local tile's wait must give up by itself and
    the status word must say so; the next call runs normally."""
    N, H, K, Nc, cb = 4, 256, 128, 256, 64
    A, shards, B = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=5)
    sd, Bd = to_dev(A, shards, B)
    run(sd, Bd, cb, skip_producer=True, timeout_us=2000)
    rc, info = ag.check()
    assert rc == ag.AG_ETIMEOUT and info[0] == 1
    rc, info = ag.check()
    assert rc == ag.AG_OK
    C = run(sd, Bd, cb)
    _, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
    assert_close_to_oracle(C, C32)
    assert ag.check()[0] == ag.AG_OK


def test_streams_and_back_to_back_calls():
    """Calls on two streams share the workspace: the library orders them, results stay right."""
    N, H, K, Nc, cb = 4, 128, 256, 256, 32
    A, shards, B = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=9)
    sd, Bd = to_dev(A, shards, B)
    _, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for i in range(6):
        st = s1 if i % 2 == 0 else s2
        with torch.cuda.stream(st):
            outs.append(ag.ag_gemm(sd, Bd, cb, local_rank=i % N, stream=st))
    torch.cuda.synchronize()
    for C in outs:
        assert_close_to_oracle(C, C32)


# ------------------------------------------------------------------------------ full-size, sampled
def sample_positions(M, Nc, H, cb, n_random=3000, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.integers(0, M, n_random // 3).tolist())
    for b in list(range(0, M, 256)) + list(range(0, M, H)) + list(range(0, M, cb)):
        rows.update({b, max(0, b - 1), min(M - 1, b + 1)})
    rows.add(M - 1)
    cols = set(rng.integers(0, Nc, 64).tolist()) | {0, 1, 255, 256, Nc - 1, Nc - 2}
    cols = sorted(cols)
    rows = sorted(rows)
    ms = np.array([r for r in rows for _ in range(2)], dtype=np.int64)
    ns = np.array([cols[(i * 7 + r) % len(cols)] for i, r in enumerate(ms)], dtype=np.int64)
    extra_m = rng.integers(0, M, n_random)
    extra_n = rng.integers(0, Nc, n_random)
    return np.concatenate([ms, extra_m]), np.concatenate([ns, extra_n])


@pytest.mark.parametrize("cfg", [workloads.AG_SQUARE, workloads.AG_MLP_UP, workloads.AG_RAGGED],
                         ids=lambda c: c.name)
def test_full_size_workloads_sampled(cfg):
    print("full-size %s" % cfg.name, flush=True)
    A, shards, B = workloads.make_ag_gemm(cfg)
    sd, Bd = to_dev(A, shards, B)
    a_out = torch.full((cfg.M, cfg.K), float("nan"), dtype=torch.bfloat16, device=DEV)
    C_f = run(sd, Bd, cfg.cb, a_out=a_out)
    assert torch.equal(a_out.view(torch.int16), A.to(DEV).view(torch.int16))   # gathered A exact
    C_u = run(sd, Bd, cfg.cb, mode="unfused")
    C_g = run(sd, Bd, cfg.cb, mode="gemm_only", a_out=a_out)
    assert torch.equal(C_f.view(torch.int16), C_u.view(torch.int16))
    assert torch.equal(C_f.view(torch.int16), C_g.view(torch.int16))
    assert ag.check()[0] == ag.AG_OK
    ms, ns = sample_positions(cfg.M, cfg.Nc, cfg.H, cfg.cb)
    ref = oracle.ag_gemm_at([u16(s) for s in shards], u16(B), ms, ns)
    got = C_f[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)].float().cpu().numpy()
    err = np.abs(got.astype(np.float64) - ref)
    bound = ATOL + RTOL * np.abs(ref.astype(np.float64))
    assert not np.isnan(got).any()
    assert (err <= bound).all(), "worst %g" % float((err - bound).max())
    # properties that hold everywhere: finite output
    assert torch.isfinite(C_f.float()).all()
