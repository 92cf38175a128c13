"""AG-GEMM on the GPU against the CPU oracle.

C must be within |gpu - C32| <= 1e-2 + 1.6e-2 * |C32| of the oracle's fp32-accumulated result,
element by element at every size (the full workloads through the oracle's blocked loop order,
which is bitwise its naive one).  The gathered A must equal the oracle's gather bit for bit.  The
fused (every producer), unfused and GEMM-only schedules share the tile code and k order, so their
C must agree bit for bit with each other.
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


PRODUCERS = ("side_stream", "in_kernel", "copy_engine")   # the first is the default


def assert_close_on_device(C_gpu: torch.Tensor, C32: np.ndarray, where=""):
    """Element-wise check of a large C: the oracle's values go to the device and every element is
    compared there (in row blocks, to bound memory)."""
    M = C32.shape[0]
    step = max(1, (1 << 26) // max(1, C32.shape[1]))
    bad_total = 0
    worst = 0.0
    for m0 in range(0, M, step):
        ref = torch.from_numpy(C32[m0:m0 + step]).to(C_gpu.device).double()
        got = C_gpu[m0:m0 + step].double()
        assert not torch.isnan(got).any(), "NaN in C " + where
        err = (got - ref).abs()
        bound = ATOL + RTOL * ref.abs()
        bad_total += int((err > bound).sum())
        worst = max(worst, float((err - bound).max()))
    assert bad_total == 0, "%d elements out of tolerance %s (worst excess %g)" % (bad_total, where, worst)


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
    for producer in PRODUCERS[1:]:
        a2 = torch.full((cfg.M, cfg.K), float("nan"), dtype=torch.bfloat16, device=DEV)
        C_p = run(sd, Bd, cfg.cb, local_rank=local_rank, a_out=a2, producer=producer)
        assert np.array_equal(u16(a2), A_ref), producer
        assert torch.equal(C_f.view(torch.int16), C_p.view(torch.int16)), producer
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
    C_u = run(sd, Bd, cb, mode="unfused")
    assert_close_to_oracle(C_u, C32, "unfused")
    for producer in PRODUCERS:
        a_out = torch.full((N * H, K), float("nan"), dtype=torch.bfloat16, device=DEV)
        C_f = run(sd, Bd, cb, local_rank=local, a_out=a_out, producer=producer)
        assert np.array_equal(u16(a_out), A_ref), producer
        assert torch.equal(C_f.view(torch.int16), C_u.view(torch.int16)), producer
    assert ag.check()[0] == ag.AG_OK


def test_largest_supported_k_is_exact():
    """K = 2^21, the largest the library accepts: a full 256-row tile then spans 1 GiB of A (its
    buffer offsets are 32-bit) and one workgroup runs 32768 K steps.  Entries in {-1, 0, 1} keep every
    partial sum an integer of magnitude at most 2^21, exact in fp32 in any order, so C must equal the
    oracle's rounding bit for bit in every schedule, and the gathered A the shards' bytes."""
    N, H, K, Nc, cb = 2, 128, 1 << 21, 24, 50
    print("AG-GEMM largest K: N=%d H=%d K=%d Nc=%d" % (N, H, K, Nc), flush=True)
    shards, B = workloads.make_ag_gemm_integers(N, H, K, Nc, seed=23, lim=1)
    A_ref, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
    assert np.abs(C32).max() <= K
    want = oracle.f32_to_bf16(C32)
    sd, Bd = [s.to(DEV) for s in shards], B.to(DEV)
    del shards
    a_out = torch.empty((N * H, K), dtype=torch.bfloat16, device=DEV)
    for kw in [{"producer": p} for p in PRODUCERS] + [{"mode": "unfused"}, {"local_rank": 1}]:
        a_out.fill_(float("nan"))
        C = run(sd, Bd, cb, a_out=a_out, **kw)
        assert np.array_equal(u16(C), want), kw
        if kw.get("mode") != "unfused":
            assert np.array_equal(u16(a_out), A_ref), kw
    C = run(sd, Bd, cb, a_out=a_out, mode="plain_gemm")
    assert np.array_equal(u16(C), want)
    assert ag.check()[0] == ag.AG_OK


@pytest.mark.slow
def test_gathered_a_beyond_4_gib():
    """A 4.5 GiB gathered A (2304 rows of 2 MiB): pieces, chunk rows and tile rows sit beyond 4 GiB,
    so every offset into it must be 64-bit.  Integer inputs in {-1, 0, 1}: C exact, bit for bit."""
    N, H, K, Nc, cb = 2, 1152, 1 << 20, 24, 100
    print("AG-GEMM gathered A beyond 4 GiB: N=%d H=%d K=%d Nc=%d" % (N, H, K, Nc), flush=True)
    shards, B = workloads.make_ag_gemm_integers(N, H, K, Nc, seed=29, lim=1)
    C32 = oracle.ag_gemm_fast([u16(s) for s in shards], u16(B))
    want = oracle.f32_to_bf16(C32)
    sd, Bd = [s.to(DEV) for s in shards], B.to(DEV)
    del shards
    a_out = torch.empty((N * H, K), dtype=torch.bfloat16, device=DEV)
    for kw in ({}, {"producer": "in_kernel"}, {"mode": "unfused"}):
        a_out.fill_(float("nan"))
        C = run(sd, Bd, cb, a_out=a_out, **kw)
        assert np.array_equal(u16(C), want), kw
        if kw.get("mode") != "unfused":
            for r in range(N):     # the gathered A, rank by rank, against the shards' bits
                assert torch.equal(a_out[r * H:(r + 1) * H].view(torch.int16), sd[r].view(torch.int16)), (kw, r)
    assert ag.check()[0] == ag.AG_OK


def test_largest_supported_shard_count():
    """N = 64 shards, the most the library carries in its kernel arguments, the local shard the last
    one; 20-row shards (tiles straddle up to 13 shards), 3 chunks per shard, ragged Nc."""
    N, H, K, Nc, cb, local = 64, 20, 96, 136, 7, 63
    print("AG-GEMM N=%d H=%d K=%d Nc=%d cb=%d local=%d" % (N, H, K, Nc, cb, local), flush=True)
    A, shards, B = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=64)
    A_ref, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
    sd, Bd = to_dev(A, shards, B)
    C_u = run(sd, Bd, cb, mode="unfused")
    assert_close_to_oracle(C_u, C32, "unfused")
    for producer in PRODUCERS:
        a_out = torch.full((N * H, K), float("nan"), dtype=torch.bfloat16, device=DEV)
        C_f = run(sd, Bd, cb, local_rank=local, a_out=a_out, producer=producer)
        assert np.array_equal(u16(a_out), A_ref), producer
        assert torch.equal(C_f.view(torch.int16), C_u.view(torch.int16)), producer
    assert ag.check()[0] == ag.AG_OK


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


@pytest.mark.parametrize("producer", PRODUCERS)
def test_call_after_a_timed_out_call_needs_no_check(producer):
    """A call that gave up (no copy at all, short timeout: every kernel still exits by itself) is
    followed by normal calls without ag_check in between: they must not inherit its failure or its
    half-counted chunks, and ag_check must still report the earlier give-up."""
    N, H, K, Nc, cb = 4, 256, 128, 256, 64
    print("timeout then %s" % producer, flush=True)
    A, shards, B = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=6)
    A_ref, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
    sd, Bd = to_dev(A, shards, B)
    ag.ag_gemm(sd, Bd, cb, skip_producer=True, timeout_us=2000, local_rank=1)
    for rep in range(2):
        a_out = torch.full((N * H, K), float("nan"), dtype=torch.bfloat16, device=DEV)
        C = run(sd, Bd, cb, a_out=a_out, producer=producer, local_rank=rep)
        assert np.array_equal(u16(a_out), A_ref), rep
        assert_close_to_oracle(C, C32, "call %d after the time-out" % rep)
    rc, info = ag.check()
    assert rc == ag.AG_ETIMEOUT and info[0] == 1
    assert ag.check()[0] == ag.AG_OK


@pytest.mark.parametrize("producer", PRODUCERS)
def test_new_shard_contents_every_call(producer):
    """Alternating inputs through one gathered buffer: every call must see its own shards' rows,
    never rows an earlier call left in the buffer or in a cache."""
    N, H, K, Nc, cb = 8, 160, 256, 512, 32
    print("alternating inputs %s" % producer, flush=True)
    sets = []
    for seed in (41, 42):
        A, shards, B = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=seed)
        A_ref, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
        sd, Bd = to_dev(A, shards, B)
        sets.append((sd, Bd, A_ref, C32))
    a_out = torch.empty((N * H, K), dtype=torch.bfloat16, device=DEV)
    for i in range(5):
        sd, Bd, A_ref, C32 = sets[i % 2]
        for buf in (a_out, None):
            C = run(sd, Bd, cb, a_out=buf, producer=producer, local_rank=i % N)
            if buf is not None:
                assert np.array_equal(u16(buf), A_ref), i
            assert_close_to_oracle(C, C32, "call %d" % i)
    assert ag.check()[0] == ag.AG_OK


def test_more_tiles_than_compute_units_every_producer():
    """400 output tiles (more than one per CU, so later waves of the persistent grid run), comm
    blocks that straddle tiles and shards, element-wise against the oracle for every producer and
    two local shards."""
    N, H, K, Nc, cb = 8, 640, 512, 5120, 160
    A, shards, B = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=7, b_std=0.05)
    A_ref = np.zeros((N * H, K), dtype=np.uint16)
    oracle.tgather([u16(s) for s in shards], A_ref, 1, 1, 1, H, K)
    C32 = oracle.ag_gemm_fast([u16(s) for s in shards], u16(B))
    sd, Bd = to_dev(A, shards, B)
    ref = None
    for producer in PRODUCERS:
        for local in (0, 5):
            print("400 tiles %s local=%d" % (producer, local), flush=True)
            a_out = torch.full((N * H, K), float("nan"), dtype=torch.bfloat16, device=DEV)
            C = run(sd, Bd, cb, a_out=a_out, producer=producer, local_rank=local)
            assert np.array_equal(u16(a_out), A_ref)
            if ref is None:
                assert_close_on_device(C, C32, producer)
                ref = C.clone()
            else:
                assert torch.equal(C.view(torch.int16), ref.view(torch.int16)), (producer, local)
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


# ------------------------------------------------------------------------------ full size
@pytest.mark.parametrize("cfg", [workloads.AG_SQUARE, workloads.AG_MLP_UP, workloads.AG_RAGGED],
                         ids=lambda c: c.name)
def test_full_size_workloads_every_element(cfg):
    """The three full workloads: every element of C against the oracle; the gathered A bit for bit;
    fused (each producer), unfused and GEMM-only C bit for bit equal."""
    print("full-size %s: oracle" % cfg.name, flush=True)
    A, shards, B = workloads.make_ag_gemm(cfg)
    C32 = oracle.ag_gemm_fast([u16(s) for s in shards], u16(B))
    print("full-size %s: GPU" % cfg.name, flush=True)
    sd, Bd = to_dev(A, shards, B)
    A_d = A.to(DEV)
    a_out = torch.full((cfg.M, cfg.K), float("nan"), dtype=torch.bfloat16, device=DEV)
    C_f = run(sd, Bd, cfg.cb, a_out=a_out)
    assert torch.equal(a_out.view(torch.int16), A_d.view(torch.int16))   # gathered A exact
    assert_close_on_device(C_f, C32, "fused")
    C_u = run(sd, Bd, cfg.cb, mode="unfused")
    assert torch.equal(C_f.view(torch.int16), C_u.view(torch.int16))
    C_g = run(sd, Bd, cfg.cb, mode="gemm_only", a_out=a_out)
    assert torch.equal(C_f.view(torch.int16), C_g.view(torch.int16))
    for producer in PRODUCERS[1:]:
        a_out.fill_(float("nan"))
        C_p = run(sd, Bd, cfg.cb, a_out=a_out, producer=producer, local_rank=3)
        assert torch.equal(a_out.view(torch.int16), A_d.view(torch.int16)), producer
        assert torch.equal(C_f.view(torch.int16), C_p.view(torch.int16)), producer
    assert ag.check()[0] == ag.AG_OK


def test_wait_statistics_account_for_every_waiting_tile():
    """The fused GEMM's wait counters (a measurement aid): every non-local tile either waits or
    skips its wait, nothing is copied when every flag is already raised, and in-kernel copying shows
    up as pieces copied by waiting tiles."""
    N, H, K, Nc, cb = 4, 256, 256, 512, 64
    print("wait statistics", flush=True)
    A, shards, B = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=17)
    sd, Bd = to_dev(A, shards, B)
    a_out = A.to(DEV)
    tiles_nonlocal = (N - 1) * (H // 256) * (Nc // 256)       # local shard 0: one tile row of 4
    st = torch.zeros(4, dtype=torch.int64, device=DEV)
    ag.ag_gemm(sd, Bd, cb, a_out=a_out, mode="gemm_only", wait_stats=st)
    torch.cuda.synchronize()
    ticks, waits, copied, skipped = st.cpu().tolist()
    assert waits + skipped == tiles_nonlocal and copied == 0 and ticks >= 0
    st.zero_()
    a2 = torch.empty_like(a_out)
    ag.ag_gemm(sd, Bd, cb, a_out=a2, producer="in_kernel", wait_stats=st)
    torch.cuda.synchronize()
    ticks, waits, copied, skipped = st.cpu().tolist()
    assert waits + skipped == tiles_nonlocal and waits >= 1 and ticks > 0
    assert torch.equal(a2.view(torch.int16), a_out.view(torch.int16))
    assert ag.check()[0] == ag.AG_OK
