"""ag_gemm_noalloc (the entry point for callers that cannot allocate) through the C ABI, called with
ctypes as a C caller would, against the existing entry point ag_gemm_ex on the same inputs: the
gathered A bit for bit and C bit for bit (both run the same GEMM tiles in the same k order), on two
calls in a row, the second with a smaller input, so the second call starts from the first call's
left-over control words.  Also the chunk limit, rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import allgather_gemm_amd as ag
import oracle
import workloads

pytestmark = pytest.mark.gpu

_vp = ctypes.c_void_p


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def ptrs(ts):
    return ctypes.cast((_vp * len(ts))(*[t.data_ptr() for t in ts]), _vp)


def run_both(N, H, K, Nc, cb, local, seed):
    """One ag_gemm_noalloc call and one ag_gemm_ex call on the same inputs; returns both results."""
    print("noalloc vs ag_gemm_ex N=%d H=%d K=%d Nc=%d cb=%d local=%d" % (N, H, K, Nc, cb, local), flush=True)
    A, shards, B = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=seed)
    sd = [s.cuda() for s in shards]
    Bd = B.cuda()
    M = N * H
    L = ag.lib()
    stream = torch.cuda.current_stream().cuda_stream
    a_na = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    C_na = torch.full((M, Nc), float("nan"), dtype=torch.bfloat16, device="cuda")
    assert L.ag_gemm_noalloc(ptrs(sd), N, M, K, Bd.data_ptr(), Nc, C_na.data_ptr(), cb, a_na.data_ptr(),
                             local, stream) == ag.AG_OK
    info = (ctypes.c_int64 * 4)()
    assert L.ag_check(stream, info) == ag.AG_OK, list(info)
    a_ex = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    C_ex = torch.full((M, Nc), float("nan"), dtype=torch.bfloat16, device="cuda")
    opt = ag.AgOptions(ag.MODE_FUSED, local, a_ex.data_ptr(), 0, 0, 0, ag.PRODUCER_SIDE_STREAM)
    assert L.ag_gemm_ex(ptrs(sd), N, M, K, Bd.data_ptr(), Nc, C_ex.data_ptr(), cb, stream,
                        ctypes.byref(opt)) == ag.AG_OK
    assert L.ag_check(stream, info) == ag.AG_OK, list(info)
    torch.cuda.synchronize()
    return A, shards, B, a_na, C_na, a_ex, C_ex


def test_noalloc_matches_ag_gemm_ex_on_two_calls_the_second_smaller():
    # first call: 6 shards of 200 rows, 25 chunks per shard, tiles straddling shards and chunks
    A, _, _, a_na, C_na, a_ex, C_ex = run_both(N=6, H=200, K=320, Nc=392, cb=8, local=4, seed=71)
    assert torch.equal(a_na.view(torch.int16), a_ex.view(torch.int16))
    assert np.array_equal(u16(a_na), u16(A))
    assert torch.equal(C_na.view(torch.int16), C_ex.view(torch.int16))
    # second call, smaller in every extent: fewer chunks than the first call left flags and counts for
    A, shards, B, a_na, C_na, a_ex, C_ex = run_both(N=3, H=72, K=128, Nc=136, cb=20, local=1, seed=72)
    assert torch.equal(a_na.view(torch.int16), a_ex.view(torch.int16))
    assert np.array_equal(u16(a_na), u16(A))
    assert torch.equal(C_na.view(torch.int16), C_ex.view(torch.int16))
    # and C against the oracle, to the tolerance of the other parity tests
    _, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
    got = C_na.float().cpu().numpy().astype(np.float64)
    assert (np.abs(got - C32) <= 1e-2 + 1.6e-2 * np.abs(C32)).all()


def test_noalloc_rejects_more_chunks_than_its_array_holds():
    # one row per chunk: 2 shards of 16385 rows are 32770 chunks, two more than the array holds
    L = ag.lib()
    N, H, K, Nc = 2, 16385, 8, 8
    t = torch.zeros(16, dtype=torch.bfloat16, device="cuda")   # never read: rejected before launch
    p = t.data_ptr()
    shards = (_vp * N)(p, p)
    rc = L.ag_gemm_noalloc(ctypes.cast(shards, _vp), N, N * H, K, p, Nc, p, 1, p, 0, None)
    assert rc == ag.AG_EUNSUPPORTED
