"""The C ABI's own entry points with data on the GPU, called through ctypes exactly as a C caller
would (no Python wrapper in between): ag_gemm, ag_gemm_unfused, ag_gemm_ex, tgather, tgather_ex,
ag_check.  Results against the CPU oracle."""
import ctypes

import numpy as np
import pytest
import torch

import allgather_gemm_amd as ag
import oracle
import workloads

pytestmark = pytest.mark.gpu

_vp = ctypes.c_void_p
RTOL, ATOL = 1.6e-2, 1e-2


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def ptrs(ts):
    return ctypes.cast((_vp * len(ts))(*[t.data_ptr() for t in ts]), _vp)


def close(C, C32):
    got = C.float().cpu().numpy().astype(np.float64)
    return bool((np.abs(got - C32) <= ATOL + RTOL * np.abs(C32)).all())


def test_ag_gemm_and_unfused_through_the_c_abi():
    N, H, K, Nc, cb = 4, 96, 200, 136, 40
    print("C ABI ag_gemm N=%d H=%d K=%d Nc=%d cb=%d" % (N, H, K, Nc, cb), flush=True)
    A, shards, B = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=31)
    _, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
    sd = [s.cuda() for s in shards]
    Bd = B.cuda()
    L = ag.lib()
    stream = torch.cuda.current_stream().cuda_stream
    C1 = torch.full((N * H, Nc), float("nan"), dtype=torch.bfloat16, device="cuda")
    C2 = torch.full_like(C1, float("nan"))
    assert L.ag_gemm(ptrs(sd), N, N * H, K, Bd.data_ptr(), Nc, C1.data_ptr(), cb, stream) == ag.AG_OK
    assert L.ag_gemm_unfused(ptrs(sd), N, N * H, K, Bd.data_ptr(), Nc, C2.data_ptr(), cb, stream) == ag.AG_OK
    info = (ctypes.c_int64 * 4)()
    assert L.ag_check(stream, info) == ag.AG_OK
    torch.cuda.synchronize()
    assert close(C1, C32) and close(C2, C32)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))


@pytest.mark.parametrize("producer", [0, 1, 2])
def test_ag_gemm_ex_producers_through_the_c_abi(producer):
    N, H, K, Nc, cb = 3, 128, 256, 264, 32
    print("C ABI ag_gemm_ex producer=%d" % producer, flush=True)
    A, shards, B = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=32)
    A_ref, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
    sd = [s.cuda() for s in shards]
    Bd = B.cuda()
    a_out = torch.full((N * H, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    C = torch.empty((N * H, Nc), dtype=torch.bfloat16, device="cuda")
    opt = ag.AgOptions(0, 2, a_out.data_ptr(), 0, 0, 0, producer)
    stream = torch.cuda.current_stream().cuda_stream
    assert ag.lib().ag_gemm_ex(ptrs(sd), N, N * H, K, Bd.data_ptr(), Nc, C.data_ptr(), cb, stream,
                               ctypes.byref(opt)) == ag.AG_OK
    torch.cuda.synchronize()
    assert np.array_equal(u16(a_out), A_ref)
    assert close(C, C32)


def test_tgather_and_tgather_ex_through_the_c_abi():
    N, D, H, W = 3, (2, 1, 1), 7, 48
    print("C ABI tgather", flush=True)
    src = workloads.make_tgather(N, D, H, W, torch.float32, seed=33)
    sd = [s.cuda() for s in src]
    expect = np.zeros(D[0] * N * H * W, dtype=np.float32)
    oracle.tgather([s.numpy() for s in src], expect, *D, H, W)
    L = ag.lib()
    stream = torch.cuda.current_stream().cuda_stream
    dst = torch.full((D[0], 1, 1, N * H, W), -1.0, device="cuda")
    assert L.tgather(ptrs(sd), N, dst.data_ptr(), *D, H, W, 3, 20, 4, stream) == ag.AG_OK
    tall = torch.full((D[0], 1, 1, N * H + 5, W), -1.0, device="cuda")
    assert L.tgather_ex(ptrs(sd), N, tall.data_ptr(), *D, H, W, N * H + 5, 2, 33, 4, N - 1, stream) == ag.AG_OK
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().reshape(-1).view(np.uint32), expect.view(np.uint32))
    t = tall.cpu().numpy()
    assert np.array_equal(t[:, :, :, :N * H].reshape(-1).view(np.uint32), expect.view(np.uint32))
    assert (t[:, :, :, N * H:] == -1).all()
