"""FP8 output (the MatMul's FP8_OUTPUT variant, "Triton第四课：基于对称内存融合 AllGather 与 MatMul"
section MatMul 按需等待): C = e4m3fn(acc * out_scale), one byte per element, against the oracle's
E4M3 "fn" conversion.

* Bit-exact: with small integer inputs every partial sum is an integer below 2^24, so the fp32
  accumulator holds the exact sum whatever the summation order, and the FP8 code is fully decided:
  it must equal the oracle's code for the oracle's (equally exact) sum, in every schedule.  The
  scales put values on ties, into the subnormal range, past 448 (NaN), and one is not a power of
  two (the product is rounded in fp32 on both sides).
* Random data: the kernel's fp32 sum and the oracle's differ by at most the summation error, so
  the code must lie between the oracle's codes for sum - bound and sum + bound (rounding is
  monotone); that bound is 2 K 2^-24 sum|a||b| plus the scale's rounding.
"""
import numpy as np
import pytest
import torch

import allgather_gemm_amd as ag
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def codes(t):
    return t.detach().contiguous().cpu().view(torch.uint8).numpy()


def same_codes(got, want):
    """Bitwise, except that any two NaN codes (0x7F, 0xFF) count as equal."""
    nan_g = (got & 0x7F) == 0x7F
    nan_w = (want & 0x7F) == 0x7F
    return bool(np.array_equal(nan_g, nan_w) and np.array_equal(got[~nan_g], want[~nan_w]))


def run_fp8(sd, Bd, cb, scale, **kw):
    M, Nc = len(sd) * sd[0].shape[0], Bd.shape[0]
    C = torch.full((M, Nc), 0.5, dtype=torch.float8_e4m3fn, device=DEV)
    ag.ag_gemm(sd, Bd, cb, C=C, out_dtype="fp8_e4m3", out_scale=scale, **kw)
    torch.cuda.synchronize()
    rc, info = ag.check()
    assert rc == ag.AG_OK, info
    return C


@pytest.mark.parametrize("Nc", [200, 203])
def test_fp8_output_is_bit_exact_on_exact_sums_in_every_schedule(Nc):
    N, H, K, cb = 3, 100, 256, 40
    print("fp8 exact N=%d H=%d K=%d Nc=%d" % (N, H, K, Nc), flush=True)
    shards, B = workloads.make_ag_gemm_integers(N, H, K, Nc, seed=81)
    A_ref, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
    assert np.abs(C32).max() < 2 ** 24
    sd = [s.to(DEV) for s in shards]
    Bd = B.to(DEV)
    a_full = torch.from_numpy(A_ref.view(np.int16)).view(torch.bfloat16).to(DEV)
    for scale in (1.0, 4.0, 2.0 ** -4, 2.0 ** -7, 0.3):
        want = oracle.f32_to_e4m3fn((C32.astype(np.float32) * np.float32(scale)).astype(np.float32))
        for kw in ({}, {"producer": "in_kernel"}, {"producer": "copy_engine"}, {"mode": "unfused"},
                   {"mode": "plain_gemm", "a_out": a_full}, {"mode": "gemm_only", "a_out": a_full},
                   {"local_rank": 2}):
            got = codes(run_fp8(sd, Bd, cb, scale, **kw))
            assert same_codes(got, want), (scale, kw, int((got != want).sum()))
    # the scales above reach every class of code: subnormals, ties, and overflow to NaN
    small = oracle.f32_to_e4m3fn((C32.astype(np.float32) * np.float32(2.0 ** -7)).astype(np.float32))
    assert ((small & 0x78) == 0).any() and not ((small & 0x7F) == 0x7F).any()
    big = oracle.f32_to_e4m3fn((C32.astype(np.float32) * np.float32(4.0)).astype(np.float32))
    assert ((big & 0x7F) == 0x7F).any()
    odd = C32[(np.abs(C32) >= 16) & (np.abs(C32) < 32)]
    assert (odd % 2 == 1).any()                  # ties at scale 1 (spacing 2 in [16, 32))


def bracket_ok(got, c, e):
    lo = oracle.e4m3fn_value(oracle.f32_to_e4m3fn((c - e).astype(np.float32)))
    hi = oracle.e4m3fn_value(oracle.f32_to_e4m3fn((c + e).astype(np.float32)))
    v = oracle.e4m3fn_value(got)
    ok = (v >= lo) & (v <= hi)
    return bool(ok.all()), int((~ok).sum())


def test_fp8_output_random_data_within_the_summation_error():
    N, H, K, Nc, cb = 4, 160, 512, 264, 48
    print("fp8 random N=%d H=%d K=%d Nc=%d" % (N, H, K, Nc), flush=True)
    A, shards, B = workloads.make_ag_gemm_shapes(N, H, K, Nc, seed=82, b_std=0.5)
    _, C32 = oracle.ag_gemm([u16(s) for s in shards], u16(B))
    absAB = np.abs(A.float().numpy().astype(np.float64)) @ np.abs(B.float().numpy().astype(np.float64)).T
    sd = [s.to(DEV) for s in shards]
    Bd = B.to(DEV)
    for scale in (1.0, 0.7):
        c = C32.astype(np.float64) * scale
        e = 2.0 * K * 2.0 ** -24 * absAB * scale + np.abs(c) * 2.0 ** -23
        for kw in ({}, {"mode": "unfused"}):
            ok, bad = bracket_ok(codes(run_fp8(sd, Bd, cb, scale, **kw)), c, e)
            assert ok, (scale, kw, bad)


@pytest.mark.slow
def test_fp8_output_full_size_square_workload_sampled():
    cfg = workloads.AG_SQUARE
    print("fp8 full size %s" % cfg.name, flush=True)
    A, shards, B = workloads.make_ag_gemm(cfg)
    sd = [s.to(DEV) for s in shards]
    Bd = B.to(DEV)
    got = codes(run_fp8(sd, Bd, cfg.cb, 4.0))
    rng = np.random.default_rng(83)
    ms = rng.integers(0, cfg.M, 3000)
    ns = rng.integers(0, cfg.Nc, 3000)
    c32 = oracle.ag_gemm_at([u16(s) for s in shards], u16(B), ms, ns)
    Af = A.float().numpy()
    Bf = B.float().numpy()
    absAB = np.einsum("ik,ik->i", np.abs(Af[ms]).astype(np.float64), np.abs(Bf[ns]).astype(np.float64))
    c = c32.astype(np.float64) * 4.0
    e = 2.0 * cfg.K * 2.0 ** -24 * absAB * 4.0 + np.abs(c) * 2.0 ** -23
    ok, bad = bracket_ok(got[ms, ns], c, e)
    assert ok, bad
