"""FP8 inputs: shards and B in E4M3 "fn", C = out_scale * (A B^T) in bf16 or FP8, through the library
against the oracle (the FP8 variant of "Triton第四课：基于对称内存融合 AllGather 与 MatMul", section
MatMul 按需等待, extended onto the inputs).  Every E4M3 value is exactly a bf16 value, so the oracle's
product is its bf16 GEMM on the exact bf16 images of the codes: exact products, fp32 sums.

* Bit-exact: with small integer inputs every partial sum is an integer below 2^24, exact in any
  summation order, so C (bf16, or FP8 with power-of-two scales) must equal the oracle's bit for bit
  in every schedule and producer, and the gathered A must be the shards' bytes.
* Random data: the kernel's fp32 sum and the oracle's differ by at most the summation error
  2 K 2^-24 sum|a||b|; the bf16 result must lie between the oracle's roundings of the scaled sum
  minus and plus that bound (rounding is monotone).  Fused, unfused and GEMM-only are bitwise equal.
* Full size (the square workload in FP8): sampled elements against the oracle, schedules bitwise.
"""
import numpy as np
import pytest
import torch

import allgather_gemm_amd as ag
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def b8(t):
    return t.detach().contiguous().cpu().view(torch.uint8).numpy()


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def images(codes_list):
    return [oracle.e4m3fn_to_bf16(b8(c)) for c in codes_list]


def gathered(shards):
    """The oracle's gather of the shards' bytes (TGATHER closed form, one plane)."""
    H, K = shards[0].shape
    dst = np.empty((len(shards) * H, K), dtype=np.uint8)
    return oracle.tgather([b8(s) for s in shards], dst, 1, 1, 1, H, K)


def run(sd, Bd, cb, out_dtype="bf16", scale=0.0, **kw):
    M, Nc = len(sd) * sd[0].shape[0], Bd.shape[0]
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float8_e4m3fn
    C = torch.full((M, Nc), float("nan"), dtype=dt, device=DEV)
    ag.ag_gemm(sd, Bd, cb, C=C, in_dtype="fp8_e4m3", out_dtype=out_dtype, out_scale=scale, **kw)
    torch.cuda.synchronize()
    rc, info = ag.check()
    assert rc == ag.AG_OK, info
    return C


SCHEDULES = ({}, {"producer": "in_kernel"}, {"producer": "copy_engine"}, {"mode": "unfused"},
             {"mode": "gemm_only"}, {"mode": "plain_gemm"}, {"local_rank": 2})


def check_exact(N, H, K, Nc, cb, seed, schedules=SCHEDULES):
    shards, B = workloads.make_ag_gemm_fp8_integers(N, H, K, Nc, seed=seed)
    _, C32 = oracle.ag_gemm(images(shards), oracle.e4m3fn_to_bf16(b8(B)))
    assert np.abs(C32).max() < 2 ** 24
    A_bytes = gathered(shards)
    sd = [s.to(DEV) for s in shards]
    Bd = B.to(DEV)
    a_full = torch.from_numpy(A_bytes).to(DEV)
    want = oracle.f32_to_bf16(C32)
    for kw in schedules:
        a_out = a_full if kw.get("mode") in ("gemm_only", "plain_gemm") else \
            torch.full_like(a_full, 0x7F)
        got = u16(run(sd, Bd, cb, a_out=a_out, **kw))
        assert np.array_equal(got, want), (kw, int((got != want).sum()))
        assert np.array_equal(b8(a_out), A_bytes), kw
    return sd, Bd, C32


def test_fp8_inputs_exact_integers_every_schedule():
    N, H, K, Nc, cb = 4, 64, 128, 128, 32
    print("fp8-in exact N=%d H=%d K=%d Nc=%d" % (N, H, K, Nc), flush=True)
    check_exact(N, H, K, Nc, cb, seed=101)


def test_fp8_inputs_exact_integers_ragged_k_rows_and_columns():
    # K = 528 bytes per row: four 128-byte K steps and a 16-byte tail; ragged M and Nc tiles
    N, H, K, Nc, cb = 3, 100, 528, 392, 33
    print("fp8-in exact ragged N=%d H=%d K=%d Nc=%d" % (N, H, K, Nc), flush=True)
    check_exact(N, H, K, Nc, cb, seed=102)


def test_fp8_inputs_exact_integers_more_tiles_than_compute_units():
    # 20 x 20 = 400 output tiles: every workgroup of the persistent grid takes more than one
    N, H, K, Nc, cb = 8, 640, 256, 5120, 128
    print("fp8-in exact 400 tiles", flush=True)
    check_exact(N, H, K, Nc, cb, seed=103, schedules=({}, {"producer": "in_kernel"}, {"mode": "unfused"},
                                                      {"local_rank": 5}))


def test_fp8_inputs_fp8_output_exact():
    N, H, K, Nc, cb = 3, 100, 256, 200, 40
    print("fp8-in fp8-out exact", flush=True)
    shards, B = workloads.make_ag_gemm_fp8_integers(N, H, K, Nc, seed=104)
    _, C32 = oracle.ag_gemm(images(shards), oracle.e4m3fn_to_bf16(b8(B)))
    sd = [s.to(DEV) for s in shards]
    Bd = B.to(DEV)
    for scale in (2.0 ** -4, 2.0 ** -7):
        want = oracle.f32_to_e4m3fn((C32.astype(np.float32) * np.float32(scale)).astype(np.float32))
        for kw in ({}, {"mode": "unfused"}):
            got = b8(run(sd, Bd, cb, out_dtype="fp8_e4m3", scale=scale, **kw))
            nan_g, nan_w = (got & 0x7F) == 0x7F, (want & 0x7F) == 0x7F
            assert np.array_equal(nan_g, nan_w) and np.array_equal(got[~nan_g], want[~nan_w]), (scale, kw)


def within_summation_error(got_bits, c32, absab, K, scale):
    """got (bf16 bits) lies between bf16(s (c - e)) and bf16(s (c + e)), e the summation bound."""
    c = c32.astype(np.float64) * scale
    e = 2.0 * K * 2.0 ** -24 * absab * scale + np.abs(c) * 2.0 ** -23
    lo = bf16_values(oracle.f32_to_bf16((c - e).astype(np.float32)))
    hi = bf16_values(oracle.f32_to_bf16((c + e).astype(np.float32)))
    v = bf16_values(got_bits)
    ok = (v >= lo) & (v <= hi)
    return bool(ok.all()), int((~ok).sum())


def test_fp8_inputs_random_data_within_the_summation_error():
    cfg = workloads.AgGemmConfig("fp8_random", N=4, H=160, K=512, Nc=264, cb=48, a_std=1.0, b_std=1.0, seed=105)
    print("fp8-in random %s" % cfg.name, flush=True)
    A, shards, B = workloads.make_ag_gemm_fp8(cfg)
    _, C32 = oracle.ag_gemm(images(shards), oracle.e4m3fn_to_bf16(b8(B)))
    va, vb = oracle.e4m3fn_value(b8(A)), oracle.e4m3fn_value(b8(B))
    absab = np.abs(va) @ np.abs(vb).T
    sd = [s.to(DEV) for s in shards]
    Bd = B.to(DEV)
    scale = 1.0 / np.sqrt(cfg.K)
    ref = None
    for kw in ({}, {"mode": "unfused"}, {"producer": "in_kernel"}):
        got = u16(run(sd, Bd, cfg.cb, scale=scale, **kw))
        ok, bad = within_summation_error(got, C32, absab, cfg.K, scale)
        assert ok, (kw, bad)
        if ref is None:
            ref = got
        assert np.array_equal(got, ref), kw


@pytest.mark.slow
def test_fp8_inputs_full_size_square_workload():
    cfg = workloads.AG_SQUARE_FP8
    print("fp8-in full size %s" % cfg.name, flush=True)
    A, shards, B = workloads.make_ag_gemm_fp8(cfg)
    sd = [s.to(DEV) for s in shards]
    Bd = B.to(DEV)
    scale = 1.0 / np.sqrt(cfg.K)
    a_out = torch.empty((cfg.M, cfg.K), dtype=torch.uint8, device=DEV)
    fused = run(sd, Bd, cfg.cb, scale=scale, a_out=a_out)
    assert torch.equal(a_out.cpu(), A)
    unfused = run(sd, Bd, cfg.cb, scale=scale, mode="unfused")
    assert torch.equal(fused.view(torch.int16), unfused.view(torch.int16))
    got = u16(fused)
    rng = np.random.default_rng(106)
    ms = rng.integers(0, cfg.M, 3000)
    ns = rng.integers(0, cfg.Nc, 3000)
    c32 = oracle.ag_gemm_at(images(shards), oracle.e4m3fn_to_bf16(b8(B)), ms, ns)
    va = oracle.e4m3fn_value(b8(A)[ms])
    vb = oracle.e4m3fn_value(b8(B)[ns])
    absab = np.einsum("ik,ik->i", np.abs(va), np.abs(vb))
    ok, bad = within_summation_error(got[ms, ns], c32, absab, cfg.K, scale)
    assert ok, bad


def test_fp8_inputs_largest_supported_k():
    # K = 2^21 codes per row (2 MiB): a full 256-row tile spans 512 MiB of A; values in {-1, 0, 1}
    # keep every partial sum an integer of magnitude at most 2^21, exact in any order
    N, H, K, Nc, cb = 2, 128, 1 << 21, 24, 50
    print("fp8-in largest K", flush=True)
    shards, B = workloads.make_ag_gemm_fp8_integers(N, H, K, Nc, seed=108, lim=1)
    _, C32 = oracle.ag_gemm(images(shards), oracle.e4m3fn_to_bf16(b8(B)))
    assert np.abs(C32).max() <= K
    want = oracle.f32_to_bf16(C32)
    A_bytes = gathered(shards)
    sd = [s.to(DEV) for s in shards]
    Bd = B.to(DEV)
    del shards
    a_out = torch.empty((N * H, K), dtype=torch.uint8, device=DEV)
    for kw in ({}, {"producer": "in_kernel"}, {"mode": "unfused"}, {"local_rank": 1}):
        a_out.fill_(0x7F)
        got = u16(run(sd, Bd, cb, a_out=a_out, **kw))
        assert np.array_equal(got, want), kw
        if kw.get("mode") != "unfused":
            assert np.array_equal(b8(a_out), A_bytes), kw


def test_fp8_inputs_one_chunk_rows_and_empty_k():
    # K = 16: every row is one 16-byte chunk, the rest of the 128-byte K step reads zeros
    N, H, K, Nc, cb = 2, 70, 16, 90, 20
    print("fp8-in K=16 and K=0", flush=True)
    check_exact(N, H, K, Nc, cb, seed=107, schedules=({}, {"mode": "unfused"}, {"producer": "in_kernel"}))
    # K = 0: the empty sum, C = 0
    sd = [torch.empty((H, 0), dtype=torch.uint8, device=DEV) for _ in range(N)]
    Bd = torch.empty((Nc, 0), dtype=torch.uint8, device=DEV)
    C = run(sd, Bd, cb)
    assert not torch.isnan(C.float()).any() and (C.float() == 0).all()
