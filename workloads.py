"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module holds shapes and random-number recipes only -- none of the method's arithmetic --
so that the GPU path and the CPU oracle can be fed identical inputs without sharing code.

Recipe (all on the CPU with ``torch.Generator().manual_seed(seed)``):
  * AG-GEMM: the full A (M, K) is drawn once as fp32 ``randn * a_std`` and rounded to bf16;
    shard r is rows [r*H, (r+1)*H) of it, so concatenating the shards gives A by construction.
    B (Nc, K) is then drawn from the same generator as ``randn * b_std`` rounded to bf16.
  * tgather: the N shards (D0, D1, D2, H, W) are drawn together as one fp32 tensor of shape
    (N, D0, D1, D2, H, W), ``U(-1, 1) = 2*rand - 1``, cast to the element type; ``bits`` mode
    draws raw 32-bit patterns instead (NaN payloads and subnormals included).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class AgGemmConfig:
    name: str
    N: int          # shards ("ranks")
    H: int          # rows per shard (M / N)
    K: int
    Nc: int         # rows of B = columns of C
    cb: int         # comm block rows
    a_std: float
    b_std: float
    seed: int = 0

    @property
    def M(self) -> int:
        return self.N * self.H

    @property
    def flops(self) -> int:
        return 2 * self.M * self.Nc * self.K


@dataclass(frozen=True)
class TgatherConfig:
    name: str
    N: int
    D: tuple        # (D0, D1, D2)
    H: int
    W: int
    dtype: torch.dtype
    valid_rows: int | None = None
    valid_cols: int | None = None
    seed: int = 0

    @property
    def payload_bytes(self) -> int:
        d0, d1, d2 = self.D
        return self.N * d0 * d1 * d2 * self.H * self.W * torch.empty((), dtype=self.dtype).element_size()


# The five workloads: a tiny AG-GEMM, a pure gather, the square AG-GEMM, an MLP-up projection
# shape, and a ragged pair (gather with odd tile extents + AG-GEMM with a ragged M tail).
AG_TINY = AgGemmConfig("ag_gemm_tiny_4x64x128", N=4, H=64, K=128, Nc=128, cb=32, a_std=1.0, b_std=1.0)
TG_FP16 = TgatherConfig("tgather_8x2x512x2048_f16", N=8, D=(2, 1, 1), H=512, W=2048, dtype=torch.float16)
AG_SQUARE = AgGemmConfig("ag_gemm_8192x8192x8192", N=8, H=1024, K=8192, Nc=8192, cb=128, a_std=1.0, b_std=0.02)
AG_MLP_UP = AgGemmConfig("ag_gemm_16384x14336x4096", N=8, H=2048, K=4096, Nc=14336, cb=256, a_std=1.0, b_std=0.02)
TG_RAGGED = TgatherConfig("tgather_8x1000x5000_f32_v997x4999", N=8, D=(1, 1, 1), H=1000, W=5000,
                          dtype=torch.float32, valid_rows=997, valid_cols=4999)
AG_RAGGED = AgGemmConfig("ag_gemm_4000x28672x8192", N=8, H=500, K=8192, Nc=28672, cb=100, a_std=1.0, b_std=0.02)

AG_CONFIGS = {c.name: c for c in (AG_TINY, AG_SQUARE, AG_MLP_UP, AG_RAGGED)}
TG_CONFIGS = {c.name: c for c in (TG_FP16, TG_RAGGED)}


def make_ag_gemm(cfg: AgGemmConfig, seed: int | None = None):
    """Returns (A (M,K) bf16, shards [N x (H,K) bf16 contiguous], B (Nc,K) bf16), CPU tensors."""
    g = torch.Generator().manual_seed(cfg.seed if seed is None else seed)
    A = (torch.randn(cfg.M, cfg.K, generator=g) * cfg.a_std).to(torch.bfloat16)
    B = (torch.randn(cfg.Nc, cfg.K, generator=g) * cfg.b_std).to(torch.bfloat16)
    shards = [A[r * cfg.H:(r + 1) * cfg.H].contiguous() for r in range(cfg.N)]
    return A, shards, B


def make_ag_gemm_shapes(N: int, H: int, K: int, Nc: int, seed: int = 0, a_std: float = 1.0,
                        b_std: float = 1.0):
    """Same recipe as make_ag_gemm for an ad-hoc shape (edge-case tests)."""
    cfg = AgGemmConfig("adhoc", N=N, H=H, K=K, Nc=Nc, cb=1, a_std=a_std, b_std=b_std, seed=seed)
    return make_ag_gemm(cfg)


def make_ag_gemm_integers(N: int, H: int, K: int, Nc: int, seed: int = 0, lim: int = 3):
    """Shards and B with integer entries in [-lim, lim] (exact in bf16): with small K every partial
    sum is an integer far below 2^24, so an fp32 sum is exact in any order.  Returns (shards, B)."""
    assert 0 <= lim < 128
    g = torch.Generator().manual_seed(seed)
    # int8 draws: the same values as int64 ones from the same generator, at an eighth of the memory
    shards = [torch.randint(-lim, lim + 1, (H, K), generator=g, dtype=torch.int8).to(torch.bfloat16)
              for _ in range(N)]
    B = torch.randint(-lim, lim + 1, (Nc, K), generator=g, dtype=torch.int8).to(torch.bfloat16)
    return shards, B


# FP8 inputs: the square workload with A and B in E4M3 "fn"; both ~ N(0, 1) before the conversion
# (E4M3's normal range starts at 2^-6, so a weight spread of 0.02 would sit in its subnormals), and
# the sums brought back to O(1) by out_scale = 1 / sqrt(K).
AG_SQUARE_FP8 = AgGemmConfig("ag_gemm_8192x8192x8192_fp8", N=8, H=1024, K=8192, Nc=8192, cb=128,
                             a_std=1.0, b_std=1.0)


def to_e4m3fn_codes(x: torch.Tensor) -> torch.Tensor:
    """uint8 E4M3 "fn" codes of fp32 values: torch's float8_e4m3fn conversion (round to nearest
    even), viewed as bytes."""
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def make_ag_gemm_fp8(cfg: AgGemmConfig, seed: int | None = None):
    """FP8 inputs: (A (M,K), shards [N x (H,K)], B (Nc,K)) as uint8 E4M3 codes, CPU tensors."""
    g = torch.Generator().manual_seed(cfg.seed if seed is None else seed)
    A = to_e4m3fn_codes(torch.randn(cfg.M, cfg.K, generator=g) * cfg.a_std)
    B = to_e4m3fn_codes(torch.randn(cfg.Nc, cfg.K, generator=g) * cfg.b_std)
    shards = [A[r * cfg.H:(r + 1) * cfg.H].contiguous() for r in range(cfg.N)]
    return A, shards, B


def make_ag_gemm_fp8_integers(N: int, H: int, K: int, Nc: int, seed: int = 0, lim: int = 4):
    """FP8 inputs with integer values in [-lim, lim] (exact in E4M3 for lim <= 16): every fp32
    partial sum is an integer below 2^24 for K * lim^2 < 2^24, exact in any order.  Returns
    (shards, B) as uint8 codes."""
    assert 0 <= lim <= 16
    g = torch.Generator().manual_seed(seed)
    shards = [to_e4m3fn_codes(torch.randint(-lim, lim + 1, (H, K), generator=g, dtype=torch.int8).float())
              for _ in range(N)]
    B = to_e4m3fn_codes(torch.randint(-lim, lim + 1, (Nc, K), generator=g, dtype=torch.int8).float())
    return shards, B


@dataclass(frozen=True)
class GemmRsConfig:
    """One rank's GEMM + ReduceScatter: A (M, K) and B (Nc, K) are the rank's K slices; the other
    N - 1 ranks' partials for its rows are (M / N, Nc) each."""
    name: str
    N: int
    M: int
    K: int
    Nc: int
    local: int = 0
    a_std: float = 1.0
    b_std: float = 0.02
    seed: int = 0

    @property
    def H(self) -> int:
        return self.M // self.N

    @property
    def flops(self) -> int:
        return 2 * self.M * self.Nc * self.K


RS_TINY = GemmRsConfig("gemm_rs_tiny_4x512x64x256", N=4, M=512, K=64, Nc=256, local=1, b_std=1.0)
# the square AG-GEMM workload's reduce-scatter mirror: K = 8192 split over 8 ranks
RS_SQUARE = GemmRsConfig("gemm_rs_8192x8192x1024_n8", N=8, M=8192, K=1024, Nc=8192, local=0)


def make_gemm_rs(cfg: GemmRsConfig, seed: int | None = None):
    """(A (M,K), B (Nc,K), recv: N tensors (H, Nc), recv[local] None) bf16 CPU tensors.  The peers'
    partials have the scale of a partial product, N(0, K a_std^2 b_std^2)."""
    g = torch.Generator().manual_seed(cfg.seed if seed is None else seed)
    A = (torch.randn(cfg.M, cfg.K, generator=g) * cfg.a_std).to(torch.bfloat16)
    B = (torch.randn(cfg.Nc, cfg.K, generator=g) * cfg.b_std).to(torch.bfloat16)
    sd = (cfg.K ** 0.5) * cfg.a_std * cfg.b_std
    recv = [None if j == cfg.local else (torch.randn(cfg.H, cfg.Nc, generator=g) * sd).to(torch.bfloat16)
            for j in range(cfg.N)]
    return A, B, recv


def make_tgather(N: int, D: tuple, H: int, W: int, dtype: torch.dtype, seed: int = 0,
                 bits: bool = False):
    """Returns a list of N contiguous CPU tensors of shape (D0, D1, D2, H, W)."""
    g = torch.Generator().manual_seed(seed)
    shape = (N,) + tuple(D) + (H, W)
    if bits:
        esz = torch.empty((), dtype=dtype).element_size()
        nbytes = int(np.prod(shape)) * esz
        raw = torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8)
        x = raw.view(dtype).reshape(shape)
    elif dtype.is_floating_point:
        x = (torch.rand(shape, generator=g) * 2.0 - 1.0).to(dtype)
    else:
        info = torch.iinfo(dtype)
        x = torch.randint(info.min, info.max, shape, generator=g, dtype=torch.int64).to(dtype)
    return [x[r].contiguous() for r in range(N)]


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 CPU tensor -> numpy uint16 bit patterns (the oracle's input format)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def raw_bytes(t: torch.Tensor) -> np.ndarray:
    """Any contiguous CPU tensor -> numpy uint8 view of its bytes."""
    return t.contiguous().view(torch.uint8).numpy() if t.dtype != torch.uint8 else t.contiguous().numpy()
