"""Python binding of libaggemm (include/aggemm.h): chunked AllGather fused with a bf16 GEMM, and
TGATHER, on one MI355X.

Argument marshalling only: every step of the path runs in the library's gfx950 kernels.  Tensors
are torch CUDA (HIP) tensors; the library is given their device pointers and the current stream.
The library must have been built (``python allgather_gemm_amd/build.py`` or
``__graft_entry__.build()``); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libaggemm.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "aggemm.h")

AG_OK, AG_EINVAL, AG_ENOMEM, AG_EHIP, AG_ETIMEOUT, AG_EUNSUPPORTED = 0, -1, -2, -3, -4, -5
MODE_FUSED, MODE_UNFUSED, MODE_GEMM_ONLY, MODE_PLAIN_GEMM = 0, 1, 2, 3
_MODES = {"fused": MODE_FUSED, "unfused": MODE_UNFUSED, "gemm_only": MODE_GEMM_ONLY,
          "plain_gemm": MODE_PLAIN_GEMM}
PRODUCER_SIDE_STREAM, PRODUCER_IN_KERNEL, PRODUCER_COPY_ENGINE = 0, 1, 2
OUT_BF16, OUT_FP8_E4M3 = 0, 1
IN_BF16, IN_FP8_E4M3 = 0, 1
_OUT = {"bf16": (OUT_BF16, torch.bfloat16), "fp8_e4m3": (OUT_FP8_E4M3, torch.float8_e4m3fn)}
_IN = {"bf16": (IN_BF16, (torch.bfloat16,)), "fp8_e4m3": (IN_FP8_E4M3, (torch.float8_e4m3fn, torch.uint8))}
_PRODUCERS = {"in_kernel": PRODUCER_IN_KERNEL, "side_stream": PRODUCER_SIDE_STREAM,
              "copy_engine": PRODUCER_COPY_ENGINE}

_i32, _i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p


class AgOptions(ctypes.Structure):
    _fields_ = [("mode", _i32), ("local_rank", _i32), ("a_out", _vp), ("timeout_us", _i64),
                ("reverse_order", _i32), ("skip_producer", _i32), ("producer", _i32),
                ("gemm_events", _vp * 2), ("out_dtype", _i32), ("out_scale", ctypes.c_float),
                ("wait_stats", _vp), ("in_dtype", _i32)]


class AgError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        msg = "%s failed: %s (%d)" % (what, status_str(code), code)
        if code == AG_EHIP:
            msg += ": " + lib().ag_last_error().decode(errors="replace")
        super().__init__(msg)


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libaggemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libaggemm.so is not built; run allgather_gemm_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        gemm_args = [_vp, _i32, _i64, _i64, _vp, _i64, _vp, _i64, _vp]
        for name in ("ag_gemm", "ag_gemm_unfused"):
            getattr(L, name).argtypes = gemm_args
            getattr(L, name).restype = ctypes.c_int
        L.ag_gemm_ex.argtypes = gemm_args + [ctypes.POINTER(AgOptions)]
        L.ag_gemm_ex.restype = ctypes.c_int
        L.gemm_rs.argtypes = [_vp, _vp, _i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _i32, _vp]
        L.gemm_rs.restype = ctypes.c_int
        L.ag_gemm_noalloc.argtypes = [_vp, _i32, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i32, _vp]
        L.ag_gemm_noalloc.restype = ctypes.c_int
        L.tgather.argtypes = [_vp, _i32, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i32, _vp]
        L.tgather.restype = ctypes.c_int
        L.tgather_ex.argtypes = [_vp, _i32, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                 _i32, _i32, _vp]
        L.tgather_ex.restype = ctypes.c_int
        L.ag_check.argtypes = [_vp, ctypes.POINTER(_i64)]
        L.ag_check.restype = ctypes.c_int
        L.ag_status_str.argtypes = [ctypes.c_int]
        L.ag_status_str.restype = ctypes.c_char_p
        L.ag_last_error.argtypes = []
        L.ag_last_error.restype = ctypes.c_char_p
        L.ag_finalize.argtypes = []
        L.ag_finalize.restype = None
        _lib = L
    return _lib


def declared_functions() -> list[str]:
    """Names of the functions include/aggemm.h declares (used to check the exports)."""
    text = open(HEADER_PATH, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def status_str(code: int) -> str:
    return lib().ag_status_str(code).decode()


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _ptrs(tensors) -> ctypes.Array:
    return (_vp * len(tensors))(*[t.data_ptr() for t in tensors])


def _check_dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def ag_gemm(shards, B: torch.Tensor, comm_block_rows: int, C: torch.Tensor | None = None,
            mode: str = "fused", local_rank: int = 0, a_out: torch.Tensor | None = None,
            timeout_us: int = 0, reverse_order: bool = False, skip_producer: bool = False,
            producer: str = "side_stream", gemm_events=None, stream=None, out_dtype: str = "bf16",
            out_scale: float = 1.0, wait_stats: torch.Tensor | None = None,
            in_dtype: str = "bf16") -> torch.Tensor:
    """C (M, Nc) = concat(shards) @ B^T.  shards: N tensors (H, K); B: (Nc, K), both bf16, or with
    in_dtype="fp8_e4m3" both FP8 E4M3 "fn" (torch.float8_e4m3fn or their uint8 codes; K % 16 == 0),
    when C = out_scale * (A B^T) (out_scale folds the inputs' per-tensor scales).

    mode: "fused" | "unfused" | "gemm_only" | "plain_gemm"; producer (fused only): "side_stream" |
    "in_kernel" | "copy_engine".  out_dtype: "bf16" or "fp8_e4m3" (C = e4m3fn(sum * out_scale), a
    torch.float8_e4m3fn tensor).  gemm_events: optional (start, end) torch.cuda.Event pair that the
    library records around the GEMM kernel's launch.  wait_stats: optional int64 device tensor of 4
    counters the GEMM adds to (flag-wait ticks at 100 MHz summed over workgroups, waits, pieces
    copied while waiting, tiles that skipped their wait).  The call is asynchronous on `stream`; check()
    reports a wait that gave up."""
    shards = list(shards)
    N = len(shards)
    if N == 0:
        raise ValueError("need at least one shard")
    H, K = shards[0].shape
    M = N * H
    Nc = B.shape[0]
    in_code, in_types = _IN[in_dtype]
    for i, s in enumerate(shards):
        _check_dev(s, "shard %d" % i)
        if s.dtype not in in_types or tuple(s.shape) != (H, K):
            raise ValueError("shards must all be (H, K) %s" % in_dtype)
    _check_dev(B, "B")
    if B.dtype not in in_types or B.shape[1] != K:
        raise ValueError("B must be (Nc, K) %s" % in_dtype)
    out_code, out_torch = _OUT[out_dtype]
    if C is None:
        C = torch.empty((M, Nc), dtype=out_torch, device=B.device)
    _check_dev(C, "C")
    if C.dtype != out_torch or tuple(C.shape) != (M, Nc):
        raise ValueError("C must be (M, Nc) %s" % out_torch)
    ev = (_vp * 2)(*(int(e.event_id) for e in gemm_events)) if gemm_events else (_vp * 2)(None, None)
    opt = AgOptions(_MODES[mode], local_rank, a_out.data_ptr() if a_out is not None else None,
                    timeout_us, int(reverse_order), int(skip_producer), _PRODUCERS[producer], ev,
                    out_code, float(out_scale), None, in_code)
    if wait_stats is not None:
        _check_dev(wait_stats, "wait_stats")
        if wait_stats.dtype != torch.int64 or wait_stats.numel() < 4:
            raise ValueError("wait_stats must be an int64 device tensor of 4 counters")
        opt.wait_stats = wait_stats.data_ptr()
    if a_out is not None:
        _check_dev(a_out, "a_out")
        if a_out.dtype not in in_types or tuple(a_out.shape) != (M, K):
            raise ValueError("a_out must be (M, K) %s" % in_dtype)
    rc = lib().ag_gemm_ex(ctypes.cast(_ptrs(shards), _vp), N, M, K, B.data_ptr(), Nc,
                          C.data_ptr(), comm_block_rows, _stream_ptr(stream), ctypes.byref(opt))
    if rc != AG_OK:
        raise AgError(rc, "ag_gemm_ex")
    return C


def ag_gemm_noalloc(shards, B: torch.Tensor, comm_block_rows: int, C: torch.Tensor, a_out: torch.Tensor,
                    local_rank: int = 0, stream=None) -> torch.Tensor:
    """ag_gemm for callers that cannot allocate: C and a_out are the caller's; the library's control
    words are a fixed array per GPU (calls that overlap on one GPU race)."""
    shards = list(shards)
    N = len(shards)
    if N == 0:
        raise ValueError("need at least one shard")
    H, K = shards[0].shape
    M, Nc = N * H, B.shape[0]
    for i, s in enumerate(shards):
        _check_dev(s, "shard %d" % i)
        if s.dtype != torch.bfloat16 or tuple(s.shape) != (H, K):
            raise ValueError("shards must all be (H, K) bfloat16")
    for t, name, shape in ((B, "B", (Nc, K)), (C, "C", (M, Nc)), (a_out, "a_out", (M, K))):
        _check_dev(t, name)
        if t.dtype != torch.bfloat16 or tuple(t.shape) != shape:
            raise ValueError("%s must be %s bfloat16" % (name, shape))
    rc = lib().ag_gemm_noalloc(ctypes.cast(_ptrs(shards), _vp), N, M, K, B.data_ptr(), Nc, C.data_ptr(),
                               comm_block_rows, a_out.data_ptr(), local_rank, _stream_ptr(stream))
    if rc != AG_OK:
        raise AgError(rc, "ag_gemm_noalloc")
    return C


RS_FUSED, RS_UNFUSED = 0, 1


def gemm_rs(A: torch.Tensor, B: torch.Tensor, recv, local_rank: int, P: torch.Tensor | None = None,
            out: torch.Tensor | None = None, fused: bool = True, stream=None):
    """One rank's GEMM + ReduceScatter.  A (M, K), B (Nc, K) bf16: this rank's K slices; recv: N
    tensors (H, Nc) bf16, H = M / N, the other ranks' partials for this rank's rows (recv[local_rank]
    may be None).  Returns (P, out): P (M, Nc) = A B^T, out (H, Nc) = the reduction of this rank's
    row block over the N partials."""
    recv = list(recv)
    N = len(recv)
    M, K = A.shape
    Nc = B.shape[0]
    if N == 0 or M % N != 0:
        raise ValueError("need N >= 1 partials and M % N == 0")
    H = M // N
    for t, name in ((A, "A"), (B, "B")):
        _check_dev(t, name)
        if t.dtype != torch.bfloat16:
            raise ValueError("%s must be bfloat16" % name)
    if B.shape[1] != K:
        raise ValueError("B must be (Nc, K)")
    for j, t in enumerate(recv):
        if j == local_rank:
            continue
        _check_dev(t, "recv[%d]" % j)
        if t.dtype != torch.bfloat16 or tuple(t.shape) != (H, Nc):
            raise ValueError("recv[%d] must be (H, Nc) bfloat16" % j)
    if P is None:
        P = torch.empty((M, Nc), dtype=torch.bfloat16, device=A.device)
    if out is None:
        out = torch.empty((H, Nc), dtype=torch.bfloat16, device=A.device)
    for t, name, shape in ((P, "P", (M, Nc)), (out, "out", (H, Nc))):
        _check_dev(t, name)
        if t.dtype != torch.bfloat16 or tuple(t.shape) != shape:
            raise ValueError("%s must be %s bfloat16" % (name, shape))
    ptrs = (_vp * N)(*[None if j == local_rank or t is None else t.data_ptr() for j, t in enumerate(recv)])
    rc = lib().gemm_rs(A.data_ptr(), B.data_ptr(), N, local_rank, M, Nc, K, ctypes.cast(ptrs, _vp),
                       P.data_ptr(), out.data_ptr(), RS_FUSED if fused else RS_UNFUSED, _stream_ptr(stream))
    if rc != AG_OK:
        raise AgError(rc, "gemm_rs")
    return P, out


def ag_gemm_unfused(shards, B, comm_block_rows, C=None, a_out=None, stream=None):
    return ag_gemm(shards, B, comm_block_rows, C=C, mode="unfused", a_out=a_out, stream=stream)


def _as5d(t: torch.Tensor) -> tuple:
    if t.dim() == 5:
        return tuple(t.shape)
    if t.dim() == 2:
        return (1, 1, 1) + tuple(t.shape)
    if t.dim() == 1:
        return (1, 1, 1, 1, t.shape[0])
    raise ValueError("tgather takes (D0, D1, D2, H, W), (H, W) or (W,) tensors")


def tgather(shards, valid_rows: int, valid_cols: int, dst: torch.Tensor | None = None,
            dst_rows: int | None = None, root: int = 0, stream=None) -> torch.Tensor:
    """dst[d0, d1, d2, r*H + i, j] = shards[r][d0, d1, d2, i, j]; returns dst."""
    shards = list(shards)
    N = len(shards)
    if N == 0:
        raise ValueError("need at least one shard")
    shape = _as5d(shards[0])
    D0, D1, D2, H, W = shape
    dt = shards[0].dtype
    for i, s in enumerate(shards):
        _check_dev(s, "shard %d" % i)
        if _as5d(s) != shape or s.dtype != dt:
            raise ValueError("all shards must share shape and dtype")
    if dst_rows is None:
        dst_rows = N * H
    if dst is None:
        dst = torch.empty((D0, D1, D2, dst_rows, W), dtype=dt, device=shards[0].device)
    _check_dev(dst, "dst")
    if dst.numel() != D0 * D1 * D2 * dst_rows * W or dst.dtype != dt:
        raise ValueError("dst must hold (D0, D1, D2, dst_rows, W) elements of the shards' dtype")
    esz = shards[0].element_size()
    rc = lib().tgather_ex(ctypes.cast(_ptrs(shards), _vp), N, dst.data_ptr(), D0, D1, D2, H, W,
                          dst_rows, valid_rows, valid_cols, esz, root, _stream_ptr(stream))
    if rc != AG_OK:
        raise AgError(rc, "tgather_ex")
    return dst


def check(stream=None) -> tuple[int, list[int]]:
    """Waits for the stream and returns (status, [code, chunk, tile, epoch]) of the device status
    word (the first wait that gave up since the last check, and its call's flag epoch)."""
    info = (_i64 * 4)()
    rc = lib().ag_check(_stream_ptr(stream), info)
    return rc, [int(x) for x in info]


def finalize():
    lib().ag_finalize()
