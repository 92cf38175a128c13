"""CPU oracle for the chunked AllGather + bf16 GEMM path and for TGATHER (ctypes binding).

TEST INFRASTRUCTURE ONLY.  The test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package; the GPU library (``allgather_gemm_amd``) never does and
shares no code with it.  The arithmetic lives in ``oracle.c``; this module only builds the
shared object with gcc and marshals numpy arrays.

Pages followed (see oracle.h): the fused AllGather+MatMul article ("Triton第四课：基于对称内存融合
AllGather 与 MatMul，提速1.56倍") and the TGATHER deep dive ("CANN PTO-ISA TGATHER 指令深度解析").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS when set, else the runtime's default)."""
    return int(lib().oracle_num_threads())


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so next to it and return its path."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
               "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_f32_to_bf16_rne.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16_rne.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16_array.argtypes = [_vp, _i64, _vp]
        L.oracle_f32_to_bf16_array.restype = None
        L.oracle_reduce_block.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp]
        L.oracle_reduce_block.restype = None
        L.oracle_f32_to_e4m3fn.argtypes = [ctypes.c_float]
        L.oracle_f32_to_e4m3fn.restype = ctypes.c_uint8
        L.oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3fn_value.restype = ctypes.c_double
        L.oracle_e4m3fn_to_bf16.argtypes = [_vp, _i64, _vp]
        L.oracle_e4m3fn_to_bf16.restype = ctypes.c_int
        L.oracle_tgather.argtypes = [_vp, ctypes.c_int, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                     ctypes.c_int]
        L.oracle_tgather.restype = ctypes.c_int
        L.oracle_gemm_f32.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp]
        L.oracle_gemm_f32.restype = None
        L.oracle_ag_gemm_at.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _i64, _vp, _vp, _i64,
                                        _vp]
        L.oracle_ag_gemm_at.restype = ctypes.c_int
        L.oracle_ag_gemm.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _i64, _vp, _vp]
        L.oracle_ag_gemm.restype = ctypes.c_int
        L.oracle_gemm_f32_fast.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp]
        L.oracle_gemm_f32_fast.restype = None
        L.oracle_ag_gemm_fast.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _i64, _vp]
        L.oracle_ag_gemm_fast.restype = ctypes.c_int
        L.oracle_chunk_of_row.argtypes = [_i64, _i64, _i64]
        L.oracle_chunk_of_row.restype = _i64
        L.oracle_chunks_overlapping.argtypes = [_i64, _i64, _i64, _i64, _vp, _i64]
        L.oracle_chunks_overlapping.restype = _i64
        L.oracle_grouped_tile.argtypes = [_i64, _i64, _i64, _i64, _vp, _vp]
        L.oracle_grouped_tile.restype = None
        L.oracle_ag_gemm_pivoted.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _i64, _i64, _i64,
                                             _i64, _i64, ctypes.c_int, _vp, _vp, _vp]
        L.oracle_ag_gemm_pivoted.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def _ptr_array(arrs) -> ctypes.Array:
    return (ctypes.c_void_p * len(arrs))(*[_ptr(a) for a in arrs])


def _as_u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, "bf16 data travels as uint16 bit patterns"
    return a


# ---------------------------------------------------------------------------------------------
def bf16_to_f32(bits: int) -> float:
    return float(lib().oracle_bf16_to_f32(bits))


def f32_to_bf16_rne(x: float) -> int:
    return int(lib().oracle_f32_to_bf16_rne(x))


def f32_to_bf16(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32 values, round to nearest even."""
    xs = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(xs.shape, dtype=np.uint16)
    lib().oracle_f32_to_bf16_array(_ptr(xs), xs.size, _ptr(out))
    return out


def reduce_block(parts) -> np.ndarray:
    """One rank's ReduceScatter block: bf16 of the fp32 sum, ascending rank, of parts (H, Nc) bf16."""
    parts = [_as_u16(p) for p in parts]
    H, Nc = parts[0].shape
    out = np.empty((H, Nc), dtype=np.uint16)
    lib().oracle_reduce_block(ctypes.cast(_ptr_array(parts), _vp), len(parts), H, Nc, _ptr(out))
    return out


def gemm_rs(A, B, recv, local: int):
    """One rank's GEMM + ReduceScatter (row-parallel partial products, reduced over M blocks).

    A (M, K) and B (Nc, K) bf16 are this rank's K slices; recv[j] (H, Nc) bf16, H = M / N, is rank j's
    partial for this rank's rows (recv[local] unused).  Returns (P, out): P (M, Nc) bf16 =
    bf16_rne(A B^T) with fp32 ascending-k sums, and out (H, Nc) bf16 = reduce_block of the N partials
    for rows [local H, (local + 1) H), this rank's own rows of P in slot `local`."""
    P = f32_to_bf16(gemm_f32(A, B))
    N = len(recv)
    H = P.shape[0] // N
    parts = [P[local * H:(local + 1) * H] if j == local else _as_u16(recv[j]) for j in range(N)]
    return P, reduce_block(parts)


def f32_to_e4m3fn(x) -> np.ndarray:
    """E4M3 "fn" codes (uint8) of fp32 values, element by element (see oracle.h)."""
    xs = np.asarray(x, dtype=np.float32)
    f = lib().oracle_f32_to_e4m3fn
    return np.array([f(float(v)) for v in xs.ravel()], dtype=np.uint8).reshape(xs.shape)


def e4m3fn_value(codes) -> np.ndarray:
    """Values (float64) of E4M3 "fn" codes."""
    cs = np.asarray(codes, dtype=np.uint8)
    f = lib().oracle_e4m3fn_value
    return np.array([f(int(c)) for c in cs.ravel()], dtype=np.float64).reshape(cs.shape)


def e4m3fn_to_bf16(codes) -> np.ndarray:
    """bf16 bit patterns (uint16) of E4M3 "fn" codes' values, exact (see oracle.h).  The GEMM of FP8
    inputs is gemm_f32 / ag_gemm_at on these patterns."""
    cs = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(cs.shape, dtype=np.uint16)
    if lib().oracle_e4m3fn_to_bf16(_ptr(cs), cs.size, _ptr(out)) != 0:
        raise ValueError("an E4M3 value was not exactly a bf16 value")
    return out


def tgather(shards, dst: np.ndarray, D0: int, D1: int, D2: int, H: int, W: int,
            dst_rows: int | None = None) -> np.ndarray:
    """TGATHER closed form (TGATHER deep dive, section 二 数学语义) into ``dst`` in place."""
    shards = [np.ascontiguousarray(s) for s in shards]
    esz = dst.itemsize
    for s in shards:
        assert s.itemsize == esz and s.size == D0 * D1 * D2 * H * W
    if dst_rows is None:
        dst_rows = len(shards) * H
    assert dst.flags.c_contiguous and dst.size == D0 * D1 * D2 * dst_rows * W
    ptrs = _ptr_array(shards)
    rc = lib().oracle_tgather(ctypes.cast(ptrs, _vp), len(shards), _ptr(dst), D0, D1, D2, H, W,
                              dst_rows, esz)
    if rc != 0:
        raise ValueError("oracle_tgather rejected its arguments (rc=%d)" % rc)
    return dst


def gemm_f32(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """C = A @ B^T, fp32 accumulation in ascending k (A (M,K), B (Nc,K) as bf16 bits)."""
    A, B = _as_u16(A), _as_u16(B)
    M, K = A.shape
    Nc, K2 = B.shape
    assert K == K2
    C = np.empty((M, Nc), dtype=np.float32)
    lib().oracle_gemm_f32(_ptr(A), _ptr(B), M, Nc, K, _ptr(C))
    return C


def ag_gemm(shards, B: np.ndarray):
    """Gather the shards, then GEMM.  Returns (A (M,K) bf16 bits, C (M,Nc) fp32)."""
    shards = [_as_u16(s) for s in shards]
    B = _as_u16(B)
    H, K = shards[0].shape
    M = H * len(shards)
    Nc = B.shape[0]
    A = np.empty((M, K), dtype=np.uint16)
    C = np.empty((M, Nc), dtype=np.float32)
    ptrs = _ptr_array(shards)
    rc = lib().oracle_ag_gemm(ctypes.cast(ptrs, _vp), len(shards), M, K, _ptr(B), Nc, _ptr(A),
                              _ptr(C))
    if rc != 0:
        raise ValueError("oracle_ag_gemm rc=%d" % rc)
    return A, C


def gemm_f32_fast(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """gemm_f32's C bit for bit, in a blocked loop order (for the full-size workloads)."""
    A, B = _as_u16(A), _as_u16(B)
    M, K = A.shape
    Nc, K2 = B.shape
    assert K == K2
    C = np.empty((M, Nc), dtype=np.float32)
    rows = (ctypes.c_void_p * max(M, 1))(*[A.ctypes.data + m * K * 2 for m in range(M)])
    lib().oracle_gemm_f32_fast(ctypes.cast(rows, _vp), _ptr(B), M, Nc, K, _ptr(C))
    return C


def ag_gemm_fast(shards, B: np.ndarray) -> np.ndarray:
    """C (M,Nc) fp32 of gather(shards) @ B^T, bit for bit ag_gemm's C, in the blocked loop order."""
    shards = [_as_u16(s) for s in shards]
    B = _as_u16(B)
    H, K = shards[0].shape
    M = H * len(shards)
    Nc = B.shape[0]
    C = np.empty((M, Nc), dtype=np.float32)
    ptrs = _ptr_array(shards)
    rc = lib().oracle_ag_gemm_fast(ctypes.cast(ptrs, _vp), len(shards), M, K, _ptr(B), Nc, _ptr(C))
    if rc != 0:
        raise ValueError("oracle_ag_gemm_fast rc=%d" % rc)
    return C


def ag_gemm_at(shards, B: np.ndarray, ms, ns) -> np.ndarray:
    """Elements C[ms[i], ns[i]] of gather(shards) @ B^T, fp32 ascending-k accumulation."""
    shards = [_as_u16(s) for s in shards]
    B = _as_u16(B)
    H, K = shards[0].shape
    M = H * len(shards)
    Nc = B.shape[0]
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ms.shape[0], dtype=np.float32)
    ptrs = _ptr_array(shards)
    rc = lib().oracle_ag_gemm_at(ctypes.cast(ptrs, _vp), len(shards), M, K, _ptr(B), Nc, _ptr(ms),
                                 _ptr(ns), ms.shape[0], _ptr(out))
    if rc != 0:
        raise ValueError("oracle_ag_gemm_at rc=%d" % rc)
    return out


def chunk_of_row(row: int, H: int, cb: int) -> int:
    return int(lib().oracle_chunk_of_row(row, H, cb))


def chunks_overlapping(m0: int, m1: int, H: int, cb: int) -> list[int]:
    cap = max(1, m1 - m0 + 1)
    out = np.zeros(cap, dtype=np.int64)
    n = int(lib().oracle_chunks_overlapping(m0, m1, H, cb, _ptr(out), cap))
    return [int(x) for x in out[:n]]


def grouped_tile(t: int, num_pid_m: int, num_pid_n: int, group_m: int) -> tuple[int, int]:
    pm = ctypes.c_int64()
    pn = ctypes.c_int64()
    lib().oracle_grouped_tile(t, num_pid_m, num_pid_n, group_m, ctypes.byref(pm),
                              ctypes.byref(pn))
    return int(pm.value), int(pn.value)


def ag_gemm_pivoted(shards, B: np.ndarray, cb: int, BM: int, BN: int, group_m: int,
                    local_rank: int):
    """Fused-schedule simulation.  Returns (rc, A_prime, C, stats dict)."""
    shards = [_as_u16(s) for s in shards]
    B = _as_u16(B)
    H, K = shards[0].shape
    M = H * len(shards)
    Nc = B.shape[0]
    A = np.empty((M, K), dtype=np.uint16)
    C = np.empty((M, Nc), dtype=np.float32)
    stats = np.zeros(6, dtype=np.int64)
    ptrs = _ptr_array(shards)
    rc = lib().oracle_ag_gemm_pivoted(ctypes.cast(ptrs, _vp), len(shards), M, K, _ptr(B), Nc, cb,
                                      BM, BN, group_m, local_rank, _ptr(A), _ptr(C), _ptr(stats))
    keys = ("waited_tiles", "flag_checks", "local_tiles", "first_pid_m",
            "tiles_before_first_remote", "published_before_drain")
    return rc, A, C, {k: int(v) for k, v in zip(keys, stats)}
