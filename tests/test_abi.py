"""C-ABI checks that need no GPU: the library loads, exports every function include/aggemm.h
declares, and rejects invalid arguments before touching the device."""
import ctypes

import pytest

import allgather_gemm_amd as ag

_vp = ctypes.c_void_p


def test_library_exports_every_declared_function():
    names = ag.declared_functions()
    for expected in ("ag_gemm", "ag_gemm_unfused", "ag_gemm_ex", "tgather", "tgather_ex",
                     "ag_check", "ag_status_str", "ag_last_error", "ag_finalize"):
        assert expected in names
    L = ag.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in (ag.AG_OK, ag.AG_EINVAL, ag.AG_ENOMEM, ag.AG_EHIP, ag.AG_ETIMEOUT, ag.AG_EUNSUPPORTED):
        assert ag.status_str(code) and ag.status_str(code) != "unknown status"
    assert ag.status_str(12345) == "unknown status"


def _fake_ptrs(n, base=0x10000):
    # never dereferenced: every call below is rejected (or is a no-op) before any device access
    return (_vp * n)(*[base + 256 * i for i in range(n)])


@pytest.mark.parametrize("N,M,K,Nc,cb,why", [
    (0, 0, 8, 8, 1, "no shards"),
    (65, 65, 8, 8, 1, "more shards than the library carries"),
    (3, 10, 8, 8, 1, "M not a multiple of N"),
    (2, 8, 12, 8, 1, "K not a multiple of 8"),
    (2, 8, 8, 8, 0, "comm block of zero rows"),
    (2, -2, 8, 8, 1, "negative M"),
])
def test_ag_gemm_rejects_invalid_shapes(N, M, K, Nc, cb, why):
    L = ag.lib()
    rc = L.ag_gemm(ctypes.cast(_fake_ptrs(max(N, 1)), _vp), N, M, K, _vp(0x20000), Nc,
                   _vp(0x30000), cb, None)
    assert rc == ag.AG_EINVAL, why


def test_ag_gemm_rejects_unaligned_or_null():
    L = ag.lib()
    ptrs = _fake_ptrs(2)
    assert L.ag_gemm(ctypes.cast(ptrs, _vp), 2, 8, 8, None, 8, _vp(0x30000), 4, None) == ag.AG_EINVAL
    assert L.ag_gemm(ctypes.cast(ptrs, _vp), 2, 8, 8, _vp(0x20008), 8, _vp(0x30000), 4, None) == ag.AG_EINVAL
    bad = (_vp * 2)(0x10000, 0x10004)
    assert L.ag_gemm(ctypes.cast(bad, _vp), 2, 8, 8, _vp(0x20000), 8, _vp(0x30000), 4, None) == ag.AG_EINVAL
    assert L.ag_gemm(None, 2, 8, 8, _vp(0x20000), 8, _vp(0x30000), 4, None) == ag.AG_EINVAL
    assert L.ag_gemm(ctypes.cast(ptrs, _vp), 2, 8, 1 << 22, _vp(0x20000), 8, _vp(0x30000), 4,
                     None) == ag.AG_EUNSUPPORTED


def test_ag_gemm_ex_rejects_bad_options():
    L = ag.lib()
    ptrs = ctypes.cast(_fake_ptrs(2), _vp)
    for opt in (ag.AgOptions(7, 0, None, 0, 0, 0, 0),       # unknown mode
                ag.AgOptions(0, 2, None, 0, 0, 0, 0),       # local rank out of range
                ag.AgOptions(2, 0, None, 0, 0, 0, 0),       # GEMM-only needs the gathered A
                ag.AgOptions(0, 0, 0x40004, 0, 0, 0, 0),    # unaligned a_out
                ag.AgOptions(0, 0, None, 0, 0, 3, 0),       # skip_producer is 0 or 1
                ag.AgOptions(0, 0, None, 0, 0, 0, 3),       # unknown producer
                ag.AgOptions(0, 0, None, 0, 0, 0, -1),
                ag.AgOptions(0, 0, None, 0, 0, 0, 0, (_vp * 2)(None, None), 2, 1.0),   # unknown C type
                ag.AgOptions(0, 0, None, 0, 0, 0, 0, (_vp * 2)(None, None), 1, float("inf")),
                ag.AgOptions(0, 0, None, 0, 0, 0, 0, (_vp * 2)(None, None), 1, float("nan")),
                ag.AgOptions(0, 0, None, 0, 0, 0, 0, (_vp * 2)(None, None), 0, 1.0, None, 2),   # unknown input type
                ag.AgOptions(0, 0, None, 0, 0, 0, 0, (_vp * 2)(None, None), 0, 1.0, None, -1)):
        assert L.ag_gemm_ex(ptrs, 2, 8, 8, _vp(0x20000), 8, _vp(0x30000), 4, None,
                            ctypes.byref(opt)) == ag.AG_EINVAL
    # FP8 inputs: rows must be whole 16-byte chunks (K % 16 == 0), which bf16 rows of K = 8 are
    fp8 = ag.AgOptions(0, 0, None, 0, 0, 0, 0, (_vp * 2)(None, None), 0, 1.0, None, ag.IN_FP8_E4M3)
    assert L.ag_gemm_ex(ptrs, 2, 8, 8, _vp(0x20000), 8, _vp(0x30000), 4, None,
                        ctypes.byref(fp8)) == ag.AG_EINVAL
    assert L.ag_gemm_ex(ptrs, 2, 8, 24, _vp(0x20000), 8, _vp(0x30000), 4, None,
                        ctypes.byref(fp8)) == ag.AG_EINVAL


def test_gemm_rs_rejects_bad_arguments():
    L = ag.lib()
    recv = ctypes.cast(_fake_ptrs(4), _vp)
    ok = dict(A=_vp(0x20000), B=_vp(0x30000), N=4, local=1, M=64, Nc=64, K=32, recv=recv,
              P=_vp(0x40000), out=_vp(0x50000), mode=0)

    def call(**kw):
        a = dict(ok, **kw)
        return L.gemm_rs(a["A"], a["B"], a["N"], a["local"], a["M"], a["Nc"], a["K"], a["recv"], a["P"],
                         a["out"], a["mode"], None)
    for kw in (dict(N=0), dict(local=4), dict(local=-1), dict(M=66), dict(K=30), dict(Nc=60), dict(mode=2),
               dict(P=_vp(0x40004)), dict(out=None), dict(A=None), dict(recv=None)):
        assert call(**kw) == ag.AG_EINVAL, kw
    assert call(M=0) == ag.AG_OK and call(Nc=0) == ag.AG_OK


def test_empty_shapes_enqueue_nothing():
    L = ag.lib()
    ptrs = ctypes.cast(_fake_ptrs(2), _vp)
    assert L.ag_gemm(ptrs, 2, 0, 8, _vp(0x20000), 8, _vp(0x30000), 4, None) == ag.AG_OK
    assert L.ag_gemm(ptrs, 2, 8, 8, _vp(0x20000), 0, _vp(0x30000), 4, None) == ag.AG_OK
    # TGATHER deep dive §7.4: an empty shape returns without moving anything
    for dims in ((0, 1, 1, 4, 4), (1, 1, 1, 0, 4), (1, 1, 1, 4, 0), (1, 0, 1, 4, 4)):
        assert L.tgather(ptrs, 2, _vp(0x30000), *dims, 1, 1, 4, None) == ag.AG_OK


@pytest.mark.parametrize("args,why", [
    ((2, 1, 1, 1, 4, 4, 0, 1, 4), "valid_rows < 1"),
    ((2, 1, 1, 1, 4, 4, 1, 0, 4), "valid_cols < 1"),
    ((2, 1, 1, 1, 4, 4, 1, 1, 3), "element size not 1/2/4/8"),
    ((0, 1, 1, 1, 4, 4, 1, 1, 4), "no ranks"),
])
def test_tgather_rejects_invalid(args, why):
    L = ag.lib()
    N, D0, D1, D2, H, W, vr, vc, esz = args
    rc = L.tgather(ctypes.cast(_fake_ptrs(max(N, 1)), _vp), N, _vp(0x30000), D0, D1, D2, H, W,
                   vr, vc, esz, None)
    assert rc == ag.AG_EINVAL, why


def test_tgather_ex_rejects_short_dst():
    """TGATHER deep dive §7.2: the destination must hold N*H rows."""
    L = ag.lib()
    rc = L.tgather_ex(ctypes.cast(_fake_ptrs(4), _vp), 4, _vp(0x30000), 1, 1, 1, 8, 8, 31, 8, 8, 4,
                      0, None)
    assert rc == ag.AG_EINVAL


@pytest.mark.parametrize("root", [-1, 4, 100])
def test_tgather_ex_rejects_root_outside_the_ranks(root):
    """TGATHER deep dive (RunGatherWithRoot): the root is one of the N ranks."""
    L = ag.lib()
    rc = L.tgather_ex(ctypes.cast(_fake_ptrs(4), _vp), 4, _vp(0x30000), 1, 1, 1, 8, 8, 32, 8, 8, 4,
                      root, None)
    assert rc == ag.AG_EINVAL
