"""Host-side checks of the C ABI (no GPU needed).

The library loads, exports every entry point include/prune24.h declares, and
its validation rejects bad arguments with the documented status before
anything is enqueued (the pointers used here are never dereferenced).
"""
import ctypes

import pytest

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")


@pytest.fixture(scope="module")
def L():
    try:
        return p24.lib()
    except RuntimeError as e:
        pytest.fail(f"library not built: {e}")


def test_exports_every_declared_symbol(L):
    syms = p24.header_symbols()
    assert len(syms) == len(set(syms)) == 38
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(p24._SIGNATURES), "binding signatures drift from the header"


def test_version_and_strerror(L):
    assert L.prune24_abi_version() == 1
    for code in range(-9, 1):
        assert p24.strerror(code)
    assert p24.strerror(-99) == "unknown status"


def test_size_helpers(L):
    # canonical: K/2 bf16 values and ceil(K/32) words per row
    assert L.prune24_values_bytes(3, 36, p24.P24_LAYOUT_CANONICAL) == 3 * 18 * 2
    assert L.prune24_meta_bytes(3, 36, p24.P24_LAYOUT_CANONICAL) == 3 * 2 * 4
    # device: rows rounded up to 32, K % 64 required
    assert L.prune24_values_bytes(33, 128, p24.P24_LAYOUT_DEVICE) == 128 * 64 * 2      # rows padded to 128
    assert L.prune24_meta_bytes(33, 128, p24.P24_LAYOUT_DEVICE) == 4 * 2 * 64 * 4
    assert L.prune24_values_bytes(128, 64, p24.P24_LAYOUT_DEVICE) == 128 * 32 * 2
    assert L.prune24_meta_bytes(129, 64, p24.P24_LAYOUT_DEVICE) == 8 * 1 * 64 * 4
    assert L.prune24_values_bytes(32, 96, p24.P24_LAYOUT_DEVICE) == 0
    assert L.prune24_values_bytes(4, 6, p24.P24_LAYOUT_CANONICAL) == 0
    assert L.tvw_workspace_bytes(4096, 4096, 128, 2048) == 32 * 4096 * 8
    assert L.tvw_noalloc_scratch_bytes() == 8 << 20
    assert L.gemm_bf16_packed_bytes(40, 128) == 64 * 128 * 2
    assert L.gemm_bf16_packed_bytes(40, 96) == 0


FAKE = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced
MISALIGNED = ctypes.c_void_p((1 << 20) + 2)
NUL = ctypes.c_void_p(0)


def test_compress_validation(L):
    f = L.prune24_compress
    assert f(FAKE, 7, 4, 8, 8, FAKE, FAKE, 0, NUL) == p24.P24_ERR_DTYPE
    assert f(FAKE, 0, 4, 8, 8, FAKE, FAKE, 5, NUL) == p24.P24_ERR_LAYOUT
    assert f(FAKE, 0, 4, 6, 8, FAKE, FAKE, 0, NUL) == p24.P24_ERR_SHAPE          # K % 4
    assert f(FAKE, 0, 4, 8, 4, FAKE, FAKE, 0, NUL) == p24.P24_ERR_SHAPE          # ldw < K
    assert f(FAKE, 0, -1, 8, 8, FAKE, FAKE, 0, NUL) == p24.P24_ERR_SHAPE
    assert f(FAKE, 0, 4, 96, 96, FAKE, FAKE, 1, NUL) == p24.P24_ERR_UNSUPPORTED  # device needs K % 64
    assert f(NUL, 0, 4, 8, 8, FAKE, FAKE, 0, NUL) == p24.P24_ERR_NULL
    assert f(MISALIGNED, 0, 4, 8, 8, FAKE, FAKE, 0, NUL) == p24.P24_ERR_ALIGN
    assert f(FAKE, 0, 4, 8, 10, FAKE, FAKE, 0, NUL) == p24.P24_ERR_ALIGN          # ldw % 4
    assert f(NUL, 0, 0, 8, 8, NUL, NUL, 0, NUL) == p24.P24_OK                     # M == 0: no-op


def test_mask_validation(L):
    f = L.prune24_refresh            # same rules as prune24_compress
    assert f(FAKE, 7, 4, 8, 8, FAKE, FAKE, 0, NUL) == p24.P24_ERR_DTYPE
    assert f(FAKE, 0, 4, 6, 8, FAKE, FAKE, 0, NUL) == p24.P24_ERR_SHAPE
    assert f(FAKE, 0, 4, 96, 96, FAKE, FAKE, 1, NUL) == p24.P24_ERR_UNSUPPORTED
    assert f(MISALIGNED, 0, 4, 8, 8, FAKE, FAKE, 0, NUL) == p24.P24_ERR_ALIGN
    assert f(NUL, 0, 0, 8, 8, NUL, NUL, 0, NUL) == p24.P24_OK
    g = L.prune24_mask_apply
    assert g(FAKE, 5, 4, 8, 8, FAKE, 0, NUL) == p24.P24_ERR_DTYPE
    assert g(FAKE, 0, 4, 8, 8, FAKE, 3, NUL) == p24.P24_ERR_LAYOUT
    assert g(FAKE, 0, 4, 6, 8, FAKE, 0, NUL) == p24.P24_ERR_SHAPE           # K % 4
    assert g(FAKE, 0, 4, 8, 4, FAKE, 0, NUL) == p24.P24_ERR_SHAPE           # ldw < K
    assert g(FAKE, 0, 4, 96, 96, FAKE, 1, NUL) == p24.P24_ERR_UNSUPPORTED   # device layout: K % 64
    assert g(FAKE, 0, 4, 8, 8, NUL, 0, NUL) == p24.P24_ERR_NULL
    assert g(MISALIGNED, 0, 4, 8, 8, FAKE, 0, NUL) == p24.P24_ERR_ALIGN
    assert g(FAKE, 0, 4, 8, 10, FAKE, 0, NUL) == p24.P24_ERR_ALIGN          # ldw % 4
    assert g(NUL, 0, 0, 8, 8, NUL, 0, NUL) == p24.P24_OK


def test_spmm_validation(L):
    f = L.spmm24
    args = lambda **k: [k.get("v", FAKE), k.get("m", FAKE), k.get("layout", 1), k.get("M", 64),
                        k.get("K", 128), k.get("X", FAKE), k.get("ldx", 64), k.get("N", 64), k.get("Y", FAKE),
                        k.get("yd", 0), k.get("ldy", 64), k.get("algo", 0), NUL]
    assert f(*args(layout=0)) == p24.P24_ERR_LAYOUT
    assert f(*args(K=96)) == p24.P24_ERR_UNSUPPORTED
    assert f(*args(yd=3)) == p24.P24_ERR_DTYPE
    assert f(*args(algo=9)) == p24.P24_ERR_UNSUPPORTED
    assert f(*args(algo=3)) == p24.P24_ERR_UNSUPPORTED
    assert f(*args(algo=-1)) == p24.P24_ERR_UNSUPPORTED
    for algo in (0, 1, 2):     # every accepted algorithm runs the same validation
        assert f(*args(algo=algo, layout=0)) == p24.P24_ERR_LAYOUT
        assert f(*args(algo=algo, K=96)) == p24.P24_ERR_UNSUPPORTED
        assert f(*args(algo=algo, M=0, v=NUL, m=NUL, X=NUL, Y=NUL)) == p24.P24_OK
    assert f(*args(ldx=32)) == p24.P24_ERR_SHAPE
    assert f(*args(ldx=68, N=60)) == p24.P24_ERR_ALIGN
    assert f(*args(X=MISALIGNED)) == p24.P24_ERR_ALIGN
    assert f(*args(v=NUL)) == p24.P24_ERR_NULL
    assert f(*args(M=0, v=NUL, m=NUL, X=NUL, Y=NUL)) == p24.P24_OK
    assert f(*args(N=0, ldx=0, ldy=0, v=NUL, m=NUL, X=NUL, Y=NUL)) == p24.P24_OK


def test_fused_validation(L):
    f = L.spmm24_fused
    args = lambda **k: [k.get("v", FAKE), k.get("m", FAKE), k.get("layout", 1), k.get("M", 64),
                        k.get("K", 128), k.get("X", FAKE), k.get("ldx", 128), k.get("xo", 0), k.get("N", 64),
                        k.get("Y", FAKE), k.get("yd", 0), k.get("ldy", 64), k.get("bias", NUL),
                        k.get("act", 0), NUL]
    assert f(*args(layout=0)) == p24.P24_ERR_LAYOUT
    assert f(*args(xo=2)) == p24.P24_ERR_UNSUPPORTED
    assert f(*args(act=3)) == p24.P24_ERR_UNSUPPORTED
    assert f(*args(act=-1)) == p24.P24_ERR_UNSUPPORTED
    assert f(*args(K=96)) == p24.P24_ERR_UNSUPPORTED
    assert f(*args(yd=3)) == p24.P24_ERR_DTYPE
    assert f(*args(bias=MISALIGNED)) == p24.P24_ERR_ALIGN
    assert f(*args(v=NUL)) == p24.P24_ERR_NULL
    assert f(*args(ldx=32, xo=0)) == p24.P24_ERR_SHAPE          # K x N: ldx < N
    assert f(*args(ldx=96, xo=1)) == p24.P24_ERR_SHAPE          # N x K: ldx < K
    assert f(*args(M=0, v=NUL, m=NUL, X=NUL, Y=NUL, act=2)) == p24.P24_OK
    assert f(*args(N=0, ldy=0, v=NUL, m=NUL, X=NUL, Y=NUL, act=1)) == p24.P24_OK


def test_tvw_validation(L):
    f = L.tvw_compress
    base = dict(W=FAKE, wd=0, M=256, K=256, ldw=256, tile=128, keep=128, kept=FAKE, v=FAKE, m=FAKE, layout=1,
                ws=FAKE, wsb=1 << 30)
    def call(**k):
        a = {**base, **k}
        return f(a["W"], a["wd"], a["M"], a["K"], a["ldw"], a["tile"], a["keep"], a["kept"], a["v"], a["m"],
                 a["layout"], a["ws"], a["wsb"], NUL)
    assert call(wd=1) == p24.P24_ERR_DTYPE
    assert call(tile=100) == p24.P24_ERR_SHAPE
    assert call(keep=300) == p24.P24_ERR_SHAPE
    assert call(keep=130) == p24.P24_ERR_SHAPE
    assert call(keep=132) == p24.P24_ERR_UNSUPPORTED         # device layout: keep % 64
    assert call(wsb=16) == p24.P24_ERR_WORKSPACE
    assert call(ws=NUL) == p24.P24_ERR_WORKSPACE
    g = L.spmm_tvw
    assert g(FAKE, FAKE, FAKE, 1, 256, 256, 64, 128, FAKE, 64, 64, FAKE, 0, 64, NUL) == p24.P24_ERR_UNSUPPORTED
    assert g(FAKE, FAKE, FAKE, 0, 256, 256, 128, 128, FAKE, 64, 64, FAKE, 0, 64, NUL) == p24.P24_ERR_LAYOUT
    h = L.spmm_tvw_fused      # spmm_tvw's rules plus the epilogue's
    assert h(FAKE, FAKE, FAKE, 1, 256, 256, 128, 128, FAKE, 64, 64, FAKE, 0, 64, NUL, 3, NUL) == p24.P24_ERR_UNSUPPORTED
    assert h(FAKE, FAKE, FAKE, 1, 256, 256, 128, 128, FAKE, 64, 64, FAKE, 0, 64, MISALIGNED, 1, NUL) \
        == p24.P24_ERR_ALIGN
    assert h(FAKE, FAKE, FAKE, 0, 256, 256, 128, 128, FAKE, 64, 64, FAKE, 0, 64, NUL, 1, NUL) == p24.P24_ERR_LAYOUT
    assert h(NUL, NUL, NUL, 1, 0, 256, 128, 128, NUL, 64, 64, NUL, 0, 64, NUL, 2, NUL) == p24.P24_OK
    v = L.spmm_tvw_var_fused
    assert v(FAKE, FAKE, FAKE, FAKE, FAKE, 256, 256, FAKE, 64, 64, FAKE, 0, 64, NUL, -1, NUL) == p24.P24_ERR_UNSUPPORTED
    assert v(FAKE, NUL, FAKE, FAKE, FAKE, 256, 256, FAKE, 64, 64, FAKE, 0, 64, NUL, 1, NUL) == p24.P24_ERR_NULL
    assert v(NUL, NUL, NUL, NUL, NUL, 0, 256, NUL, 64, 64, NUL, 0, 64, NUL, 1, NUL) == p24.P24_OK
    w = L.spmm_tw_fused       # spmm_tw's rules plus the epilogue's
    assert w(FAKE, FAKE, 256, 256, 128, 128, FAKE, 64, 64, FAKE, 0, 64, NUL, 3, NUL) == p24.P24_ERR_UNSUPPORTED
    assert w(FAKE, FAKE, 256, 256, 128, 128, FAKE, 64, 64, FAKE, 0, 64, MISALIGNED, 1, NUL) == p24.P24_ERR_ALIGN
    assert w(FAKE, FAKE, 256, 256, 64, 128, FAKE, 64, 64, FAKE, 0, 64, NUL, 1, NUL) == p24.P24_ERR_UNSUPPORTED
    assert w(FAKE, FAKE, 256, 256, 128, 300, FAKE, 64, 64, FAKE, 0, 64, NUL, 1, NUL) == p24.P24_ERR_SHAPE
    assert w(NUL, FAKE, 256, 256, 128, 128, FAKE, 64, 64, FAKE, 0, 64, NUL, 2, NUL) == p24.P24_ERR_NULL
    assert w(NUL, NUL, 0, 256, 128, 128, NUL, 64, 64, NUL, 0, 64, NUL, 2, NUL) == p24.P24_OK
    u = L.spmm_tw_var_fused
    assert u(FAKE, FAKE, FAKE, FAKE, 256, 256, FAKE, 64, 64, FAKE, 0, 64, NUL, 7, NUL) == p24.P24_ERR_UNSUPPORTED
    assert u(FAKE, FAKE, FAKE, FAKE, 256, 256, FAKE, 64, 64, FAKE, 0, 64, MISALIGNED, 2, NUL) == p24.P24_ERR_ALIGN
    assert u(FAKE, FAKE, FAKE, FAKE, 256, 96, FAKE, 64, 64, FAKE, 0, 64, NUL, 1, NUL) == p24.P24_ERR_UNSUPPORTED
    assert u(FAKE, NUL, FAKE, FAKE, 256, 256, FAKE, 64, 64, FAKE, 0, 64, NUL, 1, NUL) == p24.P24_ERR_NULL
    assert u(NUL, NUL, NUL, NUL, 0, 256, NUL, 64, 64, NUL, 0, 64, NUL, 1, NUL) == p24.P24_OK


def test_tvw_var_validation(L):
    # T = ceil(M / 128) tiles: scores (T*K fp64, 256 B rounded) + selection state (a 2048-bin
    # histogram and the cut, 8216 B, rounded to 8448) + 2 counts per tile
    assert L.tvw_var_workspace_bytes(4096, 4096) == 32 * 4096 * 8 + 8448 + 2 * 32 * 4
    assert L.tvw_var_workspace_bytes(300, 64) == 3 * 64 * 8 + 8448 + 2 * 3 * 4   # 1536 B of scores
    f = L.tvw_var_compress
    base = dict(W=FAKE, wd=0, M=256, K=256, ldw=256, total=256, off=FAKE, order=FAKE, kept=FAKE, v=FAKE, m=FAKE,
                ws=FAKE, wsb=1 << 30)
    def call(**k):
        a = {**base, **k}
        return f(a["W"], a["wd"], a["M"], a["K"], a["ldw"], a["total"], a["off"], a["order"], a["kept"], a["v"],
                 a["m"], a["ws"], a["wsb"], NUL)
    assert call(wd=1) == p24.P24_ERR_DTYPE
    assert call(K=160, ldw=160) == p24.P24_ERR_UNSUPPORTED           # K % 64
    assert call(ldw=128) == p24.P24_ERR_SHAPE
    assert call(total=0) == p24.P24_ERR_SHAPE
    assert call(total=2 * 256 + 1) == p24.P24_ERR_SHAPE               # more than T*K
    assert call(off=NUL) == p24.P24_ERR_NULL
    assert call(order=NUL) == p24.P24_ERR_NULL
    assert call(wsb=16) == p24.P24_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p((1 << 20) + 64)) == p24.P24_ERR_ALIGN   # workspace 256 B aligned
    assert call(off=ctypes.c_void_p((1 << 20) + 4)) == p24.P24_ERR_ALIGN
    assert call(M=0, W=NUL, off=NUL, order=NUL, kept=NUL, v=NUL, m=NUL, ws=NUL) == p24.P24_OK
    g = L.spmm_tvw_var
    gargs = lambda **k: [k.get("off", FAKE), k.get("order", FAKE), k.get("kept", FAKE), k.get("v", FAKE),
                         k.get("m", FAKE), k.get("M", 256), k.get("K", 256), k.get("X", FAKE), k.get("ldx", 64),
                         k.get("N", 64), k.get("Y", FAKE), k.get("yd", 0), k.get("ldy", 64), NUL]
    assert g(*gargs(K=96)) == p24.P24_ERR_UNSUPPORTED
    assert g(*gargs(order=NUL)) == p24.P24_ERR_NULL
    assert g(*gargs(off=ctypes.c_void_p((1 << 20) + 4))) == p24.P24_ERR_ALIGN
    assert g(*gargs(yd=5)) == p24.P24_ERR_DTYPE
    assert g(*gargs(M=0, off=NUL, order=NUL, kept=NUL, v=NUL, m=NUL, X=NUL, Y=NUL)) == p24.P24_OK
    # X addressed with 32 bits: 2 * K * ldx < 2^32
    assert g(*gargs(K=65536, ldx=32768, N=64)) == p24.P24_ERR_UNSUPPORTED
    assert L.spmm_tvw(FAKE, FAKE, FAKE, 1, 256, 65536, 128, 128, FAKE, 32768, 64, FAKE, 0, 64, NUL) \
        == p24.P24_ERR_UNSUPPORTED
    # one K step of X rows: 128 * ldx < 2^32
    assert L.spmm24(FAKE, FAKE, 1, 64, 128, FAKE, 1 << 25, 64, FAKE, 0, 64, 0, NUL) == p24.P24_ERR_UNSUPPORTED


def test_tw_validation(L):
    f = L.tw_compress
    base = dict(W=FAKE, wd=0, M=256, K=256, ldw=256, tile=128, keep=128, kept=FAKE, wp=FAKE, ws=FAKE, wsb=1 << 30)
    def call(**k):
        a = {**base, **k}
        return f(a["W"], a["wd"], a["M"], a["K"], a["ldw"], a["tile"], a["keep"], a["kept"], a["wp"], a["ws"],
                 a["wsb"], NUL)
    assert call(wd=1) == p24.P24_ERR_DTYPE
    assert call(tile=100) == p24.P24_ERR_SHAPE
    assert call(keep=300) == p24.P24_ERR_SHAPE
    assert call(keep=96) == p24.P24_ERR_UNSUPPORTED          # keep % 64
    assert call(wsb=16) == p24.P24_ERR_WORKSPACE
    assert call(wp=MISALIGNED) == p24.P24_ERR_ALIGN
    assert call(kept=NUL) == p24.P24_ERR_NULL
    assert call(M=0, W=NUL, kept=NUL, wp=NUL, ws=NUL) == p24.P24_OK
    g = L.spmm_tw
    gargs = lambda **k: [k.get("kept", FAKE), k.get("wp", FAKE), k.get("M", 256), k.get("K", 256),
                         k.get("tile", 128), k.get("keep", 128), k.get("X", FAKE), k.get("ldx", 64),
                         k.get("N", 64), k.get("Y", FAKE), k.get("yd", 0), k.get("ldy", 64), NUL]
    assert g(*gargs(tile=64)) == p24.P24_ERR_UNSUPPORTED
    assert g(*gargs(keep=96)) == p24.P24_ERR_UNSUPPORTED
    assert g(*gargs(keep=512)) == p24.P24_ERR_SHAPE
    assert g(*gargs(wp=NUL)) == p24.P24_ERR_NULL
    assert g(*gargs(K=65536, ldx=32768)) == p24.P24_ERR_UNSUPPORTED
    assert g(*gargs(M=0, kept=NUL, wp=NUL, X=NUL, Y=NUL)) == p24.P24_OK
    h = L.tw_var_compress
    assert h(FAKE, 0, 256, 160, 160, 100, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, NUL) == p24.P24_ERR_UNSUPPORTED
    assert h(FAKE, 0, 256, 256, 256, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, NUL) == p24.P24_ERR_SHAPE
    assert h(FAKE, 0, 256, 256, 256, 100, FAKE, FAKE, FAKE, NUL, FAKE, 1 << 30, NUL) == p24.P24_ERR_NULL
    assert h(FAKE, 0, 256, 256, 256, 100, FAKE, FAKE, FAKE, FAKE, FAKE, 64, NUL) == p24.P24_ERR_WORKSPACE
    v = L.spmm_tw_var
    assert v(FAKE, NUL, FAKE, FAKE, 256, 256, FAKE, 64, 64, FAKE, 0, 64, NUL) == p24.P24_ERR_NULL
    assert v(FAKE, FAKE, FAKE, FAKE, 256, 96, FAKE, 64, 64, FAKE, 0, 64, NUL) == p24.P24_ERR_UNSUPPORTED
    assert v(NUL, NUL, NUL, NUL, 0, 256, NUL, 64, 64, NUL, 0, 64, NUL) == p24.P24_OK


def test_pattern_validation(L):
    assert L.bw_workspace_bytes(300, 256) == 3 * 256 * 8 + 3 * 4 * 12
    f = L.bw_compress
    assert f(FAKE, 1, 256, 256, 256, 2, FAKE, FAKE, FAKE, 1 << 30, NUL) == p24.P24_ERR_DTYPE
    assert f(FAKE, 0, 256, 200, 200, 2, FAKE, FAKE, FAKE, 1 << 30, NUL) == p24.P24_ERR_UNSUPPORTED   # K % 64
    assert f(FAKE, 0, 256, 256, 256, 5, FAKE, FAKE, FAKE, 1 << 30, NUL) == p24.P24_ERR_SHAPE         # > K/64 blocks
    assert f(FAKE, 0, 256, 256, 256, 0, FAKE, FAKE, FAKE, 1 << 30, NUL) == p24.P24_ERR_SHAPE
    assert f(FAKE, 0, 256, 256, 256, 2, NUL, FAKE, FAKE, 1 << 30, NUL) == p24.P24_ERR_NULL
    assert f(FAKE, 0, 256, 256, 256, 2, FAKE, FAKE, FAKE, 64, NUL) == p24.P24_ERR_WORKSPACE
    assert f(NUL, 0, 0, 256, 256, 2, NUL, NUL, NUL, 0, NUL) == p24.P24_OK
    g = L.ew_compress
    assert g(FAKE, 1, 64, 64, 64, 10, FAKE, FAKE, FAKE, FAKE, 1 << 30, NUL) == p24.P24_ERR_DTYPE
    assert g(FAKE, 0, 64, 64, 64, 0, FAKE, FAKE, FAKE, FAKE, 1 << 30, NUL) == p24.P24_ERR_SHAPE
    assert g(FAKE, 0, 64, 64, 64, 64 * 64 + 1, FAKE, FAKE, FAKE, FAKE, 1 << 30, NUL) == p24.P24_ERR_SHAPE
    assert g(FAKE, 0, 1 << 17, 1 << 16, 1 << 16, 10, FAKE, FAKE, FAKE, FAKE, 1 << 30, NUL) == p24.P24_ERR_SHAPE
    assert g(FAKE, 0, 64, 64, 64, 10, FAKE, NUL, FAKE, FAKE, 1 << 30, NUL) == p24.P24_ERR_NULL
    assert g(FAKE, 0, 64, 64, 64, 10, FAKE, FAKE, FAKE, FAKE, 16, NUL) == p24.P24_ERR_WORKSPACE
    assert g(FAKE, 0, 64, 64, 64, 10, FAKE, FAKE, FAKE, ctypes.c_void_p((1 << 20) + 64), 1 << 30, NUL) \
        == p24.P24_ERR_ALIGN
    h = L.spmm_ew
    assert h(FAKE, FAKE, FAKE, 64, 64, FAKE, 64, 64, FAKE, 7, 64, NUL) == p24.P24_ERR_DTYPE
    assert h(FAKE, FAKE, FAKE, 64, 64, FAKE, 32, 64, FAKE, 0, 64, NUL) == p24.P24_ERR_SHAPE          # ldx < N
    assert h(FAKE, FAKE, FAKE, 64, 64, FAKE, 68, 64, FAKE, 0, 64, NUL) == p24.P24_ERR_ALIGN          # ldx % 8
    assert h(FAKE, NUL, FAKE, 64, 64, FAKE, 64, 64, FAKE, 0, 64, NUL) == p24.P24_ERR_NULL
    assert h(NUL, NUL, NUL, 0, 64, NUL, 64, 64, NUL, 0, 64, NUL) == p24.P24_OK


def test_dense_validation(L):
    assert L.gemm_bf16_pack(FAKE, 64, 96, 96, FAKE, NUL) == p24.P24_ERR_UNSUPPORTED
    assert L.gemm_bf16_pack(FAKE, 64, 128, 132, FAKE, NUL) == p24.P24_ERR_ALIGN
    assert L.gemm_bf16(NUL, 64, 128, FAKE, 64, 64, FAKE, 1, 64, NUL) == p24.P24_ERR_NULL


def test_tvw_compress_noalloc_validation(L):
    """The no-allocation variant checks its arguments as tvw_compress does, and refuses a
    problem whose scores would not fit its fixed scratch, all before touching a device."""
    f = L.tvw_compress_noalloc
    assert f(FAKE, 1, 256, 256, 256, 128, 128, FAKE, FAKE, FAKE, 1, NUL) == p24.P24_ERR_DTYPE
    assert f(FAKE, 0, 256, 256, 256, 128, 128, FAKE, FAKE, FAKE, 7, NUL) == p24.P24_ERR_LAYOUT
    assert f(FAKE, 0, 256, 256, 256, 100, 128, FAKE, FAKE, FAKE, 1, NUL) == p24.P24_ERR_SHAPE     # tile % 32
    assert f(FAKE, 0, 256, 256, 256, 128, 130, FAKE, FAKE, FAKE, 0, NUL) == p24.P24_ERR_SHAPE     # keep % 4
    assert f(FAKE, 0, 256, 256, 256, 128, 100, FAKE, FAKE, FAKE, 1, NUL) == p24.P24_ERR_UNSUPPORTED
    assert f(NUL, 0, 256, 256, 256, 128, 128, FAKE, FAKE, FAKE, 1, NUL) == p24.P24_ERR_NULL
    assert f(MISALIGNED, 0, 256, 256, 256, 128, 128, FAKE, FAKE, FAKE, 1, NUL) == p24.P24_ERR_ALIGN
    assert f(FAKE, 0, 0, 256, 256, 128, 128, NUL, NUL, NUL, 1, NUL) == p24.P24_OK                # M == 0
    # scores of 2048 tiles x 1024 columns (16 MiB) exceed the 8 MiB scratch; 1024 tiles fit exactly
    assert f(FAKE, 0, 2048 * 128, 1024, 1024, 128, 512, FAKE, FAKE, FAKE, 1, NUL) == p24.P24_ERR_SCRATCH
    assert L.tvw_workspace_bytes(1024 * 128, 1024, 128, 512) == L.tvw_noalloc_scratch_bytes()
    assert "scratch" in p24.strerror(p24.P24_ERR_SCRATCH)
