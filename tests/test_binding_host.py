"""Host-side checks of the Python binding's own argument handling (no GPU).

Every entry point refuses host tensors and wrong dtypes before it reaches the
library, so a caller without a device gets a clear error instead of a call
with host pointers; the status-to-exception path names the failing call.
"""
import pytest

torch = pytest.importorskip("torch")
p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")


def test_host_tensors_are_refused():
    W = torch.zeros(128, 128)
    X = torch.zeros(128, 64, dtype=torch.bfloat16)
    for call in (lambda: p24.compress(W), lambda: p24.refresh(W), lambda: p24.tvw_compress(W, 128, 64),
                 lambda: p24.tvw_var_compress(W), lambda: p24.tw_compress(W, 128, 64),
                 lambda: p24.tw_var_compress(W), lambda: p24.bw_compress(W, 1), lambda: p24.ew_compress(W, 10),
                 lambda: p24.pack_dense(W.to(torch.bfloat16)), lambda: p24.transpose(X)):
        with pytest.raises(ValueError, match="device tensor"):
            call()


def test_dtype_rules():
    with pytest.raises(ValueError):
        p24._out_code(torch.float16)
    assert p24._out_code(torch.float32) == p24.P24_F32 and p24._out_code(torch.bfloat16) == p24.P24_BF16
    with pytest.raises(ValueError):
        p24._w_code(torch.zeros(4, 4, dtype=torch.float16))
    assert p24._w_code(torch.zeros(4, 4)) == p24.P24_F32


def test_rowmajor_rule():
    t = torch.zeros(8, 16)
    assert p24._rowmajor(t, "t") == 16
    assert p24._rowmajor(torch.zeros(8, 20)[:, :16], "t") == 20      # padded rows are fine
    with pytest.raises(ValueError):
        p24._rowmajor(t.t(), "t")                                      # column-major
    with pytest.raises(ValueError):
        p24._rowmajor(torch.zeros(2, 3, 4), "t")


def test_fused_argument_rules():
    with pytest.raises(ValueError, match="act"):
        p24._fused_args(None, "tanh", 8, None)
    assert p24._fused_args(None, "none", 8, None) == (None, p24.P24_ACT_NONE, False)
    assert p24._fused_args(None, "gelu", 8, None) == (None, p24.P24_ACT_GELU, True)
    with pytest.raises(ValueError):
        p24._fused_args(torch.zeros(8), "relu", 8, None)                # a host bias


def test_status_becomes_a_named_error():
    with pytest.raises(p24.P24Error, match="spmm24: status -5"):
        p24._check(p24.P24_ERR_UNSUPPORTED, "spmm24")
    p24._check(p24.P24_OK, "spmm24")


class _LibGuard:
    """The real library for its host-only size helpers; any other call fails the test,
    so an argument error must be raised before anything would be launched."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name.endswith("_bytes") or name in ("prune24_strerror", "prune24_abi_version"):
            return getattr(self._real, name)
        raise AssertionError(f"{name} was reached with arguments the binding should refuse")


@pytest.fixture
def meta_device(monkeypatch):
    """Tensors on torch's 'meta' device stand in for device tensors (no GPU here): the
    binding's device check accepts them and refuses host tensors, and the library
    refuses to be called."""
    def require(t, name):
        if t.device.type != "meta":
            raise ValueError(f"{name} must be a CUDA/HIP device tensor")
    monkeypatch.setattr(p24, "_require_cuda", require)
    guard = _LibGuard(p24.lib())
    monkeypatch.setattr(p24, "lib", lambda: guard)
    return torch.device("meta")


def _c24(M, K, dev):
    return p24.Compressed24(torch.empty(M * K // 2, dtype=torch.bfloat16, device=dev),
                            torch.empty(M * K // 32, dtype=torch.int32, device=dev), M, K, p24.P24_LAYOUT_DEVICE)


def test_out_is_checked_before_any_launch(meta_device):
    dev = meta_device
    c = _c24(256, 128, dev)
    X = torch.empty(128, 64, dtype=torch.bfloat16, device=dev)
    XT = torch.empty(64, 128, dtype=torch.bfloat16, device=dev)
    bad_outs = [torch.empty(255, 64, dtype=torch.bfloat16, device=dev),        # too few rows
                torch.empty(256, 32, dtype=torch.bfloat16, device=dev),        # too few columns
                torch.empty(256, 64, dtype=torch.float16, device=dev),         # neither fp32 nor bf16
                torch.empty(256, 64, dtype=torch.bfloat16)]                    # a host tensor
    for out in bad_outs:
        for call in (lambda: p24.spmm24(c, X, out=out), lambda: p24.spmm24_xt(c, XT, out=out),
                     lambda: p24.spmm24(c, X, out=out, act="relu")):
            with pytest.raises(ValueError):
                call()
    t = p24.CompressedTVW(torch.empty(2, 64, dtype=torch.int32, device=dev),
                          torch.empty(256 * 32, dtype=torch.bfloat16, device=dev),
                          torch.empty(256 * 2, dtype=torch.int32, device=dev), 256, 128, 128, 64,
                          p24.P24_LAYOUT_DEVICE)
    tw = p24.CompressedTW(torch.empty(2, 64, dtype=torch.int32, device=dev),
                          torch.empty(256 * 64, dtype=torch.bfloat16, device=dev), 256, 128, 128, 64)
    for out in bad_outs:
        for call in (lambda: p24.spmm_tvw(t, X, out=out), lambda: p24.spmm_tw(tw, X, out=out)):
            with pytest.raises(ValueError):
                call()
    # a host operand of the compressed matrix is refused too
    c_host = p24.Compressed24(torch.empty(256 * 64, dtype=torch.bfloat16), c.meta, 256, 128, c.layout)
    with pytest.raises(ValueError, match="device tensor"):
        p24.spmm24(c_host, X)


def test_gemm_bf16_checks(meta_device):
    dev = meta_device
    M, K, N = 256, 128, 64
    need = p24.lib().gemm_bf16_packed_bytes(M, K)
    Wp = torch.empty(need // 2, dtype=torch.bfloat16, device=dev)
    X = torch.empty(K, N, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="Wp holds"):
        p24.gemm_bf16(Wp[:-1], M, K, X)                                        # undersized packed W
    with pytest.raises(ValueError, match="bfloat16"):
        p24.gemm_bf16(Wp, M, K, torch.empty(K, N, device=dev))                 # fp32 X
    with pytest.raises(ValueError, match="rows"):
        p24.gemm_bf16(Wp, M, K, torch.empty(K + 64, N, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError, match="out is"):
        p24.gemm_bf16(Wp, M, K, X, out=torch.empty(M, N - 8, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError, match="device tensor"):
        p24.gemm_bf16(Wp, M, K, X, out=torch.empty(M, N, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="columns"):
        p24.gemm_bf16_xt(Wp, M, K, torch.empty(N, K + 64, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError, match="Wp holds"):
        p24.gemm_bf16_xt(Wp[: need // 4], M, K, torch.empty(N, K, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError, match="out must be"):
        p24.transpose(X, out=torch.empty(N, K + 1, dtype=torch.bfloat16, device=dev))
