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
