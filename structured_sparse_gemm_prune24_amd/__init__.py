"""Python binding of libprune24.so: 2:4 structured-sparse GEMM on AMD MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/prune24.h``; PyTorch provides
device memory and the current HIP stream, nothing else.  If the library has
not been built this module raises on first use -- there is no fallback.

    import structured_sparse_gemm_prune24_amd as p24
    c = p24.compress(W)                 # W: cuda fp32/bf16 [M, K]  (magnitude 2:4)
    Y = p24.spmm24(c, X)                # X: cuda bf16 [K, N] -> Y bf16 [M, N]
    t = p24.tvw_compress(W, 128, K // 2)
    Y = p24.spmm_tvw(t, X)
    v = p24.tvw_var_compress(W)         # per-tile keep counts from one global ranking
    Y = p24.spmm_tvw_var(v, X)
    w = p24.tw_compress(W, 128, K // 2) # tile column drop only, dense MFMA
    Y = p24.spmm_tw(w, X)
    c = p24.refresh(W); p24.mask_apply(W, c)   # masked fine-tuning
    b = p24.bw_compress(W, 16); e = p24.ew_compress(W, W.numel() // 4)   # comparison patterns
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# P24_LIBRARY may name another build of the same library (the host-sanitized copy
# that build.py --sanitize writes, for CPU test runs)
LIB_PATH = os.environ.get("P24_LIBRARY") or os.path.join(PKG_DIR, "libprune24.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "prune24.h")

# status codes / enums (mirror include/prune24.h)
P24_OK = 0
P24_ERR_NULL = -1
P24_ERR_SHAPE = -2
P24_ERR_ALIGN = -3
P24_ERR_DTYPE = -4
P24_ERR_UNSUPPORTED = -5
P24_ERR_HIP = -6
P24_ERR_WORKSPACE = -7
P24_ERR_LAYOUT = -8
P24_ERR_SCRATCH = -9
P24_F32, P24_BF16 = 0, 1
P24_LAYOUT_CANONICAL, P24_LAYOUT_DEVICE = 0, 1
P24_ALGO_AUTO, P24_ALGO_SMFMAC, P24_ALGO_DECOMP_MFMA = 0, 1, 2
_ALGOS = {"auto": P24_ALGO_AUTO, "smfmac": P24_ALGO_SMFMAC, "decomp_mfma": P24_ALGO_DECOMP_MFMA}
P24_X_KN, P24_X_NK = 0, 1
P24_ACT_NONE, P24_ACT_RELU, P24_ACT_GELU = 0, 1, 2
_ACTS = {"none": P24_ACT_NONE, "relu": P24_ACT_RELU, "gelu": P24_ACT_GELU}

_c_i32, _c_i64, _c_size, _c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes)
_SIGNATURES = {
    "prune24_abi_version": (_c_i32, []),
    "prune24_strerror": (ctypes.c_char_p, [_c_i32]),
    "prune24_values_bytes": (_c_size, [_c_i64, _c_i64, _c_i32]),
    "prune24_meta_bytes": (_c_size, [_c_i64, _c_i64, _c_i32]),
    "prune24_compress": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_i32, _c_vp]),
    "prune24_refresh": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_i32, _c_vp]),
    "prune24_mask_apply": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_vp, _c_i32, _c_vp]),
    "prune24_decompress": (_c_i32, [_c_vp, _c_vp, _c_i32, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp]),
    "spmm24": (_c_i32, [_c_vp, _c_vp, _c_i32, _c_i64, _c_i64, _c_vp, _c_i64, _c_i64, _c_vp, _c_i32,
                        _c_i64, _c_i32, _c_vp]),
    "tvw_workspace_bytes": (_c_size, [_c_i64, _c_i64, _c_i64, _c_i64]),
    "tvw_compress": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp,
                              _c_i32, _c_vp, _c_size, _c_vp]),
    "tvw_noalloc_scratch_bytes": (_c_size, []),
    "tvw_compress_noalloc": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp,
                                      _c_i32, _c_vp]),
    "spmm_tvw": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_i64,
                          _c_i64, _c_vp, _c_i32, _c_i64, _c_vp]),
    "spmm_tvw_fused": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_i64,
                                _c_i64, _c_vp, _c_i32, _c_i64, _c_vp, _c_i32, _c_vp]),
    "spmm24_tvw_chain": (_c_i32, [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_i32, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64,
                                  _c_i64, _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_i32, _c_i64, _c_vp, _c_i32,
                                  _c_vp]),
    "spmm_tvw_var_fused": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_i64,
                                    _c_vp, _c_i32, _c_i64, _c_vp, _c_i32, _c_vp]),
    "tvw_var_workspace_bytes": (_c_size, [_c_i64, _c_i64]),
    "tvw_var_compress": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp,
                                  _c_vp, _c_vp, _c_size, _c_vp]),
    "spmm_tvw_var": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_i64, _c_vp,
                              _c_i32, _c_i64, _c_vp]),
    "tw_compress": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_size,
                             _c_vp]),
    "spmm_tw": (_c_i32, [_c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_i64, _c_vp, _c_i32, _c_i64,
                         _c_vp]),
    "tw_var_compress": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                 _c_size, _c_vp]),
    "spmm_tw_var": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_i64, _c_vp, _c_i32,
                             _c_i64, _c_vp]),
    "spmm_tw_fused": (_c_i32, [_c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_i64, _c_vp, _c_i32,
                               _c_i64, _c_vp, _c_i32, _c_vp]),
    "spmm_tw_var_fused": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_i64, _c_vp,
                                   _c_i32, _c_i64, _c_vp, _c_i32, _c_vp]),
    "bw_workspace_bytes": (_c_size, [_c_i64, _c_i64]),
    "bw_compress": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
    "ew_workspace_bytes": (_c_size, [_c_i64, _c_i64]),
    "ew_compress": (_c_i32, [_c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_size,
                             _c_vp]),
    "spmm_ew": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_i64, _c_vp, _c_i32, _c_i64, _c_vp]),
    "spmm24_xt": (_c_i32, [_c_vp, _c_vp, _c_i32, _c_i64, _c_i64, _c_vp, _c_i64, _c_i64, _c_vp, _c_i32,
                           _c_i64, _c_vp]),
    "spmm24_fused": (_c_i32, [_c_vp, _c_vp, _c_i32, _c_i64, _c_i64, _c_vp, _c_i64, _c_i32, _c_i64, _c_vp,
                              _c_i32, _c_i64, _c_vp, _c_i32, _c_vp]),
    "transpose_bf16": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp]),
    "gemm_bf16_xt": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_i64, _c_vp, _c_i32, _c_i64, _c_vp]),
    "gemm_bf16_packed_bytes": (_c_size, [_c_i64, _c_i64]),
    "gemm_bf16_pack": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp]),
    "gemm_bf16": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_i64, _c_vp, _c_i32, _c_i64, _c_vp]),
}

_LIB = None


class P24Error(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: status {code} ({strerror(code)})")


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python structured_sparse_gemm_prune24_amd/build.py")
        # One HIP runtime per process: torch opens its own copy by path, so torch is
        # loaded first and the library, which names the runtime by soname, binds to
        # that copy instead of bringing a second one.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def header_symbols() -> list[str]:
    """Entry points declared with P24_API in include/prune24.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return re.findall(r"P24_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def strerror(code: int) -> str:
    return lib().prune24_strerror(code).decode()


def _check(code: int, where: str):
    if code != P24_OK:
        raise P24Error(code, where)


# ----------------------------------------------------------------------------
# tensor plumbing
# ----------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream(dev):
    torch = _torch()
    return _c_vp(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return _c_vp(t.data_ptr())


def _require_cuda(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA/HIP device tensor")


def _rowmajor(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit stride along its last dimension")
    return t.stride(0)


def _same_device(t, dev, name):
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, the operation runs on {dev}")


def _x_bf16(X, name, device=None):
    """X must be a bf16 device tensor, 2-D, unit stride along its last dimension; returns its row stride."""
    torch = _torch()
    _require_cuda(X, name)
    if X.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16")
    if device is not None:
        _same_device(X, device, name)
    return _rowmajor(X, name)


def _operands_on(device, *named):
    """Every (tensor, name) of a compressed operand must live on the device the product runs on."""
    for t, name in named:
        if t is not None:
            _require_cuda(t, name)
            _same_device(t, device, name)


def _out_tensor(out, M, N, out_dtype, device):
    """The output: a new (M, N) tensor, or the caller's, checked before any launch: a device
    tensor on `device`, shape exactly (M, N), fp32 or bf16, unit column stride."""
    torch = _torch()
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=device)
    else:
        _require_cuda(out, "out")
        _same_device(out, device, "out")
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out is {tuple(out.shape)}, the product is {(M, N)}")
    ldy = _rowmajor(out, "out")
    _out_code(out.dtype)
    return out, ldy


def _out_code(out_dtype):
    torch = _torch()
    if out_dtype == torch.float32:
        return P24_F32
    if out_dtype == torch.bfloat16:
        return P24_BF16
    raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")


def _layout_code(layout):
    if layout in ("device", P24_LAYOUT_DEVICE):
        return P24_LAYOUT_DEVICE
    if layout in ("canonical", P24_LAYOUT_CANONICAL):
        return P24_LAYOUT_CANONICAL
    raise ValueError("layout must be 'device' or 'canonical'")


@dataclass
class Compressed24:
    """A 2:4-compressed M x K matrix: bf16 values + int32 words of 2-bit positions."""
    values: object       # torch.bfloat16, flat
    meta: object         # torch.int32, flat (bit patterns of the uint32 words)
    M: int
    K: int
    layout: int


@dataclass
class CompressedTVW:
    """TVW-compressed matrix: kept column lists per tile + 2:4 compression of the compacted rows."""
    kept: object         # torch.int32 [T, keep_k]
    values: object
    meta: object
    M: int
    K: int
    tile_m: int
    keep_k: int
    layout: int


@dataclass
class CompressedTVWVar:
    """TVW with a keep count per 128-row tile: tile t's columns are
    kept[offsets[t]:offsets[t+1]] and its device-layout storage starts at
    column offsets[t] of the concatenation; `order` lists the tiles heaviest first."""
    offsets: object      # torch.int64 [T + 1]
    order: object        # torch.int32 [T]
    kept: object         # torch.int32, capacity T*K
    values: object       # torch.bfloat16, capacity T*K*64
    meta: object         # torch.int32, capacity T*K*4
    M: int
    K: int
    total_keep: int


@dataclass
class CompressedTW:
    """TW (tile column drop, no 2:4): kept lists per tile + the dense bf16 operand of the kept columns."""
    kept: object         # torch.int32 [T, keep_k]
    Wp: object           # torch.bfloat16, dense operand order
    M: int
    K: int
    tile_m: int
    keep_k: int


@dataclass
class CompressedTWVar:
    """TW with a keep count per 128-row tile (storage as CompressedTVWVar, dense per tile)."""
    offsets: object      # torch.int64 [T + 1]
    order: object        # torch.int32 [T]
    kept: object         # torch.int32, capacity T*K
    Wp: object           # torch.bfloat16, capacity T*K*128
    M: int
    K: int
    total_keep: int


def _w_code(W):
    torch = _torch()
    if W.dtype == torch.float32:
        return P24_F32
    if W.dtype == torch.bfloat16:
        return P24_BF16
    raise ValueError("W must be float32 or bfloat16")


@dataclass
class CompressedEW:
    """Unstructured sparsity in CSR form (bf16 values)."""
    row_ptr: object      # torch.int64 [M + 1]
    cols: object         # torch.int32 [keep_total]
    vals: object         # torch.bfloat16 [keep_total]
    M: int
    K: int
    keep_total: int


def compress(W, layout="device") -> Compressed24:
    """Magnitude 2:4 prune + compress of W (cuda fp32 or bf16, [M, K])."""
    return _compress(W, layout, refresh=False)


def _compress(W, layout, refresh: bool) -> Compressed24:
    torch = _torch()
    _require_cuda(W, "W")
    ldw = _rowmajor(W, "W")
    wd = _w_code(W)
    M, K = W.shape
    lc = _layout_code(layout)
    L = lib()
    vb, mb = L.prune24_values_bytes(M, K, lc), L.prune24_meta_bytes(M, K, lc)
    if (vb == 0 or mb == 0) and M * K:
        raise P24Error(P24_ERR_SHAPE if K % 4 else P24_ERR_UNSUPPORTED, "prune24_compress")
    values = torch.empty(max(vb // 2, 1), dtype=torch.bfloat16, device=W.device)
    meta = torch.empty(max(mb // 4, 1), dtype=torch.int32, device=W.device)
    f, name = (L.prune24_refresh, "prune24_refresh") if refresh else (L.prune24_compress, "prune24_compress")
    _check(f(_ptr(W), wd, M, K, ldw, _ptr(values), _ptr(meta), lc, _stream(W.device)), name)
    return Compressed24(values, meta, M, K, lc)


def refresh(W, layout="device") -> Compressed24:
    """Re-prune for masked fine-tuning: compress(W) and, in the same pass, W's dropped entries
    set to +0 in place."""
    return _compress(W, layout, refresh=True)


def mask_apply(W, c: Compressed24):
    """W[m][k] := +0 wherever c's stored positions do not select k (in place); returns W."""
    _require_cuda(W, "W")
    ldw = _rowmajor(W, "W")
    if tuple(W.shape) != (c.M, c.K):
        raise ValueError(f"W is {tuple(W.shape)}, the mask is for {(c.M, c.K)}")
    _check(lib().prune24_mask_apply(_ptr(W), _w_code(W), c.M, c.K, ldw, _ptr(c.meta), c.layout,
                                    _stream(W.device)), "prune24_mask_apply")
    return W


def decompress(c: Compressed24):
    """Dense bf16 [M, K] with the kept values in place and zeros elsewhere."""
    torch = _torch()
    out = torch.empty((c.M, c.K), dtype=torch.bfloat16, device=c.values.device)
    _check(lib().prune24_decompress(_ptr(c.values), _ptr(c.meta), c.layout, c.M, c.K, _ptr(out), c.K,
                                    _stream(out.device)), "prune24_decompress")
    return out


def _fused_args(bias, act, M, device):
    """(bias pointer, act code, needs fused) after checking bias and act."""
    torch = _torch()
    if act not in _ACTS:
        raise ValueError(f"act must be one of {sorted(_ACTS)}")
    if bias is None:
        return None, _ACTS[act], act != "none"
    _require_cuda(bias, "bias")
    if bias.dtype != torch.float32 or bias.dim() != 1 or bias.shape[0] != M or not bias.is_contiguous():
        raise ValueError(f"bias must be a contiguous fp32 vector of {M} values")
    if bias.device != device:
        raise ValueError("bias must be on the same device as X")
    return _ptr(bias), _ACTS[act], True


def spmm24(c: Compressed24, X, out_dtype=None, out=None, algo="auto", bias=None, act="none"):
    """Y = act(W X + bias) for compressed W (device layout) and X bf16 [K, N].

    algo: "smfmac" (sparse MFMA on the compressed operand; what "auto" picks) or
    "decomp_mfma" (operand expanded to a dense LDS tile, dense MFMA).
    bias (fp32 [M], one value per output row) and act ("none", "relu", "gelu")
    run fused in the sparse-MFMA kernel's epilogue."""
    if algo not in _ALGOS:
        raise ValueError(f"algo must be one of {sorted(_ALGOS)}")
    ldx = _x_bf16(X, "X")
    if X.shape[0] != c.K:
        raise ValueError(f"X has {X.shape[0]} rows, W has K = {c.K}")
    N = X.shape[1]
    _operands_on(X.device, (c.values, "values"), (c.meta, "meta"))
    out, ldy = _out_tensor(out, c.M, N, out_dtype, X.device)
    bptr, act_code, fused = _fused_args(bias, act, c.M, X.device)
    if fused:
        if algo == "decomp_mfma":
            raise ValueError("the fused epilogue runs with the sparse MFMA (algo 'auto' or 'smfmac')")
        _check(lib().spmm24_fused(_ptr(c.values), _ptr(c.meta), c.layout, c.M, c.K, _ptr(X), ldx, P24_X_KN, N,
                                  _ptr(out), _out_code(out.dtype), ldy, bptr, act_code, _stream(X.device)),
               "spmm24_fused")
        return out
    _check(lib().spmm24(_ptr(c.values), _ptr(c.meta), c.layout, c.M, c.K, _ptr(X), ldx, N, _ptr(out),
                        _out_code(out.dtype), ldy, _ALGOS[algo], _stream(X.device)), "spmm24")
    return out


def tvw_compress(W, tile_m: int = 128, keep_k: int | None = None, layout="device") -> CompressedTVW:
    """TVW selection (per tile_m-row tile keep keep_k columns by L1 norm) + 2:4 compression."""
    torch = _torch()
    _require_cuda(W, "W")
    if W.dtype != torch.float32:
        raise ValueError("tvw_compress takes fp32 W")
    ldw = _rowmajor(W, "W")
    M, K = W.shape
    keep_k = K // 2 if keep_k is None else int(keep_k)
    lc = _layout_code(layout)
    L = lib()
    T = (M + tile_m - 1) // tile_m
    vb, mb = L.prune24_values_bytes(M, keep_k, lc), L.prune24_meta_bytes(M, keep_k, lc)
    wsb = L.tvw_workspace_bytes(M, K, tile_m, keep_k)
    kept = torch.empty((T, keep_k), dtype=torch.int32, device=W.device)
    values = torch.empty(max(vb // 2, 1), dtype=torch.bfloat16, device=W.device)
    meta = torch.empty(max(mb // 4, 1), dtype=torch.int32, device=W.device)
    ws = torch.empty(max(wsb, 8), dtype=torch.uint8, device=W.device)
    _check(L.tvw_compress(_ptr(W), P24_F32, M, K, ldw, tile_m, keep_k, _ptr(kept), _ptr(values), _ptr(meta),
                          lc, _ptr(ws), ws.numel(), _stream(W.device)), "tvw_compress")
    return CompressedTVW(kept, values, meta, M, K, tile_m, keep_k, lc)


def tvw_compress_noalloc(W, tile_m: int = 128, keep_k: int | None = None, layout="device", out=None):
    """tvw_compress through the library's no-allocation entry point (its fixed device scratch,
    no workspace).  `out`, a CompressedTVW of the same shape, receives the result in place
    (then nothing is allocated here either); without it the output tensors are new."""
    torch = _torch()
    _require_cuda(W, "W")
    if W.dtype != torch.float32:
        raise ValueError("tvw_compress_noalloc takes fp32 W")
    ldw = _rowmajor(W, "W")
    M, K = W.shape
    keep_k = K // 2 if keep_k is None else int(keep_k)
    lc = _layout_code(layout)
    L = lib()
    T = (M + tile_m - 1) // tile_m
    if out is None:
        vb, mb = L.prune24_values_bytes(M, keep_k, lc), L.prune24_meta_bytes(M, keep_k, lc)
        out = CompressedTVW(torch.empty((T, keep_k), dtype=torch.int32, device=W.device),
                            torch.empty(max(vb // 2, 1), dtype=torch.bfloat16, device=W.device),
                            torch.empty(max(mb // 4, 1), dtype=torch.int32, device=W.device),
                            M, K, tile_m, keep_k, lc)
    elif (out.M, out.K, out.tile_m, out.keep_k, out.layout) != (M, K, tile_m, keep_k, lc):
        raise ValueError("out was made for another shape, tile, keep count or layout")
    _operands_on(W.device, (out.kept, "kept"), (out.values, "values"), (out.meta, "meta"))
    _check(L.tvw_compress_noalloc(_ptr(W), P24_F32, M, K, ldw, tile_m, keep_k, _ptr(out.kept), _ptr(out.values),
                                  _ptr(out.meta), lc, _stream(W.device)), "tvw_compress_noalloc")
    return out


def spmm_tvw(t: CompressedTVW, X, out_dtype=None, out=None, bias=None, act="none"):
    """Y = act(W X + bias) for a TVW-compressed W; X bf16 [K, N] (rows gathered per tile)."""
    ldx = _x_bf16(X, "X")
    if X.shape[0] != t.K:
        raise ValueError(f"X has {X.shape[0]} rows, W has K = {t.K}")
    N = X.shape[1]
    _operands_on(X.device, (t.kept, "kept"), (t.values, "values"), (t.meta, "meta"))
    out, ldy = _out_tensor(out, t.M, N, out_dtype, X.device)
    bptr, act_code, fused = _fused_args(bias, act, t.M, X.device)
    if fused:
        _check(lib().spmm_tvw_fused(_ptr(t.kept), _ptr(t.values), _ptr(t.meta), t.layout, t.M, t.K, t.tile_m,
                                    t.keep_k, _ptr(X), ldx, N, _ptr(out), _out_code(out.dtype), ldy, bptr, act_code,
                                    _stream(X.device)), "spmm_tvw_fused")
        return out
    _check(lib().spmm_tvw(_ptr(t.kept), _ptr(t.values), _ptr(t.meta), t.layout, t.M, t.K, t.tile_m, t.keep_k,
                          _ptr(X), ldx, N, _ptr(out), _out_code(out.dtype), ldy, _stream(X.device)), "spmm_tvw")
    return out


def spmm24_tvw_chain(c1: Compressed24, t2: CompressedTVW, X, bias1=None, act1="gelu", bias2=None, act2="none",
                     out_dtype=None, out=None, hidden=None):
    """Two layers: H = bf16(act1(W1 X + bias1)) with W1 2:4-compressed, then
    Y2 = act2(W2 H + bias2) with W2 TVW-compressed over K = W1's rows.  Layer 1's
    epilogue writes H in the row-major layout layer 2's gather reads.  Returns (Y2, H);
    `hidden` may supply H's buffer (bf16 [M1, N])."""
    torch = _torch()
    ldx = _x_bf16(X, "X")
    if X.shape[0] != c1.K:
        raise ValueError(f"X has {X.shape[0]} rows, W1 has K = {c1.K}")
    if t2.K != c1.M:
        raise ValueError(f"layer 2 takes K = {t2.K} inputs, layer 1 gives {c1.M}")
    if c1.layout != P24_LAYOUT_DEVICE or t2.layout != P24_LAYOUT_DEVICE:
        raise ValueError("both layers must be in the device layout")
    N = X.shape[1]
    _operands_on(X.device, (c1.values, "values1"), (c1.meta, "meta1"), (t2.kept, "kept2"), (t2.values, "values2"),
                 (t2.meta, "meta2"))
    if hidden is None:
        hidden = torch.empty((c1.M, N), dtype=torch.bfloat16, device=X.device)
    else:
        _require_cuda(hidden, "hidden")
        _same_device(hidden, X.device, "hidden")
        if hidden.dtype != torch.bfloat16 or tuple(hidden.shape) != (c1.M, N):
            raise ValueError(f"hidden must be bfloat16 of shape {(c1.M, N)}")
    ldh = _rowmajor(hidden, "hidden")
    out, ldy = _out_tensor(out, t2.M, N, out_dtype, X.device)
    b1, a1, _ = _fused_args(bias1, act1, c1.M, X.device)
    b2, a2, _ = _fused_args(bias2, act2, t2.M, X.device)
    _check(lib().spmm24_tvw_chain(_ptr(c1.values), _ptr(c1.meta), c1.M, c1.K, b1, a1, _ptr(t2.kept), _ptr(t2.values),
                                  _ptr(t2.meta), t2.M, t2.tile_m, t2.keep_k, _ptr(X), ldx, N, _ptr(hidden), ldh,
                                  _ptr(out), _out_code(out.dtype), ldy, b2, a2, _stream(X.device)),
           "spmm24_tvw_chain")
    return out, hidden


def tvw_var_compress(W, total_keep: int | None = None) -> CompressedTVWVar:
    """TVW with per-tile keep counts from one global ranking of the 128-row tiles'
    column scores (total_keep columns over all tiles, default half of them)."""
    torch = _torch()
    _require_cuda(W, "W")
    if W.dtype != torch.float32:
        raise ValueError("tvw_var_compress takes fp32 W")
    ldw = _rowmajor(W, "W")
    M, K = W.shape
    T = (M + 127) // 128
    total_keep = T * K // 2 if total_keep is None else int(total_keep)
    L = lib()
    dev = W.device
    cap = max(T * K, 1)
    offsets = torch.empty(T + 1, dtype=torch.int64, device=dev)
    order = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    kept = torch.empty(cap, dtype=torch.int32, device=dev)
    values = torch.empty(cap * 64, dtype=torch.bfloat16, device=dev)
    meta = torch.empty(cap * 4, dtype=torch.int32, device=dev)
    wsb = L.tvw_var_workspace_bytes(M, K)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    _check(L.tvw_var_compress(_ptr(W), P24_F32, M, K, ldw, total_keep, _ptr(offsets), _ptr(order), _ptr(kept),
                              _ptr(values), _ptr(meta), _ptr(ws), ws.numel(), _stream(dev)), "tvw_var_compress")
    return CompressedTVWVar(offsets, order, kept, values, meta, M, K, total_keep)


def spmm_tvw_var(t: CompressedTVWVar, X, out_dtype=None, out=None, bias=None, act="none"):
    """Y = act(W X + bias) for a per-tile-keep TVW matrix; X bf16 [K, N]."""
    ldx = _x_bf16(X, "X")
    if X.shape[0] != t.K:
        raise ValueError(f"X has {X.shape[0]} rows, W has K = {t.K}")
    N = X.shape[1]
    _operands_on(X.device, (t.offsets, "offsets"), (t.order, "order"), (t.kept, "kept"), (t.values, "values"),
                 (t.meta, "meta"))
    out, ldy = _out_tensor(out, t.M, N, out_dtype, X.device)
    bptr, act_code, fused = _fused_args(bias, act, t.M, X.device)
    if fused:
        _check(lib().spmm_tvw_var_fused(_ptr(t.offsets), _ptr(t.order), _ptr(t.kept), _ptr(t.values), _ptr(t.meta),
                                        t.M, t.K, _ptr(X), ldx, N, _ptr(out), _out_code(out.dtype), ldy, bptr,
                                        act_code, _stream(X.device)), "spmm_tvw_var_fused")
        return out
    _check(lib().spmm_tvw_var(_ptr(t.offsets), _ptr(t.order), _ptr(t.kept), _ptr(t.values), _ptr(t.meta), t.M,
                              t.K, _ptr(X), ldx, N, _ptr(out), _out_code(out.dtype), ldy, _stream(X.device)),
           "spmm_tvw_var")
    return out


def _x_out(X, K, M, out_dtype, out, *operands):
    """X checks, the compressed operand's tensors on X's device, and the output."""
    ldx = _x_bf16(X, "X")
    if X.shape[0] != K:
        raise ValueError(f"X has {X.shape[0]} rows, W has K = {K}")
    _operands_on(X.device, *operands)
    out, ldy = _out_tensor(out, M, X.shape[1], out_dtype, X.device)
    return ldx, X.shape[1], out, ldy


def tw_compress(W, tile_m: int = 128, keep_k: int | None = None) -> CompressedTW:
    """TW: per tile_m-row tile keep keep_k columns by L1 norm; the kept columns stay dense (bf16)."""
    torch = _torch()
    _require_cuda(W, "W")
    if W.dtype != torch.float32:
        raise ValueError("tw_compress takes fp32 W")
    ldw = _rowmajor(W, "W")
    M, K = W.shape
    keep_k = K // 2 if keep_k is None else int(keep_k)
    L = lib()
    T = (M + tile_m - 1) // tile_m
    kept = torch.empty((T, keep_k), dtype=torch.int32, device=W.device)
    Wp = torch.empty(max(L.gemm_bf16_packed_bytes(M, keep_k) // 2, 1), dtype=torch.bfloat16, device=W.device)
    wsb = L.tvw_workspace_bytes(M, K, tile_m, keep_k)
    ws = torch.empty(max(wsb, 8), dtype=torch.uint8, device=W.device)
    _check(L.tw_compress(_ptr(W), P24_F32, M, K, ldw, tile_m, keep_k, _ptr(kept), _ptr(Wp), _ptr(ws), ws.numel(),
                         _stream(W.device)), "tw_compress")
    return CompressedTW(kept, Wp, M, K, tile_m, keep_k)


def spmm_tw(t: CompressedTW, X, out_dtype=None, out=None, bias=None, act="none"):
    """Y = act(W X + bias) for a TW-compressed W; X bf16 [K, N] (rows gathered per tile)."""
    ldx, N, out, ldy = _x_out(X, t.K, t.M, out_dtype, out, (t.kept, "kept"), (t.Wp, "Wp"))
    bptr, act_code, fused = _fused_args(bias, act, t.M, X.device)
    if fused:
        _check(lib().spmm_tw_fused(_ptr(t.kept), _ptr(t.Wp), t.M, t.K, t.tile_m, t.keep_k, _ptr(X), ldx, N,
                                   _ptr(out), _out_code(out.dtype), ldy, bptr, act_code, _stream(X.device)),
               "spmm_tw_fused")
        return out
    _check(lib().spmm_tw(_ptr(t.kept), _ptr(t.Wp), t.M, t.K, t.tile_m, t.keep_k, _ptr(X), ldx, N, _ptr(out),
                         _out_code(out.dtype), ldy, _stream(X.device)), "spmm_tw")
    return out


def tw_var_compress(W, total_keep: int | None = None) -> CompressedTWVar:
    """TW with per-tile keep counts (the plan of tvw_var_compress), kept columns dense (bf16)."""
    torch = _torch()
    _require_cuda(W, "W")
    if W.dtype != torch.float32:
        raise ValueError("tw_var_compress takes fp32 W")
    ldw = _rowmajor(W, "W")
    M, K = W.shape
    T = (M + 127) // 128
    total_keep = T * K // 2 if total_keep is None else int(total_keep)
    L = lib()
    dev = W.device
    cap = max(T * K, 1)
    offsets = torch.empty(T + 1, dtype=torch.int64, device=dev)
    order = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    kept = torch.empty(cap, dtype=torch.int32, device=dev)
    Wp = torch.empty(cap * 128, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(L.tvw_var_workspace_bytes(M, K), 256), dtype=torch.uint8, device=dev)
    _check(L.tw_var_compress(_ptr(W), P24_F32, M, K, ldw, total_keep, _ptr(offsets), _ptr(order), _ptr(kept),
                             _ptr(Wp), _ptr(ws), ws.numel(), _stream(dev)), "tw_var_compress")
    return CompressedTWVar(offsets, order, kept, Wp, M, K, total_keep)


def spmm_tw_var(t: CompressedTWVar, X, out_dtype=None, out=None, bias=None, act="none"):
    """Y = act(W X + bias) for a per-tile-keep TW matrix; X bf16 [K, N]."""
    ldx, N, out, ldy = _x_out(X, t.K, t.M, out_dtype, out, (t.offsets, "offsets"), (t.order, "order"),
                              (t.kept, "kept"), (t.Wp, "Wp"))
    bptr, act_code, fused = _fused_args(bias, act, t.M, X.device)
    if fused:
        _check(lib().spmm_tw_var_fused(_ptr(t.offsets), _ptr(t.order), _ptr(t.kept), _ptr(t.Wp), t.M, t.K,
                                       _ptr(X), ldx, N, _ptr(out), _out_code(out.dtype), ldy, bptr, act_code,
                                       _stream(X.device)), "spmm_tw_var_fused")
        return out
    _check(lib().spmm_tw_var(_ptr(t.offsets), _ptr(t.order), _ptr(t.kept), _ptr(t.Wp), t.M, t.K, _ptr(X), ldx, N,
                             _ptr(out), _out_code(out.dtype), ldy, _stream(X.device)), "spmm_tw_var")
    return out


def bw_compress(W, keep_blocks: int) -> CompressedTW:
    """Block-wise: per 128-row tile keep the keep_blocks 64-column blocks of largest L1 norm;
    the result runs with spmm_tw."""
    torch = _torch()
    _require_cuda(W, "W")
    if W.dtype != torch.float32:
        raise ValueError("bw_compress takes fp32 W")
    ldw = _rowmajor(W, "W")
    M, K = W.shape
    keep = int(keep_blocks) * 64
    L = lib()
    T = (M + 127) // 128
    kept = torch.empty((T, keep), dtype=torch.int32, device=W.device)
    Wp = torch.empty(max(L.gemm_bf16_packed_bytes(M, keep) // 2, 1), dtype=torch.bfloat16, device=W.device)
    ws = torch.empty(max(L.bw_workspace_bytes(M, K), 8), dtype=torch.uint8, device=W.device)
    _check(L.bw_compress(_ptr(W), P24_F32, M, K, ldw, int(keep_blocks), _ptr(kept), _ptr(Wp), _ptr(ws),
                         ws.numel(), _stream(W.device)), "bw_compress")
    return CompressedTW(kept, Wp, M, K, 128, keep)


def ew_compress(W, keep_total: int) -> CompressedEW:
    """Unstructured: the keep_total largest-magnitude weights of the whole matrix, in CSR form."""
    torch = _torch()
    _require_cuda(W, "W")
    if W.dtype != torch.float32:
        raise ValueError("ew_compress takes fp32 W")
    ldw = _rowmajor(W, "W")
    M, K = W.shape
    keep_total = int(keep_total)
    L = lib()
    dev = W.device
    row_ptr = torch.empty(M + 1, dtype=torch.int64, device=dev)
    cols = torch.empty(max(keep_total, 1), dtype=torch.int32, device=dev)
    vals = torch.empty(max(keep_total, 1), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(L.ew_workspace_bytes(M, K), 256), dtype=torch.uint8, device=dev)
    _check(L.ew_compress(_ptr(W), P24_F32, M, K, ldw, keep_total, _ptr(row_ptr), _ptr(cols), _ptr(vals), _ptr(ws),
                         ws.numel(), _stream(dev)), "ew_compress")
    return CompressedEW(row_ptr, cols, vals, M, K, keep_total)


def spmm_ew(t: CompressedEW, X, out_dtype=None, out=None):
    """Y = W X for an unstructured (CSR) W; X bf16 [K, N]."""
    ldx, N, out, ldy = _x_out(X, t.K, t.M, out_dtype, out, (t.row_ptr, "row_ptr"), (t.cols, "cols"),
                              (t.vals, "vals"))
    _check(lib().spmm_ew(_ptr(t.row_ptr), _ptr(t.cols), _ptr(t.vals), t.M, t.K, _ptr(X), ldx, N, _ptr(out),
                         _out_code(out.dtype), ldy, _stream(X.device)), "spmm_ew")
    return out


def pack_dense(W):
    """Dense bf16 W [M, K] -> MFMA operand order (input of gemm_bf16)."""
    torch = _torch()
    _require_cuda(W, "W")
    if W.dtype != torch.bfloat16:
        raise ValueError("W must be bfloat16")
    ldw = _rowmajor(W, "W")
    M, K = W.shape
    nb = lib().gemm_bf16_packed_bytes(M, K)
    if nb == 0 and M * K:
        raise P24Error(P24_ERR_UNSUPPORTED, "gemm_bf16_pack")
    Wp = torch.empty(max(nb // 2, 1), dtype=torch.bfloat16, device=W.device)
    _check(lib().gemm_bf16_pack(_ptr(W), M, K, ldw, _ptr(Wp), _stream(W.device)), "gemm_bf16_pack")
    return Wp


def _packed_w(Wp, M: int, K: int, device):
    """Wp: a bf16 device tensor on `device` holding at least gemm_bf16_packed_bytes(M, K)."""
    torch = _torch()
    _require_cuda(Wp, "Wp")
    _same_device(Wp, device, "Wp")
    if Wp.dtype != torch.bfloat16:
        raise ValueError("Wp must be bfloat16 (the output of pack_dense)")
    need = lib().gemm_bf16_packed_bytes(M, K)
    if need == 0 and M * K:
        raise P24Error(P24_ERR_UNSUPPORTED, "gemm_bf16")
    if Wp.numel() * 2 < need:
        raise ValueError(f"Wp holds {Wp.numel() * 2} bytes, a packed {M} x {K} matrix needs {need}")


def gemm_bf16(Wp, M: int, K: int, X, out_dtype=None, out=None):
    """Dense baseline Y = W X from packed W (see pack_dense)."""
    ldx = _x_bf16(X, "X")
    if X.shape[0] != K:
        raise ValueError(f"X has {X.shape[0]} rows, W has K = {K}")
    N = X.shape[1]
    _packed_w(Wp, M, K, X.device)
    out, ldy = _out_tensor(out, M, N, out_dtype, X.device)
    _check(lib().gemm_bf16(_ptr(Wp), M, K, _ptr(X), ldx, N, _ptr(out), _out_code(out.dtype), ldy,
                           _stream(X.device)), "gemm_bf16")
    return out


def transpose(src, out=None):
    """bf16 src [R, C] -> out [C, R] (bit copy on the GPU)."""
    torch = _torch()
    lds = _x_bf16(src, "src")
    R, Cc = src.shape
    if out is None:
        out = torch.empty((Cc, R), dtype=src.dtype, device=src.device)
    else:
        _require_cuda(out, "out")
        _same_device(out, src.device, "out")
        if out.dtype != torch.bfloat16 or tuple(out.shape) != (Cc, R):
            raise ValueError(f"out must be bfloat16 of shape {(Cc, R)}")
    ldd = _rowmajor(out, "out")
    _check(lib().transpose_bf16(_ptr(src), R, Cc, lds, _ptr(out), ldd, _stream(src.device)), "transpose_bf16")
    return out


def spmm24_xt(c: Compressed24, XT, out_dtype=None, out=None, bias=None, act="none"):
    """Y = act(W X + bias) for compressed W with X supplied transposed: XT bf16 [N, K]."""
    ldxt = _x_bf16(XT, "XT")
    if XT.shape[1] != c.K:
        raise ValueError(f"XT has {XT.shape[1]} columns, W has K = {c.K}")
    N = XT.shape[0]
    _operands_on(XT.device, (c.values, "values"), (c.meta, "meta"))
    out, ldy = _out_tensor(out, c.M, N, out_dtype, XT.device)
    bptr, act_code, fused = _fused_args(bias, act, c.M, XT.device)
    if fused:
        _check(lib().spmm24_fused(_ptr(c.values), _ptr(c.meta), c.layout, c.M, c.K, _ptr(XT), ldxt, P24_X_NK, N,
                                  _ptr(out), _out_code(out.dtype), ldy, bptr, act_code, _stream(XT.device)),
               "spmm24_fused")
        return out
    _check(lib().spmm24_xt(_ptr(c.values), _ptr(c.meta), c.layout, c.M, c.K, _ptr(XT), ldxt, N, _ptr(out),
                           _out_code(out.dtype), ldy, _stream(XT.device)), "spmm24_xt")
    return out


def gemm_bf16_xt(Wp, M: int, K: int, XT, out_dtype=None, out=None):
    """Dense baseline with X supplied transposed: XT bf16 [N, K]."""
    ldxt = _x_bf16(XT, "XT")
    if XT.shape[1] != K:
        raise ValueError(f"XT has {XT.shape[1]} columns, W has K = {K}")
    N = XT.shape[0]
    _packed_w(Wp, M, K, XT.device)
    out, ldy = _out_tensor(out, M, N, out_dtype, XT.device)
    _check(lib().gemm_bf16_xt(_ptr(Wp), M, K, _ptr(XT), ldxt, N, _ptr(out), _out_code(out.dtype), ldy,
                              _stream(XT.device)), "gemm_bf16_xt")
    return out
