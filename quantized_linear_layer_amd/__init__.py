"""fp4lin: FP4 (E2M1) quantized linear layer forward on AMD MI355X (gfx950).

Python binding of libfp4lin.so. The functions named ``fp4lin_*`` mirror the C
ABI one to one: they take torch tensors that already live on the GPU, pass
their device pointers, sizes and the current HIP stream, and raise
``Fp4linError`` on a non-zero status. The helpers without the prefix only add
output allocation on top of them. All arithmetic runs in the HIP kernels; there
is no CPU path.
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import BF16, F32, Coo, ForwardOffsets

__all__ = [
    "Fp4linError", "lib", "packed_ld", "quantile_rank", "select_workspace_bytes",
    "weight_workspace_bytes", "workspace_bytes", "forward_layout",
    "fp4lin_outlier_select", "fp4lin_outlier_select_noalloc", "fp4lin_quantize_act", "fp4lin_quantize_weight", "fp4lin_gemm",
    "fp4lin_sparse_add", "fp4lin_forward", "outlier_select", "quantize_act", "quantize_weight", "gemm", "forward",
    "CooBuffers", "mx_scales_ld", "fp4lin_quantize_act_mx", "fp4lin_quantize_weight_mx",
    "fp4lin_gemm_mx", "quantize_act_mx", "quantize_weight_mx", "gemm_mx",
    "fp4lin_forward_mx", "forward_mx", "forward_layout_mx",
]


class Fp4linError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().fp4lin_status_str(status).decode()
        if status == _lib.ERR_LAUNCH:
            msg += f": {lib().fp4lin_last_hip_error_name().decode()}"
        super().__init__(f"{where}: status {status} ({msg})")
        self.status = status


def lib():
    return _lib.load()


def _check(status: int, where: str):
    if status != _lib.OK:
        raise Fp4linError(status, where)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"fp4lin takes float32 or bfloat16 inputs, got {t.dtype}")


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (fp4lin has no CPU path)")
    return ctypes.c_void_p(t.data_ptr())


def _matrix(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D row-major tensor with unit column stride")
    return t.shape[0], t.shape[1], t.stride(0)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ---- host helpers --------------------------------------------------------------
def packed_ld(L: int) -> int:
    return int(lib().fp4lin_packed_ld(L))


def quantile_rank(n: int, q: float) -> int:
    return int(lib().fp4lin_quantile_rank(n, q))


def select_workspace_bytes(M: int, K: int, dtype_code: int) -> int:
    return int(lib().fp4lin_select_workspace_bytes(M, K, dtype_code))


def weight_workspace_bytes(K: int, N: int) -> int:
    return int(lib().fp4lin_weight_workspace_bytes(K, N))


def workspace_bytes(M: int, K: int, N: int, dtype_code: int, q: float) -> int:
    return int(lib().fp4lin_workspace_bytes(M, K, N, dtype_code, q))


def forward_layout(M: int, K: int, N: int, dtype_code: int, q: float) -> ForwardOffsets:
    o = ForwardOffsets()
    _check(lib().fp4lin_forward_layout(M, K, N, dtype_code, q, ctypes.byref(o)),
           "fp4lin_forward_layout")
    return o


class CooBuffers:
    """Device arrays of a COO dA (int32 row/col, float32 val, int32 row_ptr)."""

    def __init__(self, row, col, val, row_ptr):
        self.row, self.col, self.val, self.row_ptr = row, col, val, row_ptr

    @property
    def capacity(self) -> int:
        return int(self.row.numel())

    def struct(self) -> Coo:
        return Coo(self.row.data_ptr(), self.col.data_ptr(), self.val.data_ptr(),
                   self.row_ptr.data_ptr(), self.capacity)

    @classmethod
    def empty(cls, M: int, capacity: int, device):
        torch = _torch()
        cap = max(int(capacity), 1)
        return cls(torch.empty(cap, dtype=torch.int32, device=device),
                   torch.empty(cap, dtype=torch.int32, device=device),
                   torch.empty(cap, dtype=torch.float32, device=device),
                   torch.empty(M + 1, dtype=torch.int32, device=device))


# ---- the C ABI, one to one -------------------------------------------------------
def fp4lin_outlier_select(A, q, tau, coo: CooBuffers, ws, stream=None):
    M, K, lda = _matrix(A, "A")
    _dev(tau, "tau"), _dev(ws, "ws"), _dev(coo.row, "coo")
    _check(lib().fp4lin_outlier_select(_dev(A, "A"), _dtype_code(A), M, K, lda, float(q),
                                       _dev(tau, "tau"), coo.struct(), _dev(ws, "ws"),
                                       ws.numel() * ws.element_size(), _stream(stream)),
           "fp4lin_outlier_select")


def fp4lin_outlier_select_noalloc(A, q, tau, coo: CooBuffers, stream=None):
    M, K, lda = _matrix(A, "A")
    _dev(coo.row, "coo")
    _check(lib().fp4lin_outlier_select_noalloc(_dev(A, "A"), _dtype_code(A), M, K, lda,
                                               float(q), _dev(tau, "tau"), coo.struct(),
                                               _stream(stream)),
           "fp4lin_outlier_select_noalloc")


def fp4lin_quantize_act(X, tau, Xq, sX, stream=None):
    M, K, ldx = _matrix(X, "X")
    _check(lib().fp4lin_quantize_act(_dev(X, "X"), _dtype_code(X), M, K, ldx, _dev(tau, "tau"),
                                     _dev(Xq, "Xq"), _dev(sX, "sX"), _stream(stream)),
           "fp4lin_quantize_act")


def fp4lin_quantize_weight(W, Wq, sW, ws, stream=None):
    K, N, ldw = _matrix(W, "W")
    _check(lib().fp4lin_quantize_weight(_dev(W, "W"), _dtype_code(W), K, N, ldw, _dev(Wq, "Wq"),
                                        _dev(sW, "sW"), _dev(ws, "ws"),
                                        ws.numel() * ws.element_size(), _stream(stream)),
           "fp4lin_quantize_weight")


def fp4lin_gemm(Aq, sA, Bq, sB, M, N, K, coo: CooBuffers | None, W, Y, stream=None):
    _, _, ldy = _matrix(Y, "Y")
    if coo is not None:
        _, _, ldw = _matrix(W, "W")
        c = coo.struct()
        cp, wp, wdt = ctypes.byref(c), _dev(W, "W"), _dtype_code(W)
    else:
        cp, wp, wdt, ldw = None, None, F32, 0
    _check(lib().fp4lin_gemm(_dev(Aq, "Aq"), _dev(sA, "sA"), _dev(Bq, "Bq"), _dev(sB, "sB"),
                             M, N, K, cp, wp, wdt, ldw, _dev(Y, "Y"), ldy, _stream(stream)),
           "fp4lin_gemm")


def fp4lin_sparse_add(coo: CooBuffers, W, Y, stream=None):
    """Y += dA . W (Y must already hold the scaled FP4 product)."""
    M, N, ldy = _matrix(Y, "Y")
    K, _, ldw = _matrix(W, "W")
    c = coo.struct()
    _check(lib().fp4lin_sparse_add(ctypes.byref(c), _dev(W, "W"), _dtype_code(W), K, ldw, M, N,
                                   _dev(Y, "Y"), ldy, _stream(stream)),
           "fp4lin_sparse_add")


def fp4lin_forward(A, W, q, Y, ws, stream=None):
    M, K, lda = _matrix(A, "A")
    K2, N, ldw = _matrix(W, "W")
    if K2 != K:
        raise ValueError(f"A is {M}x{K} but W is {K2}x{N}")
    if A.dtype != W.dtype:
        raise TypeError("A and W must have the same dtype")
    _, _, ldy = _matrix(Y, "Y")
    _check(lib().fp4lin_forward(_dev(A, "A"), _dev(W, "W"), _dtype_code(A), M, K, N, lda, ldw,
                                float(q), _dev(Y, "Y"), ldy, _dev(ws, "ws"),
                                ws.numel() * ws.element_size(), _stream(stream)),
           "fp4lin_forward")


def fp4lin_quantize_act_mx(X, tau, Xq, Xs, stream=None):
    M, K, ldx = _matrix(X, "X")
    _check(lib().fp4lin_quantize_act_mx(_dev(X, "X"), _dtype_code(X), M, K, ldx,
                                        _dev(tau, "tau"), _dev(Xq, "Xq"), _dev(Xs, "Xs"),
                                        _stream(stream)),
           "fp4lin_quantize_act_mx")


def fp4lin_quantize_weight_mx(W, Wq, Ws, stream=None):
    K, N, ldw = _matrix(W, "W")
    _check(lib().fp4lin_quantize_weight_mx(_dev(W, "W"), _dtype_code(W), K, N, ldw,
                                           _dev(Wq, "Wq"), _dev(Ws, "Ws"), _stream(stream)),
           "fp4lin_quantize_weight_mx")


def fp4lin_gemm_mx(Aq, As, Bq, Bs, M, N, K, coo: CooBuffers | None, W, Y, stream=None):
    _, _, ldy = _matrix(Y, "Y")
    if coo is not None:
        _, _, ldw = _matrix(W, "W")
        c = coo.struct()
        cp, wp, wdt = ctypes.byref(c), _dev(W, "W"), _dtype_code(W)
    else:
        cp, wp, wdt, ldw = None, None, F32, 0
    _check(lib().fp4lin_gemm_mx(_dev(Aq, "Aq"), _dev(As, "As"), _dev(Bq, "Bq"), _dev(Bs, "Bs"),
                                M, N, K, cp, wp, wdt, ldw, _dev(Y, "Y"), ldy, _stream(stream)),
           "fp4lin_gemm_mx")


def fp4lin_forward_mx(A, W, q, Y, ws, stream=None):
    M, K, lda = _matrix(A, "A")
    K2, N, ldw = _matrix(W, "W")
    if K2 != K:
        raise ValueError(f"A is {M}x{K} but W is {K2}x{N}")
    if A.dtype != W.dtype:
        raise TypeError("A and W must have the same dtype")
    _, _, ldy = _matrix(Y, "Y")
    _check(lib().fp4lin_forward_mx(_dev(A, "A"), _dev(W, "W"), _dtype_code(A), M, K, N, lda, ldw,
                                   float(q), _dev(Y, "Y"), ldy, _dev(ws, "ws"),
                                   ws.numel() * ws.element_size(), _stream(stream)),
           "fp4lin_forward_mx")


# ---- allocating helpers --------------------------------------------------------------
def _empty(shape, dtype, device):
    return _torch().empty(shape, dtype=dtype, device=device)


def outlier_select(A, q, stream=None):
    """Returns (tau[1] float32, CooBuffers)."""
    torch = _torch()
    M, K, _ = _matrix(A, "A")
    k = quantile_rank(M * K, q)
    if k < 0:
        raise Fp4linError(_lib.ERR_QUANTILE, "outlier_select")
    cap = M * K - 1 - k
    tau = _empty((1,), torch.float32, A.device)
    coo = CooBuffers.empty(M, cap, A.device)
    ws = _empty((max(select_workspace_bytes(M, K, _dtype_code(A)), 16),), torch.uint8, A.device)
    fp4lin_outlier_select(A, q, tau, coo, ws, stream)
    return tau, coo


def quantize_act(X, tau=None, stream=None):
    """Returns (Xq uint8 M x packed_ld(K), sX float32 M)."""
    torch = _torch()
    M, K, _ = _matrix(X, "X")
    Xq = _empty((M, packed_ld(K)), torch.uint8, X.device)
    sX = _empty((M,), torch.float32, X.device)
    fp4lin_quantize_act(X, tau, Xq, sX, stream)
    return Xq, sX


def quantize_weight(W, stream=None):
    """Returns (Wq uint8 N x packed_ld(K), sW float32 N)."""
    torch = _torch()
    K, N, _ = _matrix(W, "W")
    Wq = _empty((N, packed_ld(K)), torch.uint8, W.device)
    sW = _empty((N,), torch.float32, W.device)
    ws = _empty((max(weight_workspace_bytes(K, N), 16),), torch.uint8, W.device)
    fp4lin_quantize_weight(W, Wq, sW, ws, stream)
    return Wq, sW


def gemm(Aq, sA, Bq, sB, M, N, K, coo=None, W=None, stream=None):
    """Returns Y float32 M x N."""
    Y = _empty((M, N), _torch().float32, Aq.device)
    fp4lin_gemm(Aq, sA, Bq, sB, M, N, K, coo, W, Y, stream)
    return Y


def forward(A, W, q, stream=None, return_workspace=False):
    """Returns Y float32 M x N (and the workspace holding the intermediates)."""
    torch = _torch()
    M, K, _ = _matrix(A, "A")
    N = W.shape[1]
    nbytes = workspace_bytes(M, K, N, _dtype_code(A), q)
    if nbytes == 0:
        raise Fp4linError(_lib.ERR_SHAPE, "forward")
    ws = _empty((nbytes,), torch.uint8, A.device)
    Y = _empty((M, N), torch.float32, A.device)
    fp4lin_forward(A, W, q, Y, ws, stream)
    return (Y, ws) if return_workspace else Y


def mx_scales_ld(L: int) -> int:
    return lib().fp4lin_mx_scales_ld(L)


def quantize_act_mx(X, tau=None, stream=None):
    """Micro-scaled: returns (Xq uint8 M x packed_ld(K), Xs uint8 (steps, M, 4)),
    the scales step-major: Xs[s, i, j] is the byte of block 4s + j of row i."""
    torch = _torch()
    M, K, _ = _matrix(X, "X")
    Xq = _empty((M, packed_ld(K)), torch.uint8, X.device)
    Xs = _empty((mx_scales_ld(K) // 4, M, 4), torch.uint8, X.device)
    fp4lin_quantize_act_mx(X, tau, Xq, Xs, stream)
    return Xq, Xs


def quantize_weight_mx(W, stream=None):
    """Micro-scaled: returns (Wq uint8 N x packed_ld(K), Ws uint8 (steps, N, 4)),
    the scales step-major as for quantize_act_mx, per column of W."""
    torch = _torch()
    K, N, _ = _matrix(W, "W")
    Wq = _empty((N, packed_ld(K)), torch.uint8, W.device)
    Ws = _empty((mx_scales_ld(K) // 4, N, 4), torch.uint8, W.device)
    fp4lin_quantize_weight_mx(W, Wq, Ws, stream)
    return Wq, Ws


def gemm_mx(Aq, As, Bq, Bs, M, N, K, coo=None, W=None, stream=None):
    """Micro-scaled GEMM; returns Y float32 M x N."""
    Y = _empty((M, N), _torch().float32, Aq.device)
    fp4lin_gemm_mx(Aq, As, Bq, Bs, M, N, K, coo, W, Y, stream)
    return Y


def forward_layout_mx(M: int, K: int, N: int, dtype_code: int, q: float) -> ForwardOffsets:
    o = ForwardOffsets()
    _check(lib().fp4lin_forward_layout_mx(M, K, N, dtype_code, float(q), ctypes.byref(o)),
           "fp4lin_forward_layout_mx")
    return o


def forward_mx(A, W, q, stream=None, return_workspace=False):
    """Micro-scaled forward; returns Y float32 M x N (and the workspace)."""
    torch = _torch()
    M, K, _ = _matrix(A, "A")
    N = W.shape[1]
    nbytes = lib().fp4lin_workspace_bytes_mx(M, K, N, _dtype_code(A), float(q))
    if nbytes == 0:
        raise Fp4linError(_lib.ERR_SHAPE, "forward_mx")
    ws = _empty((nbytes,), torch.uint8, A.device)
    Y = _empty((M, N), torch.float32, A.device)
    fp4lin_forward_mx(A, W, q, Y, ws, stream)
    return (Y, ws) if return_workspace else Y
