"""Host-side checks of the C ABI (no GPU needed, no device work is launched).

Every call here either is a pure host helper or fails argument validation,
which the library performs before it touches the HIP runtime.
"""
import ctypes
import math
import os
import re
import subprocess
import sys

import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4lin.h")

qll = pytest.importorskip("quantized_linear_layer_amd")
from quantized_linear_layer_amd import _lib  # noqa: E402

if not os.path.exists(_lib.LIB_PATH):
    pytest.skip("libfp4lin.so not built (run __graft_entry__.build())", allow_module_level=True)

L = _lib.load()
P = ctypes.c_void_p
FAKE = P(0x10000)        # 16-byte aligned, never dereferenced (validation fails first)
MISALIGNED = P(0x10004)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4lin_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (fp4lin_\w+)", out))
    assert set(names) <= exported
    assert set(names) == set(_lib.SIGNATURES)


@pytest.mark.parametrize("n", [1, 2, 7, 100, 131072, 33554432, 84 * 2 ** 20 + 3])
@pytest.mark.parametrize("q", [0.0, 1e-9, 0.25, 0.5, 0.9, 0.99, 0.999, 0.9999999, 1.0])
def test_quantile_rank_matches_oracle(n, q):
    assert L.fp4lin_quantile_rank(n, q) == O.quantile_rank(n, q)


def test_quantile_rank_invalid():
    for n, q in [(0, 0.5), (-1, 0.5), (10, -0.01), (10, 1.01), (10, math.nan), (10, math.inf)]:
        assert L.fp4lin_quantile_rank(n, q) == -1


@pytest.mark.parametrize("K", [1, 2, 127, 128, 129, 512, 4095, 4096, 5120, 13824, 15360])
def test_packed_ld_matches_oracle(K):
    assert L.fp4lin_packed_ld(K) == O.packed_ld(K)
    assert L.fp4lin_packed_ld(K) % 64 == 0


def test_packed_ld_invalid():
    assert L.fp4lin_packed_ld(0) == -1


def test_workspace_layout_consistent():
    for (M, K, N, dt, q) in [(256, 512, 512, 0, 0.99), (8192, 4096, 11008, 1, 0.99),
                             (3, 5, 7, 1, 1.0), (16384, 5120, 15360, 1, 0.99)]:
        o = _lib.ForwardOffsets()
        assert L.fp4lin_forward_layout(M, K, N, dt, q, ctypes.byref(o)) == 0
        k = O.quantile_rank(M * K, q)
        assert o.capacity == M * K - 1 - k
        ldq = O.packed_ld(K)
        regions = sorted([
            (o.tau, 4), (o.coo_row, 4 * max(o.capacity, 1)), (o.coo_col, 4 * max(o.capacity, 1)),
            (o.coo_val, 4 * max(o.capacity, 1)), (o.row_ptr, 4 * (M + 1)), (o.Aq, M * ldq),
            (o.sA, 4 * M), (o.Wq, N * ldq), (o.sW, 4 * N),
            # the select's workspace and W's column maxima are live together
            (o.scratch, L.fp4lin_select_workspace_bytes(M, K, dt)
             + L.fp4lin_weight_workspace_bytes(K, N))])
        for (a, na), (b, _) in zip(regions, regions[1:]):
            assert a + na <= b                       # no overlap
        for off, _ in regions:
            assert off % 256 == 0                    # every region 256-byte aligned
        assert regions[-1][0] + regions[-1][1] <= o.total
        assert L.fp4lin_workspace_bytes(M, K, N, dt, q) == o.total
    assert L.fp4lin_workspace_bytes(0, 5, 7, 1, 0.5) == 0
    assert L.fp4lin_workspace_bytes(3, 5, 7, 9, 0.5) == 0
    assert L.fp4lin_workspace_bytes(3, 5, 7, 1, 2.0) == 0
    # M*K >= 2^32 is refused (32-bit histogram counts) even when the COO is small
    o = _lib.ForwardOffsets()
    assert L.fp4lin_forward_layout(2 ** 20, 2 ** 12, 8, 1, 1.0, ctypes.byref(o)) == _lib.ERR_SHAPE
    assert L.fp4lin_forward_layout(2 ** 20 - 1, 2 ** 12, 8, 1, 1.0, ctypes.byref(o)) == 0


def test_status_strings():
    for s in range(9):
        assert len(L.fp4lin_status_str(s)) > 0
    assert L.fp4lin_status_str(99) == b"unknown status"


# ---- validation errors (nothing is launched) ---------------------------------------
def coo(cap, null=None):
    f = {k: FAKE.value for k in ("row", "col", "val", "row_ptr")}
    if null:
        f[null] = None
    return _lib.Coo(f["row"], f["col"], f["val"], f["row_ptr"], cap)


def select(A=FAKE, dt=1, M=4, K=8, lda=8, q=0.5, tau=FAKE, dA=None, ws=FAKE, wsb=1 << 20):
    dA = coo(100) if dA is None else dA
    return L.fp4lin_outlier_select(A, dt, M, K, lda, q, tau, dA, ws, wsb, None)


def test_select_errors():
    assert select(A=None) == _lib.ERR_NULL
    assert select(tau=None) == _lib.ERR_NULL
    for fld in ("row", "col", "val", "row_ptr"):
        assert select(dA=coo(100, null=fld)) == _lib.ERR_NULL
    assert select(ws=None) == _lib.ERR_NULL
    assert select(dt=5) == _lib.ERR_DTYPE
    assert select(M=0) == _lib.ERR_SHAPE
    assert select(K=-1) == _lib.ERR_SHAPE
    assert select(lda=7) == _lib.ERR_SHAPE
    assert select(M=2 ** 31) == _lib.ERR_SHAPE
    # M*K >= 2^32 overflows the 32-bit histogram counts, even with a small COO
    assert select(M=2 ** 20, K=2 ** 12, lda=2 ** 12, q=1.0) == _lib.ERR_SHAPE
    assert select(q=-0.5) == _lib.ERR_QUANTILE
    assert select(q=float("nan")) == _lib.ERR_QUANTILE
    # n = 32, q = 0.5 -> k = 15, capacity needed 16
    assert select(dA=coo(15)) == _lib.ERR_CAPACITY
    assert select(ws=MISALIGNED) == _lib.ERR_ALIGN
    assert select(wsb=16) == _lib.ERR_WORKSPACE


def select_noalloc(A=FAKE, dt=1, M=4, K=8, lda=8, q=0.5, tau=FAKE, dA=None):
    dA = coo(100) if dA is None else dA
    return L.fp4lin_outlier_select_noalloc(A, dt, M, K, lda, q, tau, dA, None)


def test_select_noalloc_errors():
    """The allocation-free select checks its arguments like the workspace one,
    then refuses inputs whose scratch exceeds its 8 MiB static array, before it
    looks up the device or enqueues anything."""
    assert select_noalloc(A=None) == _lib.ERR_NULL
    assert select_noalloc(tau=None) == _lib.ERR_NULL
    assert select_noalloc(dA=coo(100, null="row_ptr")) == _lib.ERR_NULL
    assert select_noalloc(dt=5) == _lib.ERR_DTYPE
    assert select_noalloc(M=0) == _lib.ERR_SHAPE
    assert select_noalloc(q=1.5) == _lib.ERR_QUANTILE
    assert select_noalloc(dA=coo(15)) == _lib.ERR_CAPACITY
    scratch = 8 << 20
    for dt, rows in ((1, 1_865_152), (0, 2_088_896)):
        assert L.fp4lin_select_workspace_bytes(rows, 16, dt) == scratch
        assert L.fp4lin_select_workspace_bytes(rows + 1, 16, dt) > scratch
        assert select_noalloc(dt=dt, M=rows + 1, K=16, lda=16, dA=coo((rows + 1) * 16)) == \
            _lib.ERR_SCRATCH
    assert "static scratch" in L.fp4lin_status_str(_lib.ERR_SCRATCH).decode()


def quant_act(X=FAKE, dt=1, M=4, K=8, ldx=8, tau=None, Xq=FAKE, sX=FAKE):
    return L.fp4lin_quantize_act(X, dt, M, K, ldx, tau, Xq, sX, None)


def test_quantize_act_errors():
    assert quant_act(X=None) == _lib.ERR_NULL
    assert quant_act(Xq=None) == _lib.ERR_NULL
    assert quant_act(sX=None) == _lib.ERR_NULL
    assert quant_act(dt=2) == _lib.ERR_DTYPE
    assert quant_act(M=0) == _lib.ERR_SHAPE
    assert quant_act(ldx=7) == _lib.ERR_SHAPE
    assert quant_act(Xq=MISALIGNED) == _lib.ERR_ALIGN


def quant_w(W=FAKE, dt=1, K=8, N=4, ldw=4, Wq=FAKE, sW=FAKE, ws=FAKE, wsb=1 << 20):
    return L.fp4lin_quantize_weight(W, dt, K, N, ldw, Wq, sW, ws, wsb, None)


def test_quantize_weight_errors():
    assert quant_w(W=None) == _lib.ERR_NULL
    assert quant_w(ws=None) == _lib.ERR_NULL
    assert quant_w(dt=-1) == _lib.ERR_DTYPE
    assert quant_w(N=0) == _lib.ERR_SHAPE
    assert quant_w(ldw=3) == _lib.ERR_SHAPE
    assert quant_w(Wq=MISALIGNED) == _lib.ERR_ALIGN
    assert quant_w(ws=MISALIGNED) == _lib.ERR_ALIGN
    assert quant_w(wsb=4) == _lib.ERR_WORKSPACE
    # K up to 65535 tiles of 128 codes (the micro-scaled quantizer's grid
    # dimension, the same limit for both formats)
    assert quant_w(K=65535 * 128 + 1, N=1, ldw=1) == _lib.ERR_SHAPE
    # the column passes' one-dimensional grids hold fewer than 2^32 workgroups
    assert quant_w(K=1 << 22, N=1 << 30, ldw=1 << 30) == _lib.ERR_SHAPE


def gemm(Aq=FAKE, sA=FAKE, Bq=FAKE, sB=FAKE, M=4, N=4, K=8, dA=None, W=None, wdt=1, ldw=4,
         Y=FAKE, ldy=4):
    p = ctypes.byref(dA) if dA is not None else None
    return L.fp4lin_gemm(Aq, sA, Bq, sB, M, N, K, p, W, wdt, ldw, Y, ldy, None)


def test_gemm_errors():
    assert gemm(Aq=None) == _lib.ERR_NULL
    assert gemm(sB=None) == _lib.ERR_NULL
    assert gemm(Y=None) == _lib.ERR_NULL
    assert gemm(dA=coo(10), W=None) == _lib.ERR_NULL
    for fld in ("col", "val", "row_ptr"):
        assert gemm(dA=coo(10, null=fld), W=FAKE) == _lib.ERR_NULL
    assert gemm(dA=coo(10), W=FAKE, wdt=3) == _lib.ERR_DTYPE
    assert gemm(dA=coo(10), W=FAKE, ldw=3) == _lib.ERR_SHAPE
    assert gemm(dA=coo(10), W=FAKE, K=2 ** 20, ldw=2 ** 11) == _lib.ERR_SHAPE
    assert gemm(K=0) == _lib.ERR_SHAPE
    assert gemm(ldy=3) == _lib.ERR_SHAPE
    assert gemm(Aq=MISALIGNED) == _lib.ERR_ALIGN
    assert gemm(Bq=MISALIGNED) == _lib.ERR_ALIGN


def sparse_add(dA=None, W=FAKE, wdt=1, K=8, ldw=4, M=4, N=4, Y=FAKE, ldy=4):
    dA = coo(10) if dA is None else dA
    return L.fp4lin_sparse_add(ctypes.byref(dA), W, wdt, K, ldw, M, N, Y, ldy, None)


def test_sparse_add_errors():
    assert L.fp4lin_sparse_add(None, FAKE, 1, 8, 4, 4, 4, FAKE, 4, None) == _lib.ERR_NULL
    for fld in ("col", "val", "row_ptr"):
        assert sparse_add(dA=coo(10, null=fld)) == _lib.ERR_NULL
    assert sparse_add(W=None) == _lib.ERR_NULL
    assert sparse_add(Y=None) == _lib.ERR_NULL
    assert sparse_add(wdt=7) == _lib.ERR_DTYPE
    assert sparse_add(M=0) == _lib.ERR_SHAPE
    assert sparse_add(ldw=3) == _lib.ERR_SHAPE
    assert sparse_add(ldy=3) == _lib.ERR_SHAPE
    assert sparse_add(K=0) == _lib.ERR_SHAPE
    assert sparse_add(K=2 ** 20, ldw=2 ** 11) == _lib.ERR_SHAPE   # W beyond 2 GiB


def test_mx_scales_ld():
    for K in (1, 32, 127, 128, 129, 4096, 5120, 13824):
        assert L.fp4lin_mx_scales_ld(K) == O.packed_ld(K) // 16
    assert L.fp4lin_mx_scales_ld(0) == -1


def test_quantize_mx_errors():
    def act(X=FAKE, dt=1, M=4, K=8, ldx=8, Xq=FAKE, Xs=FAKE):
        return L.fp4lin_quantize_act_mx(X, dt, M, K, ldx, None, Xq, Xs, None)

    def wt(W=FAKE, dt=1, K=8, N=4, ldw=4, Wq=FAKE, Ws=FAKE):
        return L.fp4lin_quantize_weight_mx(W, dt, K, N, ldw, Wq, Ws, None)

    assert act(X=None) == _lib.ERR_NULL
    assert act(Xs=None) == _lib.ERR_NULL
    assert act(dt=7) == _lib.ERR_DTYPE
    assert act(M=0) == _lib.ERR_SHAPE
    assert act(ldx=7) == _lib.ERR_SHAPE
    assert act(Xq=MISALIGNED) == _lib.ERR_ALIGN
    assert act(Xs=MISALIGNED) == _lib.ERR_ALIGN
    assert wt(Ws=None) == _lib.ERR_NULL
    assert wt(dt=3) == _lib.ERR_DTYPE
    assert wt(N=0) == _lib.ERR_SHAPE
    assert wt(ldw=3) == _lib.ERR_SHAPE
    assert wt(K=65535 * 128 + 1, N=1, ldw=1) == _lib.ERR_SHAPE   # grid y above 65535
    assert wt(Wq=MISALIGNED) == _lib.ERR_ALIGN
    assert wt(Ws=MISALIGNED) == _lib.ERR_ALIGN


def test_gemm_mx_errors():
    def g(Aq=FAKE, As=FAKE, Bq=FAKE, Bs=FAKE, M=4, N=4, K=8, dA=None, W=None, wdt=1, ldw=4,
          Y=FAKE, ldy=4):
        p = ctypes.byref(dA) if dA is not None else None
        return L.fp4lin_gemm_mx(Aq, As, Bq, Bs, M, N, K, p, W, wdt, ldw, Y, ldy, None)

    assert g(As=None) == _lib.ERR_NULL
    assert g(Bs=None) == _lib.ERR_NULL
    assert g(M=0) == _lib.ERR_SHAPE
    assert g(ldy=3) == _lib.ERR_SHAPE
    assert g(M=2 ** 26, K=2 ** 6) == _lib.ERR_SHAPE   # (M+1)*packed_ld(K) >= 2^31
    assert g(As=MISALIGNED) == _lib.ERR_ALIGN
    assert g(Bs=MISALIGNED) == _lib.ERR_ALIGN
    c = _lib.Coo(FAKE, FAKE, FAKE, FAKE, 10)
    assert g(dA=c, W=None) == _lib.ERR_NULL
    assert g(dA=c, W=FAKE, wdt=5) == _lib.ERR_DTYPE
    assert g(dA=c, W=FAKE, ldw=3) == _lib.ERR_SHAPE


def test_workspace_layout_mx():
    """The micro-scaled forward's layout: scale regions of rows * mx_scales_ld(K)
    bytes, no overlap, 256-byte alignment, and no column-maxima scratch."""
    for (M, K, N, dt, q) in [(256, 512, 512, 0, 0.99), (8192, 4096, 11008, 1, 0.99),
                             (3, 5, 7, 1, 1.0)]:
        o = _lib.ForwardOffsets()
        assert L.fp4lin_forward_layout_mx(M, K, N, dt, q, ctypes.byref(o)) == 0
        nb = L.fp4lin_mx_scales_ld(K)
        ldq = O.packed_ld(K)
        regions = sorted([
            (o.tau, 4), (o.coo_row, 4 * max(o.capacity, 1)), (o.coo_col, 4 * max(o.capacity, 1)),
            (o.coo_val, 4 * max(o.capacity, 1)), (o.row_ptr, 4 * (M + 1)), (o.Aq, M * ldq),
            (o.sA, M * nb), (o.Wq, N * ldq), (o.sW, N * nb),
            (o.scratch, L.fp4lin_select_workspace_bytes(M, K, dt))])
        for (a, na), (b, _) in zip(regions, regions[1:]):
            assert a + na <= b
        for off, _ in regions:
            assert off % 256 == 0
        assert regions[-1][0] + regions[-1][1] <= o.total
        assert L.fp4lin_workspace_bytes_mx(M, K, N, dt, q) == o.total
    assert L.fp4lin_workspace_bytes_mx(0, 5, 7, 1, 0.5) == 0


def test_forward_mx_errors():
    def f(A=FAKE, W=FAKE, dt=1, M=4, K=8, N=4, lda=8, ldw=4, q=0.5, Y=FAKE, ldy=4, ws=FAKE,
          wsb=1 << 30):
        return L.fp4lin_forward_mx(A, W, dt, M, K, N, lda, ldw, q, Y, ldy, ws, wsb, None)
    assert f(A=None) == _lib.ERR_NULL
    assert f(ws=None) == _lib.ERR_NULL
    assert f(dt=4) == _lib.ERR_DTYPE
    assert f(N=0) == _lib.ERR_SHAPE
    assert f(lda=2) == _lib.ERR_SHAPE
    assert f(q=1.5) == _lib.ERR_QUANTILE
    assert f(ws=MISALIGNED) == _lib.ERR_ALIGN
    need = L.fp4lin_workspace_bytes_mx(4, 8, 4, 1, 0.5)
    assert f(wsb=need - 1) == _lib.ERR_WORKSPACE
    assert f(M=2 ** 20 - 1, K=2 ** 12, lda=2 ** 12, q=1.0, wsb=1 << 40) == _lib.ERR_SHAPE


def forward(A=FAKE, W=FAKE, dt=1, M=4, K=8, N=4, lda=8, ldw=4, q=0.5, Y=FAKE, ldy=4, ws=FAKE,
            wsb=1 << 30):
    return L.fp4lin_forward(A, W, dt, M, K, N, lda, ldw, q, Y, ldy, ws, wsb, None)


def test_forward_errors():
    assert forward(A=None) == _lib.ERR_NULL
    assert forward(W=None) == _lib.ERR_NULL
    assert forward(ws=None) == _lib.ERR_NULL
    assert forward(dt=4) == _lib.ERR_DTYPE
    assert forward(N=0) == _lib.ERR_SHAPE
    assert forward(lda=2) == _lib.ERR_SHAPE
    assert forward(ldy=1) == _lib.ERR_SHAPE
    assert forward(q=1.5) == _lib.ERR_QUANTILE
    assert forward(ws=MISALIGNED) == _lib.ERR_ALIGN
    need = L.fp4lin_workspace_bytes(4, 8, 4, 1, 0.5)
    assert forward(wsb=need - 1) == _lib.ERR_WORKSPACE
    # the GEMM's limits are checked before anything is enqueued (no device here:
    # a launch would fail with a launch error instead)
    assert forward(M=2 ** 20 - 1, K=2 ** 12, lda=2 ** 12, q=1.0, wsb=1 << 40) == _lib.ERR_SHAPE
    assert forward(M=1, K=2 ** 20, lda=2 ** 20, N=8, ldw=2 ** 11, ldy=8, q=1.0,
                   wsb=1 << 40) == _lib.ERR_SHAPE          # W beyond 2 GiB


def test_python_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    A = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qll.quantize_act(A)


def test_one_hip_runtime_in_process():
    """The library binds to the HIP runtime PyTorch loaded, so the process holds
    one runtime (two copies of it do not share a device context)."""
    pytest.importorskip("torch")
    maps = open("/proc/self/maps").read()
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hip) == 1, sorted(hip)


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU: --gpus 2 exits with status 2 and says so,
    before touching any device."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
