"""GPU parity of the micro-scaled (MXFP4) variant against the CPU oracle:
32-code blocks along K with one E8M0 scale each (the micro-scaling lecture
"FP4量化训练的硬件挑战：NVIDIA Blackwell架构上的微缩放格式（Micro-scaling）实现",
section 3; the per-block E8M0 scales of "训练大型语言模型的挑战").

Bit-exact: codes and scale bytes of both quantizers; the GEMM on inputs whose
every partial sum is exact in fp32. Otherwise Y is held to the fp32
accumulation bound |Y - Y64| <= (2 * blocks + 2) * 2^-24 * sum |block terms|
(plus the compensation tolerance of the token-wise path) elementwise.
"""
import numpy as np
import pytest

import oracle as O
import workloads as wl
from gpu_util import assert_bits_equal, host, log, padded, to_device

pytestmark = pytest.mark.gpu

Y_TOL = 1e-5


@pytest.fixture(scope="module")
def ql():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_linear_layer_amd as q
    q.lib()
    return q


def torch():
    import torch as t
    return t


def upload(a):
    return torch().from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def scales_to_rows(dev_scales, rows):
    """The library's step-major scale bytes (steps, rows, 4) as rows x blocks."""
    a = np.asarray(dev_scales).reshape(-1, rows, 4)
    return np.ascontiguousarray(a.transpose(1, 0, 2).reshape(rows, -1))


def scales_to_steps(row_bytes):
    """Rows x blocks scale bytes in the library's step-major layout."""
    a = np.asarray(row_bytes, np.uint8)
    R, nb = a.shape
    return np.ascontiguousarray(a.reshape(R, nb // 4, 4).transpose(1, 0, 2))


def tau_tensor(tau):
    t = torch()
    return None if tau is None else t.tensor([float(tau)], dtype=t.float32, device="cuda:0")


# ---------------------------------------------------------------------------
# quantizers
# ---------------------------------------------------------------------------
def check_act_mx(ql, X: wl.Matrix, tau=None, ld=None):
    Xd = to_device(X)
    if ld is not None:
        Xd = padded(Xd, ld)
    Xq, Xs = ql.quantize_act_mx(Xd, tau_tensor(tau))
    torch().cuda.synchronize()
    want_q, want_s, _, _ = O.quantize_act_mx(X.f32, tau)
    assert_bits_equal(scales_to_rows(host(Xs), X.shape[0]), want_s, "scale bytes")
    assert_bits_equal(host(Xq), want_q, "packed codes")


def check_weight_mx(ql, W: wl.Matrix, ld=None):
    Wd = to_device(W)
    if ld is not None:
        Wd = padded(Wd, ld)
    Wq, Ws = ql.quantize_weight_mx(Wd)
    torch().cuda.synchronize()
    want_q, want_s, _, _ = O.quantize_weight_mx(W.f32)
    assert_bits_equal(scales_to_rows(host(Ws), W.shape[1]), want_s, "scale bytes")
    assert_bits_equal(host(Wq), want_q, "packed codes")


def wide_range_matrix(rng, R, C, dtype):
    """t(3) values with a power-of-two spread of 2^-40 .. 2^40 per 16 columns, so
    neighbouring blocks have very different exponents."""
    x = rng.standard_t(3, (R, C)) * np.exp2(rng.integers(-40, 40, (R, (C + 15) // 16))).repeat(16, axis=1)[:, :C]
    return wl.from_f32(x.astype(np.float32), dtype)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("M,K", [(1, 1), (3, 7), (5, 31), (4, 32), (6, 33), (9, 129), (37, 1000),
                                 (70, 2051), (3, 16392)])
def test_quantize_act_mx_shapes(ql, dtype, M, K):
    log(f"quantize_act_mx {dtype} {M}x{K}")
    rng = np.random.default_rng(M * 1000 + K)
    X = wide_range_matrix(rng, M, K, dtype)
    check_act_mx(ql, X)
    tau, _ = O.select_threshold(X.f32, 0.9)
    check_act_mx(ql, X, tau)


def test_quantize_act_mx_every_bf16_value(ql):
    """Every finite bfloat16 value (each row a different block mix)."""
    check_act_mx(ql, wl.all_bf16_values_matrix(256))


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_quantize_act_mx_special_blocks(ql, dtype):
    """Zero, negative-zero, subnormal, block max exactly 6*2^e and its float
    neighbours, and the largest finite values."""
    K = 256
    rows = []
    f32 = np.float32
    rows.append(np.zeros(K, f32))
    rows.append(np.full(K, -0.0, f32))
    sub = np.float32(np.finfo(np.float32).tiny) * np.linspace(0, 1, K).astype(f32)
    rows.append(sub)
    for e in (-126, -3, 0, 7, 100):
        edge = np.full(K, f32(6.0 * 2.0 ** e))
        edge[1::3] = np.nextafter(edge[1::3], f32(np.inf))
        edge[2::3] = np.nextafter(edge[2::3], f32(0))
        edge[::5] *= f32(-0.37)
        rows.append(edge.astype(f32))
    big = np.full(K, f32(3.0e38), f32)       # finite in bfloat16 too
    big[::2] *= f32(-0.5)
    rows.append(big)
    X = wl.from_f32(np.stack(rows), dtype)
    check_act_mx(ql, X)
    check_act_mx(ql, X, tau=np.float32(1.0))


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_quantize_act_mx_leading_dimension(ql, dtype):
    rng = np.random.default_rng(9)
    X = wide_range_matrix(rng, 33, 250, dtype)
    check_act_mx(ql, X, ld=264)   # aligned, padded
    check_act_mx(ql, X, ld=251)   # unaligned rows -> element loads


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("K,N", [(1, 1), (1, 1000), (33, 1), (129, 7), (300, 70), (512, 520),
                                 (1000, 77), (4101, 136)])
def test_quantize_weight_mx_shapes(ql, dtype, K, N):
    log(f"quantize_weight_mx {dtype} {K}x{N}")
    rng = np.random.default_rng(K * 7 + N)
    check_weight_mx(ql, wide_range_matrix(rng, K, N, dtype))


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_quantize_weight_mx_leading_dimension(ql, dtype):
    rng = np.random.default_rng(3)
    W = wide_range_matrix(rng, 300, 100, dtype)
    check_weight_mx(ql, W, ld=104)   # aligned, padded
    check_weight_mx(ql, W, ld=101)   # unaligned rows


# ---------------------------------------------------------------------------
# GEMM with block scales
# ---------------------------------------------------------------------------
def run_gemm_mx(ql, codesA, eA, codesB, eB, K, delta=None, W=None, capacity=None):
    """capacity: length of the COO arrays (at least nnz); at most 10 per row of
    A runs the compensation in the GEMM's epilogue, more as a second kernel."""
    M, N = codesA.shape[0], codesB.shape[0]
    coo, Wd = None, None
    if delta is not None:
        nz = max(delta.nnz, 1, capacity or 0)
        pad = lambda a, dt: np.concatenate([np.asarray(a, dt), np.zeros(nz - len(a), dt)])
        coo = ql.CooBuffers(upload(pad(delta.row, np.int32)), upload(pad(delta.col, np.int32)),
                            upload(pad(delta.val32, np.float32)),
                            upload(np.asarray(delta.row_ptr, np.int32)))
        Wd = to_device(W)
    Y = ql.gemm_mx(upload(O.pack_rows(codesA)), upload(scales_to_steps(O.mx_scale_bytes(eA))),
                   upload(O.pack_rows(codesB)), upload(scales_to_steps(O.mx_scale_bytes(eB))),
                   M, N, K, coo, Wd)
    torch().cuda.synchronize()
    return host(Y).astype(np.float64)


def nblocks(K):
    return O.packed_ld(K) // 16


# K steps of 128 codes: every count below three and every residue modulo the
# three LDS stages, with ragged M and N tiles.
MNK = [(1, 1, 1), (37, 300, 700), (256, 256, 256), (130, 270, 512), (64, 300, 384),
       (96, 260, 1664), (513, 257, 4096)]


@pytest.mark.parametrize("M,N,K", MNK)
def test_gemm_mx_unit_scales_integer_exact(ql, M, N, K):
    """Every scale byte 127 (2^0): the exact integer product."""
    log(f"gemm_mx unit {M}x{N}x{K}")
    rng = np.random.default_rng(M + N + K)
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    cb = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    Y = run_gemm_mx(ql, ca, np.zeros((M, nblocks(K)), int), cb, np.zeros((N, nblocks(K)), int), K)
    assert np.array_equal(Y, O.integer_product(ca, cb))


@pytest.mark.parametrize("M,N,K", MNK)
def test_gemm_mx_block_scales_exact(ql, M, N, K):
    """Exponents in {-1, 0, 1} per (row, block) and (column, block): every
    block term is a multiple of 2^-4 below 2^13 and every partial sum fits in
    24 bits, so the fp32 result is exact whatever the order, and any block or
    lane mix-up of the scales shows."""
    log(f"gemm_mx exact {M}x{N}x{K}")
    rng = np.random.default_rng(M * 3 + N * 5 + K)
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    cb = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    ea = rng.integers(-1, 2, size=(M, nblocks(K)))
    eb = rng.integers(-1, 2, size=(N, nblocks(K)))
    Y = run_gemm_mx(ql, ca, ea, cb, eb, K)
    want, _ = O.mx_product(ca, ea, cb, eb)
    assert np.array_equal(Y, want)


def test_gemm_mx_one_block_per_pair(ql):
    """A row and a column share exactly one non-zero block, with distinct
    exponents per block: Y[i,j] is that block's product times 2^(eA+eB)."""
    M, N, K = 64, 64, 1024
    nb = nblocks(K)
    rng = np.random.default_rng(4)
    ba = rng.integers(0, nb, M)
    bb = rng.integers(0, nb, N)
    bb[:32] = ba[:32]
    ca = np.zeros((M, K), np.uint8)
    cb = np.zeros((N, K), np.uint8)
    for i in range(M):
        ca[i, ba[i] * 32:(ba[i] + 1) * 32] = rng.integers(0, 16, 32)
    for j in range(N):
        cb[j, bb[j] * 32:(bb[j] + 1) * 32] = rng.integers(0, 16, 32)
    ea = rng.integers(-30, 30, (M, nb))
    eb = rng.integers(-30, 30, (N, nb))
    Y = run_gemm_mx(ql, ca, ea, cb, eb, K)
    want, _ = O.mx_product(ca, ea, cb, eb)
    assert np.array_equal(Y, want)   # one block term per element: exact


def assert_within_accumulation_bound(Y, want, mag, K, extra=0.0):
    bound = (2 * nblocks(K) + 2) * 2.0 ** -24 * mag + extra
    bad = np.abs(Y - want) > bound
    assert not bad.any(), f"{bad.sum()} elements beyond the fp32 accumulation bound"


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("M,K,N", [(100, 300, 200), (300, 700, 520)])
def test_gemm_mx_quantized_operands(ql, dtype, M, K, N):
    """Operands from the oracle's quantizers, without and with the compensation."""
    log(f"gemm_mx quantized {dtype} {M}x{K}x{N}")
    rng = np.random.default_rng(M * K + N)
    A = wl.random_matrix(rng, M, K, dtype, dist="t3")
    W = wl.random_matrix(rng, K, N, dtype, scale=0.02)
    want, mag, tau, delta, qa, qw = O.forward_mx(A.f32, W.f32, 0.97)
    Y0 = run_gemm_mx(ql, qa[2], qa[3], qw[2], qw[3], K)
    want0, mag0 = O.mx_product(qa[2], qa[3], qw[2], qw[3])
    assert_within_accumulation_bound(Y0, want0, mag0, K)
    Y = run_gemm_mx(ql, qa[2], qa[3], qw[2], qw[3], K, delta, W)
    assert O.rel_fro(Y, want) <= Y_TOL
    # both schedules of the compensation give the same bits
    fused = run_gemm_mx(ql, qa[2], qa[3], qw[2], qw[3], K, delta, W, capacity=delta.nnz)
    separate = run_gemm_mx(ql, qa[2], qa[3], qw[2], qw[3], K, delta, W,
                           capacity=max(delta.nnz, 10 * M + 1))
    assert np.array_equal(fused.view(np.uint64), separate.view(np.uint64))


# ---------------------------------------------------------------------------
# the whole micro-scaled layer through the C ABI: select, quantize_act_mx,
# quantize_weight_mx, gemm_mx with the compensation
# ---------------------------------------------------------------------------
def run_layer_mx(ql, A, W, q):
    Ad, Wd = to_device(A), to_device(W)
    M, K = A.shape
    N = W.shape[1]
    tau, coo = ql.outlier_select(Ad, q)
    Aq, As = ql.quantize_act_mx(Ad, tau)
    Wq, Ws = ql.quantize_weight_mx(Wd)
    Y = ql.gemm_mx(Aq, As, Wq, Ws, M, N, K, coo, Wd)
    torch().cuda.synchronize()
    return Y, Aq, As, Wq, Ws, tau


@pytest.mark.parametrize("name", ["tiny", "llama1.3b_ffn_up"])
def test_layer_mx_workloads(ql, name):
    L = wl.make_layer(name, M=None if name == "tiny" else 512)
    log(f"layer_mx {name} {L.M}x{L.K}x{L.N}")
    Y, Aq, As, Wq, Ws, tau = run_layer_mx(ql, L.A, L.W, L.q)
    want, mag, otau, delta, qa, qw = O.forward_mx(L.A.f32, L.W.f32, L.q)
    assert_bits_equal(host(tau)[0], otau, "tau")
    assert_bits_equal(host(Aq), qa[0], "A codes")
    assert_bits_equal(scales_to_rows(host(As), L.M), qa[1], "A scale bytes")
    assert_bits_equal(host(Wq), qw[0], "W codes")
    assert_bits_equal(scales_to_rows(host(Ws), L.N), qw[1], "W scale bytes")
    assert O.rel_fro(host(Y), want) <= Y_TOL


# ---------------------------------------------------------------------------
# the backward GEMMs on micro-scaled operands, through the public calls:
# dgrad blocks along N (quantize_act_mx on dY and on W), wgrad blocks along M
# (quantize_weight_mx on A and on dY, then gemm_mx with K' = M)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (70, 33, 129), (300, 100, 520)])
def test_dgrad_mx_public_calls(ql, dtype, M, K, N):
    log(f"dgrad_mx {dtype} {M}x{K}x{N}")
    rng = np.random.default_rng(M + 7 * K + 11 * N)
    dY = wl.random_matrix(rng, M, N, dtype, scale=1e-3)
    W = wl.random_matrix(rng, K, N, dtype, scale=0.02)
    dq, ds = ql.quantize_act_mx(to_device(dY))
    wq, wsc = ql.quantize_act_mx(to_device(W))
    dX = ql.gemm_mx(dq, ds, wq, wsc, M, K, N)
    torch().cuda.synchronize()
    want, mag, qd, qw = O.dgrad_mx(dY.f32, W.f32)
    assert_bits_equal(host(dq), qd[0], "dY codes")
    assert_bits_equal(scales_to_rows(host(ds), M), qd[1], "dY scale bytes")
    assert_bits_equal(host(wq), qw[0], "W codes")
    assert_bits_equal(scales_to_rows(host(wsc), K), qw[1], "W scale bytes")
    assert_within_accumulation_bound(host(dX).astype(np.float64), want, mag, N)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (129, 33, 70), (1000, 100, 300)])
def test_wgrad_mx_public_calls(ql, dtype, M, K, N):
    log(f"wgrad_mx {dtype} {M}x{K}x{N}")
    rng = np.random.default_rng(M + 3 * K + 5 * N)
    A = wl.random_matrix(rng, M, K, dtype, dist="t3")
    dY = wl.random_matrix(rng, M, N, dtype, scale=1e-3)
    aq, asc = ql.quantize_weight_mx(to_device(A))
    dq, ds = ql.quantize_weight_mx(to_device(dY))
    dW = ql.gemm_mx(aq, asc, dq, ds, K, N, M)
    torch().cuda.synchronize()
    want, mag, qa, qd = O.wgrad_mx(A.f32, dY.f32)
    assert_bits_equal(host(aq), qa[0], "A codes")
    assert_bits_equal(scales_to_rows(host(asc), K), qa[1], "A scale bytes")
    assert_bits_equal(host(dq), qd[0], "dY codes")
    assert_bits_equal(scales_to_rows(host(ds), N), qd[1], "dY scale bytes")
    assert_within_accumulation_bound(host(dW).astype(np.float64), want, mag, M)


# ---------------------------------------------------------------------------
# fp4lin_forward_mx: the whole micro-scaled layer in one call
# ---------------------------------------------------------------------------
def forward_mx_views(ql, ws, M, K, N, dt, q):
    o = ql.forward_layout_mx(M, K, N, dt, q)
    nb = ql.mx_scales_ld(K)
    ldq = ql.packed_ld(K)
    b = ws
    tau = b[o.tau:o.tau + 4].view(torch().float32)
    rp = b[o.row_ptr:o.row_ptr + 4 * (M + 1)].view(torch().int32)
    Aq = b[o.Aq:o.Aq + M * ldq].view(M, ldq)
    As = b[o.sA:o.sA + M * nb]
    Wq = b[o.Wq:o.Wq + N * ldq].view(N, ldq)
    Ws = b[o.sW:o.sW + N * nb]
    return o, tau, rp, Aq, As, Wq, Ws


# ld: None (dense rows), "pad" (aligned rows, lda != K), "odd" (A and W rows
# not 16-byte aligned). The K cover every slab pattern of the row kernels.
FWD_MX_CASES = [(dt, ld, M, K, N)
                for (M, K, N) in [(37, 1000, 300), (300, 4096, 520), (70, 8192, 129),
                                  (33, 8200, 64), (24, 13824, 72), (20, 3584, 40)]
                for (dt, ld) in [(wl.BF16, None), (wl.BF16, "pad"), (wl.BF16, "odd"),
                                 (wl.F32, None)]]


@pytest.mark.parametrize("dtype,ld,M,K,N", FWD_MX_CASES)
def test_forward_mx_matches_stage_calls(ql, dtype, ld, M, K, N):
    """Every intermediate and Y of fp4lin_forward_mx are bit-identical to the
    separate calls (the forward's compaction block-quantizes A, and W's pass
    shares the row count's launch), and Y matches the oracle."""
    log(f"forward_mx {dtype} ld={ld} {M}x{K}x{N}")
    t = torch()
    rng = np.random.default_rng(M + K + N)
    A = wl.random_matrix(rng, M, K, dtype, dist="t3")
    W = wl.random_matrix(rng, K, N, dtype, scale=0.02)
    Ad, Wd = to_device(A), to_device(W)
    if ld == "pad":
        Ad = padded(Ad, (K + 7) // 8 * 8 + 8)
    elif ld == "odd":
        Ad, Wd = padded(Ad, K + 1), padded(Wd, N + 1)
    q = 0.98
    Y, ws = ql.forward_mx(Ad, Wd, q, return_workspace=True)
    tau, coo = ql.outlier_select(Ad, q)
    Aq, As = ql.quantize_act_mx(Ad, tau)
    Wq, Ws = ql.quantize_weight_mx(Wd)
    Y2 = ql.gemm_mx(Aq, As, Wq, Ws, M, N, K, coo, Wd)
    t.cuda.synchronize()
    dt = ql.BF16 if dtype == wl.BF16 else ql.F32
    o, ftau, rp, fAq, fAs, fWq, fWs = forward_mx_views(ql, ws, M, K, N, dt, q)
    assert_bits_equal(host(ftau), host(tau), "tau")
    assert_bits_equal(host(rp), host(coo.row_ptr), "row_ptr")
    assert_bits_equal(host(fAq), host(Aq), "A codes")
    assert_bits_equal(host(fAs), host(As).reshape(-1), "A scale bytes")
    assert_bits_equal(host(fWq), host(Wq), "W codes")
    assert_bits_equal(host(fWs), host(Ws).reshape(-1), "W scale bytes")
    assert_bits_equal(host(Y), host(Y2), "Y")
    want, _, _, _, _, _ = O.forward_mx(A.f32, W.f32, q)
    assert O.rel_fro(host(Y), want) <= Y_TOL
