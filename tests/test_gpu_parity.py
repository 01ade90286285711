"""GPU parity: every C-ABI entry point against the CPU oracle on seeded inputs,
small enough for the oracle to finish in seconds but spanning several tiles
and ragged tails, plus adversarial matrices (every bfloat16 value, exact
midpoints, zero / negative-zero / subnormal rows, ties at the threshold,
padded and unaligned leading dimensions).

Bit-exact: codes, scales, tau, COO (row, col, val, row_ptr).
Y: relative Frobenius error <= 1e-5 (fp32 accumulation order and the
float32 rounding of the compensation values; the exact integer GEMM core is
checked bit-exactly with unit scales).
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


# ---------------------------------------------------------------------------
# input builders
# ---------------------------------------------------------------------------
def midpoint_rows(dtype, rows=64, K=200, seed=0):
    """Rows whose amax is 6*2^e (inv exact) and whose entries sit on E2M1
    midpoints, grid points and their float neighbours."""
    rng = np.random.default_rng(seed)
    base = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1, 1.5, 2, 3, 4, 6, 0.0],
                    dtype=np.float32)
    vals = rng.choice(base, size=(rows, K)).astype(np.float32)
    if dtype == wl.F32:
        nudge = rng.integers(-1, 2, size=(rows, K))
        up = np.nextafter(vals, np.float32(10))
        dn = np.nextafter(vals, np.float32(0))
        vals = np.where(nudge > 0, up, np.where(nudge < 0, dn, vals)).astype(np.float32)
    vals[:, 0] = 6.0
    vals = np.minimum(vals, np.float32(6.0))
    signs = rng.choice([-1.0, 1.0], size=(rows, K)).astype(np.float32)
    scale = (2.0 ** rng.integers(-20, 20, size=(rows, 1))).astype(np.float32)
    return wl.from_f32(vals * signs * scale, dtype)


def all_bf16_scaled_rows():
    """Every non-negative bf16 value <= 6 (and its negative) in rows of amax 6:
    inv = 1, so y equals the value itself."""
    b = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    v = wl.bf16_bits_to_f32(b)
    v = v[v <= 6.0]
    allv = np.concatenate([v, -v])
    K = 256
    R = int(np.ceil(allv.size / (K - 1)))
    out = np.zeros((R, K), dtype=np.float32)
    flat = np.zeros(R * (K - 1), dtype=np.float32)
    flat[: allv.size] = allv
    out[:, 1:] = flat.reshape(R, K - 1)
    out[:, 0] = 6.0
    return wl.from_f32(out, wl.BF16)


def special_rows(dtype):
    """Zero, negative-zero, subnormal and single-value rows."""
    K = 300
    rows = [np.zeros(K, np.float32), np.full(K, -0.0, np.float32)]
    sub = np.zeros(K, np.float32)
    if dtype == wl.F32:
        sub[::3] = np.float32(1e-45)
        sub[1::7] = np.float32(-3e-42)
        sub[5] = np.float32(1e-39)
    else:
        sub[::3] = wl.bf16_bits_to_f32(np.array([1], np.uint16))[0]       # smallest subnormal
        sub[1::7] = -wl.bf16_bits_to_f32(np.array([0x50], np.uint16))[0]
    rows.append(sub)
    one = np.zeros(K, np.float32)
    one[123] = -7.0
    rows.append(one)
    mixed = np.linspace(-3, 3, K).astype(np.float32)
    mixed[::2] = -0.0
    rows.append(mixed)
    return wl.from_f32(np.stack(rows), dtype)


# ---------------------------------------------------------------------------
# quantize_act (token-wise)
# ---------------------------------------------------------------------------
def check_quantize_act(ql, X: wl.Matrix, tau=None, ld=None):
    t = torch()
    Xd = to_device(X)
    if ld is not None:
        Xd = padded(Xd, ld)
    taud = None if tau is None else t.tensor([float(tau)], dtype=t.float32, device="cuda:0")
    Xq, sX = ql.quantize_act(Xd, taud)
    t.cuda.synchronize()
    want_q, want_s, _ = O.quantize_act(X.f32, tau)
    assert_bits_equal(host(sX), want_s, "scales")
    assert_bits_equal(host(Xq), want_q, "packed codes")


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("M,K", [(1, 1), (3, 7), (5, 127), (4, 128), (9, 129), (37, 1000),
                                 (70, 2051),
                                 # past 8192 columns: aligned bf16 rows stay in registers
                                 # up to 16384 (32 chunks per lane), others take two reads
                                 (6, 8200), (5, 13824), (3, 16384), (4, 16392), (3, 9001)])
def test_quantize_act_shapes(ql, dtype, M, K):
    log(f"quantize_act {dtype} {M}x{K}")
    rng = np.random.default_rng(M * 1000 + K)
    X = wl.random_matrix(rng, M, K, dtype, dist="t3")
    check_quantize_act(ql, X)
    tau, _ = O.select_threshold(X.f32, 0.9)
    check_quantize_act(ql, X, tau)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_quantize_act_midpoints(ql, dtype):
    check_quantize_act(ql, midpoint_rows(dtype))


def test_quantize_act_every_bf16_value(ql):
    check_quantize_act(ql, all_bf16_scaled_rows())
    check_quantize_act(ql, wl.all_bf16_values_matrix(256))


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_quantize_act_special_rows(ql, dtype):
    X = special_rows(dtype)
    check_quantize_act(ql, X)
    check_quantize_act(ql, X, tau=np.float32(0.0))
    check_quantize_act(ql, X, tau=np.float32(1.0))


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_quantize_act_leading_dimension(ql, dtype):
    rng = np.random.default_rng(9)
    X = wl.random_matrix(rng, 33, 250, dtype)
    check_quantize_act(ql, X, ld=264)   # aligned, padded
    check_quantize_act(ql, X, ld=251)   # unaligned rows -> element loads


def test_quantize_act_tiny_workload(ql):
    L = wl.make_layer("tiny")
    tau, _ = O.select_threshold(L.A.f32, L.q)
    check_quantize_act(ql, L.A, tau)


# ---------------------------------------------------------------------------
# quantize_weight (channel-wise, packed N-major)
# ---------------------------------------------------------------------------
def check_quantize_weight(ql, W: wl.Matrix, ld=None):
    t = torch()
    Wd = to_device(W)
    if ld is not None:
        Wd = padded(Wd, ld)
    Wq, sW = ql.quantize_weight(Wd)
    t.cuda.synchronize()
    want_q, want_s, _ = O.quantize_weight(W.f32)
    assert_bits_equal(host(sW), want_s, "scales")
    assert_bits_equal(host(Wq), want_q, "packed codes")


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("K,N", [(1, 1), (1, 1000), (129, 1), (300, 70), (512, 520),
                                 (1000, 77)])
def test_quantize_weight_shapes(ql, dtype, K, N):
    log(f"quantize_weight {dtype} {K}x{N}")
    rng = np.random.default_rng(K * 7 + N)
    check_quantize_weight(ql, wl.random_matrix(rng, K, N, dtype, scale=0.02))


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_quantize_weight_adversarial(ql, dtype):
    X = midpoint_rows(dtype, rows=40, K=300)
    check_quantize_weight(ql, wl.from_f32(X.f32.T.copy(), dtype))
    S = special_rows(dtype)
    check_quantize_weight(ql, wl.from_f32(S.f32.T.copy(), dtype))


def test_quantize_weight_every_bf16_value(ql):
    X = all_bf16_scaled_rows()
    check_quantize_weight(ql, wl.from_f32(X.f32.T.copy(), wl.BF16))
    # 128 and 136 columns: every 8-column group of the column kernels full
    check_quantize_weight(ql, wl.from_f32(X.f32[:128].T.copy(), wl.BF16))
    pad = np.zeros((136, X.f32.shape[1]), np.float32)
    pad[:X.f32.shape[0]] = X.f32[:136]
    check_quantize_weight(ql, wl.from_f32(pad.T.copy(), wl.BF16))


# N % 8 == 0 with aligned bfloat16 rows: whole 8-column groups, the last
# 128-column tile ragged.
@pytest.mark.parametrize("K,N", [(1, 8), (7, 16), (129, 64), (300, 136), (4101, 72),
                                 (2, 1032)])
def test_quantize_weight_bf16_full_groups(ql, K, N):
    log(f"quantize_weight bf16 {K}x{N}")
    rng = np.random.default_rng(K * 13 + N)
    check_quantize_weight(ql, wl.random_matrix(rng, K, N, wl.BF16, scale=0.02))


def test_quantize_weight_long_k(ql):
    """K above 65535 splits of 64 rows (the column-max pass's tiles along K):
    the column passes run on one-dimensional grids, so every split is
    launched; each column's largest magnitude sits in the last split."""
    K, N = 65535 * 64 + 100, 8
    log(f"quantize_weight bf16 {K}x{N}")
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    w[K - 1 - np.arange(N), np.arange(N)] = np.float32(0.75) * (1 + np.arange(N))
    check_quantize_weight(ql, wl.from_f32(w, wl.BF16))


def test_quantize_weight_bf16_special_columns(ql):
    """Zero, negative-zero, subnormal and one-value columns inside a tile that
    also holds ordinary columns (the tile then takes the generic encoder)."""
    S = special_rows(wl.BF16).f32.T            # 300 x 5
    rng = np.random.default_rng(11)
    R = wl.random_matrix(rng, S.shape[0], 11, wl.BF16, scale=0.02).f32
    check_quantize_weight(ql, wl.from_f32(np.concatenate([S, R], axis=1), wl.BF16))
    check_quantize_weight(ql, wl.from_f32(np.tile(S[:, 3:], (1, 4)), wl.BF16))


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_quantize_weight_leading_dimension(ql, dtype):
    rng = np.random.default_rng(5)
    W = wl.random_matrix(rng, 200, 90, dtype)
    check_quantize_weight(ql, W, ld=96)
    check_quantize_weight(ql, W, ld=91)


# ---------------------------------------------------------------------------
# outlier_select (tau + COO)
# ---------------------------------------------------------------------------
def run_select(ql, A: wl.Matrix, q, ld=None):
    t = torch()
    Ad = to_device(A)
    if ld is not None:
        Ad = padded(Ad, ld)
    tau, coo = ql.outlier_select(Ad, q)
    t.cuda.synchronize()
    return tau, coo


def check_select(ql, A: wl.Matrix, q, ld=None):
    tau, coo = run_select(ql, A, q, ld)
    want_tau, k = O.select_threshold(A.f32, q)
    _, d = O.clamp_and_residual(A.f32, want_tau)
    assert_bits_equal(host(tau)[0], want_tau, "tau")
    rp = host(coo.row_ptr)
    assert_bits_equal(rp, d.row_ptr.astype(np.int32), "row_ptr")
    nnz = int(rp[-1])
    assert nnz == d.nnz
    assert_bits_equal(host(coo.row)[:nnz], d.row, "coo row")
    assert_bits_equal(host(coo.col)[:nnz], d.col, "coo col")
    assert_bits_equal(host(coo.val)[:nnz], d.val32, "coo val")
    return tau, coo


@pytest.mark.parametrize("q", [0.0, 0.3, 0.9, 0.99, 0.999, 1.0])
def test_select_tiny_workload(ql, q):
    L = wl.make_layer("tiny")
    check_select(ql, L.A, q)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("M,K", [(1, 1), (1, 5), (3, 7), (100, 700), (257, 129),
                                 # 4097 rows: the last bfloat16 histogram workgroups get no rows
                                 (4097, 16),
                                 # over 8192 rows: 2 and 3 rows per wave, the last row group short
                                 (9000, 3), (16389, 24)])
def test_select_shapes(ql, dtype, M, K):
    log(f"select {dtype} {M}x{K}")
    rng = np.random.default_rng(M + K)
    A = wl.random_matrix(rng, M, K, dtype, dist="t3")
    for q in (0.5, 0.99):
        check_select(ql, A, q)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_select_many_ties(ql, dtype):
    """Values from a small set: many entries equal tau (strict clamp)."""
    rng = np.random.default_rng(1)
    vals = rng.choice(np.array([0.0, -0.0, 0.5, -1.0, 1.0, 2.0, -3.0, 3.0], np.float32),
                      size=(150, 333))
    A = wl.from_f32(vals, dtype)
    for q in (0.0, 0.2, 0.5, 0.8, 0.95, 1.0):
        check_select(ql, A, q)


def test_select_bf16_uneven_row_blocks(ql):
    """bfloat16 select where the first 16 rows (one histogram workgroup) are
    tiny apart from a few entries near the global 0.99 quantile: that
    workgroup's own quantile estimate lies far below the global one while it
    still holds keys in the global quantile's coarse bin, so the second pass
    over A is needed. Also the mirror case: a block of huge values."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((64, 1000)).astype(np.float32)
    x[:16] *= np.float32(1e-3)
    pos = rng.choice(16 * 1000, size=48, replace=False)
    x[:16].reshape(-1)[pos] = np.float32(2.6) * rng.choice([-1.0, 1.0], size=48).astype(np.float32)
    for q in (0.99, 0.995, 0.9):
        check_select(ql, wl.from_f32(x, wl.BF16), q)
    y = rng.standard_normal((64, 1000)).astype(np.float32)
    y[32:48] *= np.float32(1e4)
    for q in (0.5, 0.74, 0.75, 0.76, 0.99):
        check_select(ql, wl.from_f32(y, wl.BF16), q)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_select_dirty_workspace(ql, dtype):
    """No select kernel may rely on memory left by an earlier call or on a
    cleared workspace: a workspace and COO pre-filled with 0xFF bytes, reused
    for a second call of another shape, must give the oracle's bits."""
    t = torch()
    rng = np.random.default_rng(12)
    shapes = [(300, 700), (40, 1000)]
    big = max(ql.select_workspace_bytes(M, K, 0 if dtype == wl.F32 else 1) for M, K in shapes)
    ws = t.full((big,), 0xFF, dtype=t.uint8, device="cuda:0")
    for M, K in shapes:
        A = wl.random_matrix(rng, M, K, dtype, dist="t3")
        Ad = to_device(A)
        q = 0.99
        k = ql.quantile_rank(M * K, q)
        coo = ql.CooBuffers.empty(M, M * K - 1 - k, Ad.device)
        for buf in (coo.row, coo.col, coo.row_ptr):
            buf.fill_(-1)
        coo.val.fill_(float("nan"))
        tau = t.full((1,), float("nan"), dtype=t.float32, device=Ad.device)
        ql.fp4lin_outlier_select(Ad, q, tau, coo, ws)
        t.cuda.synchronize()
        want_tau, _ = O.select_threshold(A.f32, q)
        _, d = O.clamp_and_residual(A.f32, want_tau)
        assert_bits_equal(host(tau)[0], want_tau, "tau")
        assert_bits_equal(host(coo.row_ptr), d.row_ptr.astype(np.int32), "row_ptr")
        nnz = d.nnz
        assert_bits_equal(host(coo.col)[:nnz], d.col, "coo col")
        assert_bits_equal(host(coo.val)[:nnz], d.val32, "coo val")


def test_forward_dirty_workspace(ql):
    """fp4lin_forward with its workspace pre-filled with 0xFF bytes, then reused
    for a smaller layer, gives the same bits as with a fresh workspace."""
    t = torch()
    rng = np.random.default_rng(13)
    layers = []
    for M, K, N in [(200, 1024, 96), (70, 512, 40)]:
        a = wl.draw_activation(rng, M, K, "t3", max(1, K // 200), 50.0)
        w = wl.draw_weight(rng, K, N)
        layers.append(wl.Layer("dirty", wl.from_f32(a, wl.BF16), wl.from_f32(w, wl.BF16), 0.99))
    big = max(ql.workspace_bytes(L.M, L.K, L.N, 1, L.q) for L in layers)
    ws = t.full((big,), 0xFF, dtype=t.uint8, device="cuda:0")
    for L in layers:
        A, W = to_device(L.A), to_device(L.W)
        Y1 = ql.forward(A, W, L.q)
        Y2 = t.full((L.M, L.N), float("nan"), dtype=t.float32, device=A.device)
        ql.fp4lin_forward(A, W, L.q, Y2, ws)
        t.cuda.synchronize()
        assert np.array_equal(host(Y1).view(np.uint32), host(Y2).view(np.uint32))


def test_select_bf16_layer_slice(ql):
    L = wl.make_layer("llama7b_ffn_up", M=64)
    check_select(ql, L.A, L.q)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_select_leading_dimension(ql, dtype):
    rng = np.random.default_rng(2)
    A = wl.random_matrix(rng, 40, 300, dtype, dist="t3")
    check_select(ql, A, 0.95, ld=312)
    check_select(ql, A, 0.95, ld=301)


def test_select_deterministic(ql):
    L = wl.make_layer("llama1.3b_ffn_up", M=512)
    t1, c1 = run_select(ql, L.A, L.q)
    t2, c2 = run_select(ql, L.A, L.q)
    for a, b in ((t1, t2), (c1.row_ptr, c2.row_ptr)):
        assert np.array_equal(host(a), host(b))
    n = int(host(c1.row_ptr)[-1])
    for a, b in ((c1.row, c2.row), (c1.col, c2.col), (c1.val, c2.val)):
        assert np.array_equal(host(a)[:n], host(b)[:n])


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------
def upload_u8(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def upload_f32(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).to("cuda:0")


def upload_i32(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).to("cuda:0")


def run_gemm(ql, codesA, sA, codesB, sB, K, delta=None, W=None):
    M, N = codesA.shape[0], codesB.shape[0]
    Aq = upload_u8(O.pack_rows(codesA))
    Bq = upload_u8(O.pack_rows(codesB))
    coo = None
    Wd = None
    if delta is not None:
        nz = max(delta.nnz, 1)
        pad = lambda a, dt: np.concatenate([np.asarray(a, dt), np.zeros(nz - len(a), dt)])
        coo = ql.CooBuffers(upload_i32(pad(delta.row, np.int32)), upload_i32(pad(delta.col, np.int32)),
                            upload_f32(pad(delta.val32, np.float32)), upload_i32(delta.row_ptr))
        Wd = to_device(W)
    Y = ql.gemm(Aq, upload_f32(sA), Bq, upload_f32(sB), M, N, K, coo, Wd)
    torch().cuda.synchronize()
    return host(Y)


# K steps of 128 codes: 1, 6, 2, 8, 32, 2 and (added) 3, 4, 13, so that every
# count below three and every residue modulo the three LDS stages is covered.
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (37, 300, 700), (256, 256, 256), (300, 520, 1000),
                                   (513, 257, 4096), (64, 700, 129), (64, 300, 384),
                                   (130, 270, 512), (96, 260, 1664)])
def test_gemm_integer_exact(ql, M, N, K):
    """Unit scales, no compensation: Y is the exact integer-valued product."""
    log(f"gemm exact {M}x{N}x{K}")
    rng = np.random.default_rng(M + N + K)
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    cb = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    Y = run_gemm(ql, ca, np.ones(M, np.float32), cb, np.ones(N, np.float32), K)
    want = O.integer_product(ca, cb)
    assert np.array_equal(Y.astype(np.float64), want)


# The 256 x 256 tiles (grids of at least 512 of them) at 1, 2, 3, 5, 8 and 33
# K steps of 128 codes: every count below the three LDS stages and every
# residue modulo them, at a launch geometry the small shapes above do not reach.
@pytest.mark.parametrize("K", [128, 256, 384, 640, 1024, 4224])
def test_gemm_large_tiles_k_steps(ql, K):
    """Unit scales, 4096 x 8192 (512 large tiles): sampled rows (the first and
    last of every 256-row tile and 32 more) are the exact integer product over
    all 8192 columns."""
    M, N = 4096, 8192
    log(f"gemm large tiles {M}x{N}x{K}")
    rng = np.random.default_rng(K)
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    cb = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    t = torch()
    Y = ql.gemm(upload_u8(O.pack_rows(ca)), t.ones(M, dtype=t.float32, device="cuda:0"),
                upload_u8(O.pack_rows(cb)), t.ones(N, dtype=t.float32, device="cuda:0"), M, N, K)
    t.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, M, 256), np.arange(255, M, 256),
                                     rng.choice(M, 32, replace=False)]))
    sel = t.as_tensor(rows, device="cuda:0")
    want = O.integer_product(ca[rows], cb)
    assert np.array_equal(host(Y[sel]).astype(np.float64), want)
    del Y


def test_gemm_one_hot_layout(ql):
    """A[i,k] = 1 only at k = p[i]; B[j,k] = 1 only at k = r[j]: Y[i,j] = [p[i] == r[j]]."""
    M, N, K = 96, 80, 512
    rng = np.random.default_rng(0)
    p = rng.integers(0, K, size=M)
    r = rng.integers(0, K, size=N)
    r[:M // 2 if M // 2 < N else N] = p[:min(M // 2, N)]
    ca = np.zeros((M, K), np.uint8)
    cb = np.zeros((N, K), np.uint8)
    ca[np.arange(M), p] = 2   # value 1.0
    cb[np.arange(N), r] = 2
    Y = run_gemm(ql, ca, np.ones(M, np.float32), cb, np.ones(N, np.float32), K)
    want = (p[:, None] == r[None, :]).astype(np.float64)
    assert np.array_equal(Y.astype(np.float64), want)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("M,K,N", [(100, 300, 200), (300, 700, 520)])
def test_gemm_scaled_with_compensation(ql, dtype, M, K, N):
    log(f"gemm scaled {dtype} {M}x{K}x{N}")
    rng = np.random.default_rng(M * K + N)
    A = wl.random_matrix(rng, M, K, dtype, dist="t3")
    W = wl.random_matrix(rng, K, N, dtype, scale=0.02)
    ops = O.forward_operands(A.f32, W.f32, 0.97)
    Y = run_gemm(ql, ops.codesA, ops.sA, ops.codesW, ops.sW, K, ops.delta, W)
    want = O.forward_output(ops, W.f32)
    err = O.rel_fro(Y, want)
    assert err <= Y_TOL, err
    # without compensation: the scaled product alone, tighter (no sparse sum)
    Y0 = run_gemm(ql, ops.codesA, ops.sA, ops.codesW, ops.sW, K)
    want0 = O.scaled_product(O.integer_product(ops.codesA, ops.codesW), ops.sA, ops.sW)
    assert O.rel_fro(Y0, want0) <= 1e-7


# ---------------------------------------------------------------------------
# full forward
# ---------------------------------------------------------------------------
def workspace_views(ql, ws, M, K, N, dtype_code, q):
    o = ql.forward_layout(M, K, N, dtype_code, q)
    b = host(ws)
    ldq = ql.packed_ld(K)
    take = lambda off, n, dt: b[off: off + n * np.dtype(dt).itemsize].view(dt)
    rp = take(o.row_ptr, M + 1, np.int32)
    nnz = int(rp[-1])
    return dict(
        tau=take(o.tau, 1, np.float32)[0], row_ptr=rp, nnz=nnz,
        row=take(o.coo_row, nnz, np.int32), col=take(o.coo_col, nnz, np.int32),
        val=take(o.coo_val, nnz, np.float32),
        Aq=take(o.Aq, M * ldq, np.uint8).reshape(M, ldq), sA=take(o.sA, M, np.float32),
        Wq=take(o.Wq, N * ldq, np.uint8).reshape(N, ldq), sW=take(o.sW, N, np.float32))


def check_forward(ql, L: wl.Layer, rows=None, lda=None, ldw=None):
    t = torch()
    A, W = to_device(L.A), to_device(L.W)
    if lda is not None:
        A = padded(A, lda)
    if ldw is not None:
        W = padded(W, ldw)
    Y, ws = ql.forward(A, W, L.q, return_workspace=True)
    t.cuda.synchronize()
    ops = O.forward_operands(L.A.f32, L.W.f32, L.q)
    v = workspace_views(ql, ws, L.M, L.K, L.N, 0 if L.A.dtype == wl.F32 else 1, L.q)
    assert_bits_equal(v["tau"], ops.tau, "tau")
    assert_bits_equal(v["row_ptr"], ops.delta.row_ptr, "row_ptr")
    assert_bits_equal(v["row"], ops.delta.row, "coo row")
    assert_bits_equal(v["col"], ops.delta.col, "coo col")
    assert_bits_equal(v["val"], ops.delta.val32, "coo val")
    assert_bits_equal(v["sA"], ops.sA, "sA")
    assert_bits_equal(v["Aq"], ops.Aq, "Aq")
    assert_bits_equal(v["sW"], ops.sW, "sW")
    assert_bits_equal(v["Wq"], ops.Wq, "Wq")
    Yh = host(Y)
    if rows is None:
        want = O.forward_output(ops, L.W.f32)
        got = Yh
    else:
        want = O.forward_output(ops, L.W.f32, rows=rows)
        got = Yh[rows]
    err = O.rel_fro(got, want)
    log(f"forward {L.name} {L.M}x{L.K}x{L.N}: nnz {ops.delta.nnz} rel_fro {err:.3e}")
    assert err <= Y_TOL, err


def test_forward_tiny_workload(ql):
    check_forward(ql, wl.make_layer("tiny"))


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("M,K,N,q", [(1, 1, 1, 0.5), (7, 129, 3, 0.9), (300, 700, 520, 0.99),
                                     (513, 1000, 300, 0.999)])
def test_forward_small(ql, dtype, M, K, N, q):
    rng = np.random.default_rng(M + 3 * K + 7 * N)
    a = wl.draw_activation(rng, M, K, "t3", max(1, K // 200), 50.0)
    w = wl.draw_weight(rng, K, N)
    L = wl.Layer(f"small-{dtype}", wl.from_f32(a, dtype), wl.from_f32(w, dtype), q)
    check_forward(ql, L)


# Rows inside fp4lin_forward stream through in slabs of 8, 4, 2 and 1 chunks
# of 8 elements per lane (4096, 2048, 1024 and 512 columns), with a last
# 1-chunk slab over a ragged end; rows that are not 16-byte aligned (or
# K % 8 != 0) are read element by element, and so are W's rows when W is not
# 16-byte aligned.
@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("M,K,N,lda,ldw", [
    (24, 8192, 64, None, None),   # two 8-chunk slabs
    (20, 8200, 72, None, None),   # two 8-chunk slabs and a ragged end
    (12, 13824, 40, None, None),  # 3 x 8, then 2 and 1 chunks
    (16, 3584, 48, None, None),   # 4, 2 and 1 chunks
    (40, 300, 80, 301, None),     # rows not 16-byte aligned
    (40, 304, 80, 312, None),     # aligned rows with lda != K
    (30, 1000, 70, None, 73),     # W rows not 16-byte aligned
    (9, 1024, 24, None, None),    # fewer rows than one workgroup of each select kernel
    (5, 7, 9, None, None),        # a ragged end only
])
def test_forward_row_paths(ql, dtype, M, K, N, lda, ldw):
    log(f"forward row paths {dtype} {M}x{K}x{N} lda={lda} ldw={ldw}")
    rng = np.random.default_rng(M * 31 + K + N)
    a = wl.draw_activation(rng, M, K, "t3", max(1, K // 200), 50.0)
    w = wl.draw_weight(rng, K, N)
    L = wl.Layer("rows", wl.from_f32(a, dtype), wl.from_f32(w, dtype), 0.99)
    check_forward(ql, L, lda=lda, ldw=ldw)


def test_forward_q_one_is_plain_quantized_gemm(ql):
    """q = 1 clamps nothing; with grid-exact inputs Y = A W exactly."""
    rng = np.random.default_rng(3)
    M, K, N = 40, 260, 90
    mags = rng.integers(0, 8, size=(M, K)); mags[:, 0] = 7
    A = (np.array([0, .5, 1, 1.5, 2, 3, 4, 6])[mags] * rng.choice([-1, 1], size=(M, K))
         * 2.0 ** rng.integers(-4, 4, size=(M, 1))).astype(np.float32)
    mags = rng.integers(0, 8, size=(K, N)); mags[0, :] = 7
    W = (np.array([0, .5, 1, 1.5, 2, 3, 4, 6])[mags] * rng.choice([-1, 1], size=(K, N))
         * 2.0 ** rng.integers(-4, 4, size=(1, N))).astype(np.float32)
    t = torch()
    Y = ql.forward(t.from_numpy(A).cuda(), t.from_numpy(W).cuda(), 1.0)
    t.cuda.synchronize()
    assert np.array_equal(host(Y).astype(np.float64), A.astype(np.float64) @ W.astype(np.float64))


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_forward_streamed_rows(ql, dtype):
    """A of 210 MB, above the 192 MiB (A + W) at which the row kernels and the
    histogram passes read A with the non-temporal hint: the forward's tau,
    COO, codes and scales are bit-exact, Y matches on every 61st row, and the
    public select (the same rule on A alone) is bit-exact too. K = 6400 ends
    in a ragged slab in every row kernel."""
    M, K, N = (8192, 6400, 72) if dtype == wl.F32 else (16384, 6400, 72)
    log(f"streamed rows {dtype} {M}x{K}x{N}")
    rng = np.random.default_rng(6400)
    a = wl.draw_activation(rng, M, K, "t3", max(1, K // 200), 50.0)
    w = wl.draw_weight(rng, K, N)
    L = wl.Layer(f"streamed-{dtype}", wl.from_f32(a, dtype), wl.from_f32(w, dtype), 0.99)
    del a
    check_forward(ql, L, rows=np.arange(0, M, 61))
    check_select(ql, L.A, L.q)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_forward_streamed_y(ql, dtype):
    """Y of 210 MB with 25.6 COO entries per row: the compensation runs after
    the GEMM and reads Y with the non-temporal hint (Y + W above 192 MiB);
    Y matches on every 61st row and the operands are bit-exact."""
    M, K, N = 8192, 256, 6400
    log(f"streamed Y {dtype} {M}x{K}x{N}")
    rng = np.random.default_rng(6401)
    a = wl.draw_activation(rng, M, K, "t3", 2, 50.0)
    w = wl.draw_weight(rng, K, N)
    L = wl.Layer(f"streamed-y-{dtype}", wl.from_f32(a, dtype), wl.from_f32(w, dtype), 0.9)
    check_forward(ql, L, rows=np.arange(0, M, 61))


@pytest.mark.parametrize("case", ["llama1.3b", "k13824", "f32", "unaligned"])
def test_forward_matches_stage_calls(ql, case):
    """fp4lin_forward == the four public calls in order (same bits): the
    forward's count, compaction and quantization of A and its paired passes
    over W against the separate select and quantizer kernels."""
    log(f"forward vs stage calls {case}")
    t = torch()
    lda = ldw = None
    if case == "llama1.3b":
        L = wl.make_layer("llama1.3b_ffn_up", M=256)
    else:
        M, K, N, dtype = {"k13824": (48, 13824, 160, wl.BF16), "f32": (64, 5120, 136, wl.F32),
                          "unaligned": (40, 2000, 90, wl.BF16)}[case]
        rng = np.random.default_rng(K + N)
        a = wl.draw_activation(rng, M, K, "t3", max(1, K // 200), 50.0)
        w = wl.draw_weight(rng, K, N)
        L = wl.Layer(case, wl.from_f32(a, dtype), wl.from_f32(w, dtype), 0.999)
        if case == "unaligned":
            lda, ldw = K + 1, N + 3
    A, W = to_device(L.A), to_device(L.W)
    if lda is not None:
        A, W = padded(A, lda), padded(W, ldw)
    Y1, ws = ql.forward(A, W, L.q, return_workspace=True)
    tau, coo = ql.outlier_select(A, L.q)
    Aq, sA = ql.quantize_act(A, tau)
    Wq, sW = ql.quantize_weight(W)
    Y2 = ql.gemm(Aq, sA, Wq, sW, L.M, L.N, L.K, coo, W)
    t.cuda.synchronize()
    assert np.array_equal(host(Y1).view(np.uint32), host(Y2).view(np.uint32))
    v = workspace_views(ql, ws, L.M, L.K, L.N, 1 if L.A.dtype == wl.BF16 else 0, L.q)
    nnz = v["nnz"]
    assert_bits_equal(v["tau"], host(tau)[0], "tau")
    assert_bits_equal(v["row_ptr"], host(coo.row_ptr), "row_ptr")
    assert_bits_equal(v["row"], host(coo.row)[:nnz], "coo row")
    assert_bits_equal(v["col"], host(coo.col)[:nnz], "coo col")
    assert_bits_equal(v["val"], host(coo.val)[:nnz], "coo val")
    assert_bits_equal(v["Aq"], host(Aq), "Aq")
    assert_bits_equal(v["sA"], host(sA), "sA")
    assert_bits_equal(v["Wq"], host(Wq), "Wq")
    assert_bits_equal(v["sW"], host(sW), "sW")


# ---------------------------------------------------------------------------
# wgrad dW = Q(A)^T Q(dY) through the public calls (reading R10)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("M,K,N", [(1, 5, 3), (300, 70, 90), (129, 256, 40), (1000, 33, 520)])
def test_wgrad_public_calls(ql, dtype, M, K, N):
    log(f"wgrad {dtype} M={M} K={K} N={N}")
    t = torch()
    rng = np.random.default_rng(M + 5 * K + 11 * N)
    A = wl.random_matrix(rng, M, K, dtype, dist="t3")
    dY = wl.random_matrix(rng, M, N, dtype, scale=1e-3)
    Aq2, s_a2 = ql.quantize_weight(to_device(A))
    dYq2, s_dy2 = ql.quantize_weight(to_device(dY))
    dW = ql.gemm(Aq2, s_a2, dYq2, s_dy2, K, N, M)
    t.cuda.synchronize()
    want, (q_a2, want_sa2, _), (q_dy2, want_sdy2, _) = O.wgrad(A.f32, dY.f32)
    assert_bits_equal(host(s_a2), want_sa2, "s_A columns")
    assert_bits_equal(host(Aq2), q_a2, "Aq columns")
    assert_bits_equal(host(s_dy2), want_sdy2, "s_dY columns")
    assert_bits_equal(host(dYq2), q_dy2, "dYq columns")
    err = O.rel_fro(host(dW), want)
    assert err <= Y_TOL, err


def test_gemm_equals_gemm_then_sparse_add(ql):
    """fp4lin_gemm(dA) == fp4lin_gemm(NULL) followed by fp4lin_sparse_add (same bits)."""
    t = torch()
    L = wl.make_layer("llama1.3b_ffn_up", M=300)
    A, W = to_device(L.A), to_device(L.W)
    tau, coo = ql.outlier_select(A, L.q)
    Aq, sA = ql.quantize_act(A, tau)
    Wq, sW = ql.quantize_weight(W)
    Y1 = ql.gemm(Aq, sA, Wq, sW, L.M, L.N, L.K, coo, W)
    Y2 = ql.gemm(Aq, sA, Wq, sW, L.M, L.N, L.K)
    ql.fp4lin_sparse_add(coo, W, Y2)
    t.cuda.synchronize()
    assert np.array_equal(host(Y1).view(np.uint32), host(Y2).view(np.uint32))


# ---------------------------------------------------------------------------
# output and weight layouts: padded / unaligned leading dimensions, ragged N
# ---------------------------------------------------------------------------
def upload_coo(ql, delta, capacity=None):
    """The COO on the device, its arrays `capacity` entries long (at least
    nnz). fp4lin_gemm runs the compensation in its epilogue when the capacity
    is at most 10 entries per row of A, else as a second kernel: the capacity
    picks the schedule, and both give the same bits."""
    nz = max(delta.nnz, 1, capacity or 0)
    pad = lambda a, dt: np.concatenate([np.asarray(a, dt), np.zeros(nz - len(a), dt)])
    return ql.CooBuffers(upload_i32(pad(delta.row, np.int32)), upload_i32(pad(delta.col, np.int32)),
                         upload_f32(pad(delta.val32, np.float32)), upload_i32(delta.row_ptr))


FUSED_MAX_PER_ROW = 10


def schedule_capacity(schedule, M, nnz):
    if schedule == "fused":
        assert nnz <= FUSED_MAX_PER_ROW * M
        return nnz
    return max(nnz, FUSED_MAX_PER_ROW * M + 1)


@pytest.mark.parametrize("schedule", ["fused", "separate"])
@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("N,ldy_pad,ldw_pad", [(203, 5, 3), (256, 4, 0), (130, 2, 1),
                                               (517, 3, 8), (8, 0, 5)])
def test_gemm_compensation_padded_layouts(ql, dtype, N, ldy_pad, ldw_pad, schedule):
    """fp4lin_gemm with dA into a padded (possibly unaligned) Y, with a padded
    (possibly unaligned) W, under both schedules of the compensation (in the
    GEMM's epilogue, or as a second kernel): the element paths of the epilogue
    and of the compensation run, the result matches the oracle, and no padding
    column of Y is written."""
    t = torch()
    M, K = 150, 300
    log(f"gemm layouts {schedule} {dtype} N={N} ldy=N+{ldy_pad} ldw=N+{ldw_pad}")
    rng = np.random.default_rng(N * 7 + ldy_pad * 3 + ldw_pad)
    A = wl.random_matrix(rng, M, K, dtype, dist="t3")
    W = wl.random_matrix(rng, K, N, dtype, scale=0.02)
    ops = O.forward_operands(A.f32, W.f32, 0.97)
    Aq, Bq = upload_u8(O.pack_rows(ops.codesA)), upload_u8(O.pack_rows(ops.codesW))
    coo = upload_coo(ql, ops.delta, schedule_capacity(schedule, M, ops.delta.nnz))
    Wd = padded(to_device(W), N + ldw_pad)
    sentinel = float("nan")
    Ybuf = t.full((M, N + ldy_pad), sentinel, dtype=t.float32, device="cuda:0")
    Y = Ybuf[:, :N]
    ql.fp4lin_gemm(Aq, upload_f32(ops.sA), Bq, upload_f32(ops.sW), M, N, K, coo, Wd, Y)
    t.cuda.synchronize()
    full = host(Ybuf)
    if ldy_pad:
        assert np.isnan(full[:, N:]).all(), "a padding column of Y was written"
    err = O.rel_fro(full[:, :N], O.forward_output(ops, W.f32))
    assert err <= Y_TOL, err
    # the same through fp4lin_gemm (no dA) + fp4lin_sparse_add: same bits
    Ybuf2 = t.full((M, N + ldy_pad), sentinel, dtype=t.float32, device="cuda:0")
    Y2 = Ybuf2[:, :N]
    ql.fp4lin_gemm(Aq, upload_f32(ops.sA), Bq, upload_f32(ops.sW), M, N, K, None, None, Y2)
    ql.fp4lin_sparse_add(coo, Wd, Y2)
    t.cuda.synchronize()
    assert np.array_equal(host(Ybuf2).view(np.uint32), full.view(np.uint32))


def synthetic_delta(rng, M, K, lengths, pools=None):
    """A COO with the given number of non-zeros per row (distinct ascending
    columns, values of mixed sign and magnitude), as the oracle's SparseDelta.
    pools: per row, the columns to draw from (default: all of K)."""
    rows, cols = [], []
    for i, n in enumerate(lengths):
        pool = K if pools is None else pools[i]
        c = np.sort(rng.choice(pool, int(n), replace=False))
        rows.append(np.full(c.size, i))
        cols.append(c)
    row = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
    col = np.concatenate(cols).astype(np.int32) if cols else np.zeros(0, np.int32)
    val32 = (rng.standard_normal(row.size) * np.exp2(rng.integers(-3, 6, row.size))).astype(np.float32)
    row_ptr = np.zeros(M + 1, np.int64)
    row_ptr[1:] = np.cumsum(lengths)
    return O.SparseDelta(row, col, val32, val32.astype(np.float64), row_ptr.astype(np.int32), (M, K))


U32 = 2.0 ** -24


@pytest.mark.parametrize("wdtype", [wl.BF16, wl.F32])
@pytest.mark.parametrize("M,N,ldw_pad,pattern", [
    (300, 256, 0, "mixed"),       # ragged M (rows past M in the last tile)
    (200, 520, 0, "mixed"),       # ragged N, N % 4 == 0: vector gathers
    (130, 203, 0, "mixed"),       # N % 4 != 0: element gathers
    (257, 264, 3, "mixed"),       # unaligned W rows: element gathers
    (384, 512, 0, "dense-rows"),  # a few long rows among empty ones
    (128, 256, 0, "empty"),       # no non-zero at all
    (300, 264, 0, "channels"),    # all rows in 12 columns (outlier channels): the same
    (257, 203, 3, "channels"),    # W rows gathered by every row, ragged M and N, unaligned W
    (256, 256, 0, "channels-17"),  # 17 shared columns
    (384, 256, 0, "channels-mixed"),  # 8 shared columns in the first tile, 40 after
])
def test_gemm_compensation_row_structures(ql, wdtype, M, N, ldw_pad, pattern):
    """The compensation under both schedules on COOs built to reach the fused
    epilogue's corners: rows with 0, 1, 7, 8, 9, 16, 17 and 40 non-zeros (its
    gathers go in groups of 8 from each row's first non-zero), long rows next to
    empty ones, wholly empty tiles, rows past M, ragged N and unaligned W. The
    two schedules give the same bits, and every element of Y is within the fp32
    bound 3u|Y0| + (n_i + 2) u sum_k |dA[i,k] W[k,j]| of the oracle's float64
    value."""
    t = torch()
    K = 300
    log(f"gemm compensation structures {wdtype} {M}x{N} ldw=N+{ldw_pad} {pattern}")
    rng = np.random.default_rng(M * 31 + N + ldw_pad)
    if pattern == "mixed":
        cycle = np.array([0, 1, 7, 8, 9, 16, 17, 40, 0, 0, 3])
        lengths = cycle[np.arange(M) % cycle.size]
    elif pattern == "dense-rows":
        lengths = np.zeros(M, np.int64)
        lengths[[5, 6, 130, 131, 300, 383]] = [90, 1, 64, 33, 120, 15]
    elif pattern.startswith("channels"):
        wide = {"channels": 12, "channels-17": 17, "channels-mixed": 40}[pattern]
        few = rng.choice(K, 8, replace=False)
        many = rng.choice(K, wide, replace=False)
        # rows 0..127 (the first 128-row tile) draw from 8 columns in the mixed pattern
        pools = [few if (pattern == "channels-mixed" and i < 128) else many for i in range(M)]
        lengths = np.array([rng.integers(0, min(len(pools[i]), 10) + 1) for i in range(M)])
        lengths[::7] = 0  # rows without non-zeros between them
        delta = synthetic_delta(rng, M, K, lengths, pools)
    else:
        lengths = np.zeros(M, np.int64)
    if not pattern.startswith("channels"):
        delta = synthetic_delta(rng, M, K, lengths)
    ca = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cb = rng.integers(0, 16, (N, K)).astype(np.uint8)
    sa = np.exp2(rng.integers(-4, 4, M)).astype(np.float32)
    sb = (rng.random(N) + 0.5).astype(np.float32)
    W = wl.random_matrix(rng, K, N, wdtype, scale=0.02)
    Aq, Bq = upload_u8(O.pack_rows(ca)), upload_u8(O.pack_rows(cb))
    Wd = padded(to_device(W), N + ldw_pad) if ldw_pad else to_device(W)
    Ys = {}
    for schedule in ("fused", "separate"):
        coo = upload_coo(ql, delta, schedule_capacity(schedule, M, delta.nnz))
        Y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda:0")
        ql.fp4lin_gemm(Aq, upload_f32(sa), Bq, upload_f32(sb), M, N, K, coo, Wd, Y)
        t.cuda.synchronize()
        Ys[schedule] = host(Y)
    assert np.array_equal(Ys["fused"].view(np.uint32), Ys["separate"].view(np.uint32))
    y0 = O.scaled_product(O.integer_product(ca, cb), sa, sb)
    W64 = W.f32.astype(np.float64)
    want = y0 + O.sparse_times_dense(delta, W64)
    D = delta.dense64()
    T = np.abs(D) @ np.abs(W64)
    n_i = np.asarray(lengths, np.float64)[:, None]
    bound = (3 * U32 * np.abs(y0) + (n_i + 2) * U32 * T) * (1 + 1e-6)
    bad = np.abs(Ys["fused"].astype(np.float64) - want) > bound
    assert not bad.any(), f"{int(bad.sum())} elements beyond the fp32 bound"


# ---------------------------------------------------------------------------
# the largest shape the 32-bit operand offsets allow
# ---------------------------------------------------------------------------
def test_gemm_largest_packed_offsets(ql):
    """(M+1) * packed_ld(K) = 2^31 - 512, just under the limit the C ABI checks:
    the last rows' tiles address the top of the 2 GiB packed operand (and of
    its scale rows in the micro-scaled GEMM). Unit scales, so sampled rows are
    exact integer products."""
    t = torch()
    K, N = 1024, 16
    ldq = O.packed_ld(K)
    M = (1 << 31) // ldq - 2
    assert (M + 1) * ldq < (1 << 31) and (M + 2) * ldq >= (1 << 31)
    log(f"gemm largest offsets M={M} K={K} N={N}")
    rng = np.random.default_rng(12)
    # packed codes generated directly (two random nibbles per byte)
    Aq = t.randint(0, 256, (M, ldq), dtype=t.uint8, device="cuda:0",
                   generator=t.Generator(device="cuda:0").manual_seed(5))
    cb = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    Bq = upload_u8(O.pack_rows(cb))
    Y = ql.gemm(Aq, t.ones(M, dtype=t.float32, device="cuda:0"), Bq,
                t.ones(N, dtype=t.float32, device="cuda:0"), M, N, K)
    nb = ql.mx_scales_ld(K)
    As = t.full((M * nb,), 127, dtype=t.uint8, device="cuda:0")
    Bs = t.full((N * nb,), 127, dtype=t.uint8, device="cuda:0")
    Ymx = ql.gemm_mx(Aq, As, Bq, Bs, M, N, K)
    t.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1, M - 2, M - 129], rng.choice(M, 60, replace=False)]))
    sel = t.as_tensor(rows, device="cuda:0")
    ca = O.unpack_rows(host(Aq[sel]), K)
    want = O.integer_product(ca, cb)
    assert np.array_equal(host(Y[sel]).astype(np.float64), want)
    assert np.array_equal(host(Ymx[sel]).astype(np.float64), want)
    del Aq, As, Y, Ymx


def test_select_largest_count(ql):
    """M*K = 2^32 - 4096, just under the 32-bit histogram counts' limit (an
    8 GiB bfloat16 A drawn on the device). Checked by properties that hold at
    any size: tau is an element of |A| with #{|a| < tau} <= k < #{|a| <= tau};
    row_ptr[M] = #{|a| > tau}; sampled rows' COO entries are exactly their
    entries above tau, in column order, with val = RN32(a - sign(a) tau)."""
    t = torch()
    M, K, q = (1 << 20) - 1, 4096, 0.999
    n = M * K
    log(f"select largest count M={M} K={K}")
    g = t.Generator(device="cuda:0").manual_seed(3)
    A = t.randn((M, K), dtype=t.float32, device="cuda:0", generator=g).to(t.bfloat16)
    tau_d, coo = ql.outlier_select(A, q)
    t.cuda.synchronize()
    k = O.quantile_rank(n, q)
    tau = float(host(tau_d)[0])
    absA = A.abs()
    below = int((absA < tau).sum())
    at_or_below = int((absA <= tau).sum())
    assert below <= k < at_or_below
    nnz = int(host(coo.row_ptr[M:M + 1])[0])
    assert nnz == n - at_or_below
    del absA
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 30, replace=False)]))
    rp = host(coo.row_ptr).astype(np.int64)
    cols = host(coo.col)
    vals = host(coo.val)
    for i in rows:
        a = A[int(i)].float().cpu().numpy()
        want_c = np.nonzero(np.abs(a) > np.float32(tau))[0]
        lo, hi = rp[i], rp[i + 1]
        assert np.array_equal(cols[lo:hi], want_c), i
        want_v = (a[want_c].astype(np.float64) - np.sign(a[want_c]) * tau).astype(np.float32)
        assert_bits_equal(vals[lo:hi], want_v, f"row {i} values")
    del A, coo


def test_sparse_add_largest_weight_offsets(ql):
    """K * ldw * 2 = 2^31 - 524288 (a 2 GiB bfloat16 W, just under the 32-bit
    byte-offset limit the C ABI checks), with entries in W's last rows: each
    row of Y equals its entries' sum of val * W[k, :] (float64 reference,
    relative error of an fp32 sum of at most 64 terms)."""
    t = torch()
    K, N, M = 32768, 32760, 48
    assert K * N * 2 < (1 << 31)
    log(f"sparse_add largest offsets K={K} N={N}")
    g = t.Generator(device="cuda:0").manual_seed(8)
    W = (t.randn((K, N), dtype=t.float32, device="cuda:0", generator=g) * 0.02).to(t.bfloat16)
    rng = np.random.default_rng(9)
    rows, cols, vals = [], [], []
    row_ptr = [0]
    for i in range(M):
        c = np.unique(np.concatenate([[K - 1, K - 2 - i], rng.choice(K, 40, replace=False)]))
        rows += [i] * len(c)
        cols += list(c)
        vals += list(rng.standard_normal(len(c)).astype(np.float32) * 10)
        row_ptr.append(len(cols))
    coo = ql.CooBuffers(upload_i32(rows), upload_i32(cols), upload_f32(vals), upload_i32(row_ptr))
    Y = t.zeros((M, N), dtype=t.float32, device="cuda:0")
    ql.fp4lin_sparse_add(coo, W, Y)
    t.cuda.synchronize()
    Yh = host(Y).astype(np.float64)
    vals = np.asarray(vals, np.float32).astype(np.float64)
    for i in range(M):
        lo, hi = row_ptr[i], row_ptr[i + 1]
        idx = t.as_tensor(np.asarray(cols[lo:hi]), device="cuda:0")
        Wr = W[idx].float().cpu().numpy().astype(np.float64)
        want = vals[lo:hi] @ Wr
        err = np.abs(Yh[i] - want).max() / max(np.abs(want).max(), 1e-30)
        assert err < 1e-5, (i, err)
    del W, Y
