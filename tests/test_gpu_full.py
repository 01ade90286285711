"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark times (one fp4lin_forward per layer).

Bit-exact over the whole arrays: tau, the COO of dA (row, col, val, row_ptr),
the packed codes and scales of A and W. Every element of Y (and of dX and dW
for the dgrad and wgrad GEMMs) is held to the fp32 error bound of the
arithmetic the library performs, against the oracle's float64 result:

  forward  Y = RN(Y0 + s), Y0 = RN(RN(acc * sA) * sW) with acc exact, s the
           fp32 FMA chain from 0 over row i's n_i non-zeros of dA (values
           rounded to fp32):
             |Y - Y64| <= 3u |Y0_64| + (n_i + 2) u T,  T = sum_k |dA[i,k] W[k,j]|
  dgrad / wgrad (no compensation):  |dX - dX64| <= 2u |dX64|
with u = 2^-24 (second-order terms covered by a factor 1 + 1e-6). The relative
Frobenius error over all of Y is also held to 1e-5.
"""
import numpy as np
import pytest

import oracle as O
import workloads as wl
from gpu_util import assert_bits_equal, host, log, to_device

pytestmark = pytest.mark.gpu

Y_TOL = 1e-5
U = 2.0 ** -24
ROW_CHUNK = 2048


@pytest.fixture(scope="module")
def ql():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_linear_layer_amd as q
    q.lib()
    return q


def sample_rows(M, seed=0, per_tile=8, tile=128):
    """Rows spread over every 128-row tile: its first and last row and
    per_tile - 2 seeded others (for checks too slow to run on every row)."""
    rng = np.random.default_rng(seed)
    out = []
    for t0 in range(0, M, tile):
        t1 = min(M, t0 + tile)
        mid = np.arange(t0 + 1, t1 - 1)
        pick = rng.choice(mid, min(per_tile - 2, mid.size), replace=False) if mid.size else []
        out.extend([t0, t1 - 1, *pick])
    return np.unique(np.array(out, dtype=np.int64))


def chunk_delta(delta, rows):
    """The dense float64 rows of dA for a contiguous block of rows (for the
    error bound's T = |dA| |W| and for Y0 = Y - dA W, as BLAS products)."""
    r0, r1 = int(rows[0]), int(rows[-1]) + 1
    lo, hi = int(delta.row_ptr[r0]), int(delta.row_ptr[r1])
    D = np.zeros((r1 - r0, delta.shape[1]), dtype=np.float64)
    D[delta.row[lo:hi] - r0, delta.col[lo:hi]] = delta.val64[lo:hi]
    return D


def check_forward_rows(ops, W32, Y_host, what):
    """Every row of Y against the oracle and the elementwise bound. The oracle's
    integer product and scale epilogue give Y0 for all rows at once; its dA
    (float64 values) times W is formed per block of rows as a dense product,
    which equals the oracle's sparse term (pinned on the CPU) up to float64
    rounding; forward_output itself is compared on the first and last row of
    every 128-row tile."""
    M = Y_host.shape[0]
    W64 = np.asarray(W32, dtype=np.float64)
    Wabs = np.abs(W64)
    n_i = np.diff(ops.delta.row_ptr.astype(np.int64))
    y0_all = O.scaled_product(O.integer_product(ops.codesA, ops.codesW), ops.sA, ops.sW)
    sample = sample_rows(M, seed=3, per_tile=2)
    num = den = 0.0
    worst = 0.0
    for r0 in range(0, M, ROW_CHUNK):
        rows = np.arange(r0, min(M, r0 + ROW_CHUNK))
        D = chunk_delta(ops.delta, rows)
        T = np.abs(D) @ Wabs
        y0 = y0_all[rows]
        want = y0 + D @ W64
        del D
        bound = (3 * U * np.abs(y0) + (n_i[rows, None] + 2) * U * T) * (1 + 1e-6)
        err = np.abs(Y_host[rows].astype(np.float64) - want)
        bad = err > bound
        if bad.any():
            i, j = np.argwhere(bad)[0]
            raise AssertionError(
                f"{what}: {int(bad.sum())} elements beyond the fp32 bound in rows "
                f"{r0}..{rows[-1]}, first Y[{rows[i]},{j}] = {Y_host[rows[i], j]!r} want "
                f"{want[i, j]!r} bound {bound[i, j]:.3e}")
        worst = max(worst, float((err / np.maximum(bound, 1e-300)).max()))
        num += float(np.sum(err * err))
        den += float(np.sum(want * want))
        mine = sample[(sample >= r0) & (sample <= rows[-1])]
        if mine.size:
            ref = O.forward_output(ops, W32, rows=mine)
            assert np.allclose(want[mine - r0], ref, rtol=1e-12, atol=1e-300), what
    rel = (num ** 0.5) / (den ** 0.5) if den else 0.0
    return rel, worst


def check_layer(ql, L: wl.Layer):
    import torch
    log(f"[full] {L.name}: M={L.M} K={L.K} N={L.N} q={L.q} — GPU forward")
    A, W = to_device(L.A), to_device(L.W)
    Y, ws = ql.forward(A, W, L.q, return_workspace=True)
    torch.cuda.synchronize()
    o = ql.forward_layout(L.M, L.K, L.N, ql.BF16 if L.A.dtype == wl.BF16 else ql.F32, L.q)
    Y_host = host(Y)
    del Y, A, W
    log(f"[full] {L.name}: oracle operands")
    ops = O.forward_operands(L.A.f32, L.W.f32, L.q)
    b = ws  # device bytes; copy slices only
    ldq = ql.packed_ld(L.K)

    def dev_slice(off, n, dt):
        nb = n * np.dtype(dt).itemsize
        return b[off: off + nb].cpu().numpy().view(dt)

    assert_bits_equal(dev_slice(o.tau, 1, np.float32)[0], ops.tau, "tau")
    rp = dev_slice(o.row_ptr, L.M + 1, np.int32)
    assert_bits_equal(rp, ops.delta.row_ptr, "row_ptr")
    nnz = int(rp[-1])
    assert nnz == ops.delta.nnz <= o.capacity
    assert_bits_equal(dev_slice(o.coo_row, nnz, np.int32), ops.delta.row, "coo row")
    assert_bits_equal(dev_slice(o.coo_col, nnz, np.int32), ops.delta.col, "coo col")
    assert_bits_equal(dev_slice(o.coo_val, nnz, np.float32), ops.delta.val32, "coo val")
    assert_bits_equal(dev_slice(o.sA, L.M, np.float32), ops.sA, "sA")
    assert_bits_equal(dev_slice(o.Aq, L.M * ldq, np.uint8).reshape(L.M, ldq), ops.Aq, "Aq")
    assert_bits_equal(dev_slice(o.sW, L.N, np.float32), ops.sW, "sW")
    assert_bits_equal(dev_slice(o.Wq, L.N * ldq, np.uint8).reshape(L.N, ldq), ops.Wq, "Wq")
    del ws, b
    log(f"[full] {L.name}: Y on all {L.M} rows against the oracle")
    rel, worst = check_forward_rows(ops, L.W.f32, Y_host, L.name)
    log(f"[full] {L.name}: nnz {nnz}, tau {float(ops.tau):.6g}, Y rel_fro {rel:.3e}, "
        f"largest error / bound {worst:.3f}")
    assert rel <= Y_TOL, rel


def check_unscaled_gemm_rows(got, want, what):
    """dX / dW: exact integer accumulation, two fp32 roundings in the epilogue."""
    err = np.abs(got.astype(np.float64) - want)
    bound = 2 * U * np.abs(want) * (1 + 1e-6)
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond 2u|x|"
    rel = O.rel_fro(got, want)
    assert rel <= Y_TOL, rel
    return rel


def test_full_llama1_3b_ffn_up(ql):
    check_layer(ql, wl.make_layer("llama1.3b_ffn_up"))


def test_full_llama7b_ffn_up(ql):
    check_layer(ql, wl.make_layer("llama7b_ffn_up"))


def test_full_llama13b_ffn_up_down(ql):
    up, down = wl.make_13b_pair()
    check_layer(ql, up)
    del up
    check_layer(ql, down)


def test_full_llama13b_qkv_forward(ql):
    check_layer(ql, wl.make_layer("llama13b_qkv"))


def test_full_llama13b_qkv_dgrad(ql):
    """dX = Q(dY) Q(W)^T through the public calls: quantize_act on dY rows and
    on W rows (both over N), then fp4lin_gemm without compensation."""
    import torch
    L = wl.make_layer("llama13b_qkv")
    M, K, N = L.M, L.K, L.N
    log(f"[full] dgrad: dY {M}x{N}, W {K}x{N}")
    dY = wl.make_grad_output(M, N)
    dYd, Wd = to_device(dY), to_device(L.W)
    dYq, s_dy = ql.quantize_act(dYd)
    Wq2, s_w2 = ql.quantize_act(Wd)
    dX = ql.gemm(dYq, s_dy, Wq2, s_w2, M, K, N)
    torch.cuda.synchronize()
    log("[full] dgrad: oracle, all rows")
    want_dX, (q_dy, want_sdy, c_dy), (q_w2, want_sw2, c_w2) = O.dgrad(dY.f32, L.W.f32)
    assert_bits_equal(host(s_dy), want_sdy, "s_dY")
    assert_bits_equal(host(dYq), q_dy, "dYq")
    assert_bits_equal(host(s_w2), want_sw2, "s_W rows")
    assert_bits_equal(host(Wq2), q_w2, "Wq rows")
    err = check_unscaled_gemm_rows(host(dX), want_dX, "dX")
    log(f"[full] dgrad: dX rel_fro on all {M} rows {err:.3e}, every element within 2u")


def test_full_llama13b_qkv_wgrad(ql):
    """dW = Q(A)^T Q(dY) through the public calls: quantize_weight on A and on
    dY (both per column over M), then fp4lin_gemm with K' = M."""
    import torch
    L = wl.make_layer("llama13b_qkv")
    M, K, N = L.M, L.K, L.N
    log(f"[full] wgrad: A {M}x{K}, dY {M}x{N}")
    dY = wl.make_grad_output(M, N)
    Ad, dYd = to_device(L.A), to_device(dY)
    Aq2, s_a2 = ql.quantize_weight(Ad)
    dYq2, s_dy2 = ql.quantize_weight(dYd)
    dW = ql.gemm(Aq2, s_a2, dYq2, s_dy2, K, N, M)
    torch.cuda.synchronize()
    log("[full] wgrad: oracle, all rows")
    want_dW, (q_a2, want_sa2, _), (q_dy2, want_sdy2, _) = O.wgrad(L.A.f32, dY.f32)
    assert_bits_equal(host(s_a2), want_sa2, "s_A columns")
    assert_bits_equal(host(Aq2), q_a2, "Aq columns")
    assert_bits_equal(host(s_dy2), want_sdy2, "s_dY columns")
    assert_bits_equal(host(dYq2), q_dy2, "dYq columns")
    err = check_unscaled_gemm_rows(host(dW), want_dW, "dW")
    log(f"[full] wgrad: dW rel_fro on all {K} rows {err:.3e}, every element within 2u")


def test_full_llama7b_ffn_up_mx(ql):
    """The micro-scaled forward at the benchmark's size, as bench.py --quant mx
    runs it (select, quantize_act_mx, quantize_weight_mx, gemm_mx with the
    compensation): codes and scale bytes bit-exact over the whole arrays; Y on
    eight rows of every 128-row tile (the oracle's block-scaled product is too
    slow for all rows), each element within the fp32 bound
    (2 b + 3) u mag + (n_i + 2) u T, where b is the number of 32-code blocks,
    mag the sum of the block terms' magnitudes and T = sum_k |dA[i,k] W[k,j]|."""
    import torch
    L = wl.make_layer("llama7b_ffn_up")
    log(f"[full] {L.name} (micro-scaled): GPU calls")
    A, W = to_device(L.A), to_device(L.W)
    tau, coo = ql.outlier_select(A, L.q)
    Aq, As = ql.quantize_act_mx(A, tau)
    Wq, Ws = ql.quantize_weight_mx(W)
    Y = ql.gemm_mx(Aq, As, Wq, Ws, L.M, L.N, L.K, coo, W)
    Yf = ql.forward_mx(A, W, L.q)          # the one-call forward, as bench.py times it
    torch.cuda.synchronize()
    assert_bits_equal(host(Yf), host(Y), "forward_mx Y against the separate calls")
    del Yf
    rows = sample_rows(L.M, seed=7)
    log(f"[full] {L.name} (micro-scaled): oracle")
    want, mag, otau, delta, qa, qw = O.forward_mx(L.A.f32, L.W.f32, L.q, rows=rows)
    assert_bits_equal(host(tau)[0], otau, "tau")
    # step-major (steps, rows, 4) scale bytes as rows x blocks
    rows_of = lambda a, R: np.ascontiguousarray(np.asarray(a).reshape(-1, R, 4)
                                                .transpose(1, 0, 2).reshape(R, -1))
    assert_bits_equal(rows_of(host(As), L.M), qa[1], "A scale bytes")
    assert_bits_equal(host(Aq), qa[0], "A codes")
    assert_bits_equal(rows_of(host(Ws), L.N), qw[1], "W scale bytes")
    assert_bits_equal(host(Wq), qw[0], "W codes")
    got = host(Y[torch.as_tensor(rows, device=Y.device)]).astype(np.float64)
    Wabs = np.abs(L.W.f32.astype(np.float64))
    T = np.concatenate([np.abs(chunk_delta(delta, [r])) @ Wabs for r in rows])
    n_i = np.diff(delta.row_ptr.astype(np.int64))[rows]
    nb = ql.packed_ld(L.K) * 2 // 32
    bound = ((2 * nb + 3) * U * mag + (n_i[:, None] + 2) * U * T) * (1 + 1e-6)
    bad = np.abs(got - want) > bound
    assert not bad.any(), f"{int(bad.sum())} elements of Y beyond the fp32 bound"
    err = O.rel_fro(got, want)
    log(f"[full] {L.name} (micro-scaled): Y rel err {err:.3g} on {rows.size} rows of all "
        f"{-(-L.M // 128)} tiles, every element within the bound")
    assert err <= Y_TOL
