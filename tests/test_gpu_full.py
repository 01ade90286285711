"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark times (one fp4lin_forward per layer).

Bit-exact over the whole arrays: tau, the COO of dA (row, col, val, row_ptr),
the packed codes and scales of A and W. Y (and dX and dW for the dgrad and
wgrad GEMMs) is compared with the oracle on sampled rows (first, last and a
seeded spread), relative Frobenius error <= 1e-5.
"""
import numpy as np
import pytest

import oracle as O
import workloads as wl
from gpu_util import assert_bits_equal, host, log, to_device

pytestmark = pytest.mark.gpu

Y_TOL = 1e-5
N_SAMPLE_ROWS = 48


@pytest.fixture(scope="module")
def ql():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_linear_layer_amd as q
    q.lib()
    return q


def sample_rows(M, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, N_SAMPLE_ROWS - 2, replace=False)]))
    return rows


def check_layer(ql, L: wl.Layer):
    import torch
    log(f"[full] {L.name}: M={L.M} K={L.K} N={L.N} q={L.q} — GPU forward")
    A, W = to_device(L.A), to_device(L.W)
    Y, ws = ql.forward(A, W, L.q, return_workspace=True)
    torch.cuda.synchronize()
    o = ql.forward_layout(L.M, L.K, L.N, ql.BF16 if L.A.dtype == wl.BF16 else ql.F32, L.q)
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
    rows = sample_rows(L.M)
    want = O.forward_output(ops, L.W.f32, rows=rows)
    got = host(Y[torch.from_numpy(rows).to(Y.device)])
    err = O.rel_fro(got, want)
    log(f"[full] {L.name}: nnz {nnz}, tau {float(ops.tau):.6g}, Y rel_fro on {rows.size} rows {err:.3e}")
    assert err <= Y_TOL, err


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
    log("[full] dgrad: oracle")
    rows = sample_rows(M, seed=1)
    want_dX, (q_dy, want_sdy, c_dy), (q_w2, want_sw2, c_w2) = O.dgrad(dY.f32, L.W.f32, rows=rows)
    assert_bits_equal(host(s_dy), want_sdy, "s_dY")
    assert_bits_equal(host(dYq), q_dy, "dYq")
    assert_bits_equal(host(s_w2), want_sw2, "s_W rows")
    assert_bits_equal(host(Wq2), q_w2, "Wq rows")
    got = host(dX[torch.from_numpy(rows).to(dX.device)])
    err = O.rel_fro(got, want_dX)
    log(f"[full] dgrad: dX rel_fro on {rows.size} rows {err:.3e}")
    assert err <= Y_TOL, err


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
    log("[full] wgrad: oracle")
    rows = sample_rows(K, seed=2)
    want_dW, (q_a2, want_sa2, _), (q_dy2, want_sdy2, _) = O.wgrad(L.A.f32, dY.f32, rows=rows)
    assert_bits_equal(host(s_a2), want_sa2, "s_A columns")
    assert_bits_equal(host(Aq2), q_a2, "Aq columns")
    assert_bits_equal(host(s_dy2), want_sdy2, "s_dY columns")
    assert_bits_equal(host(dYq2), q_dy2, "dYq columns")
    got = host(dW[torch.from_numpy(rows).to(dW.device)])
    err = O.rel_fro(got, want_dW)
    log(f"[full] wgrad: dW rel_fro on {rows.size} rows {err:.3e}")
    assert err <= Y_TOL, err


def test_full_llama7b_ffn_up_mx(ql):
    """The micro-scaled forward at the benchmark's size, as bench.py --quant mx
    runs it (select, quantize_act_mx, quantize_weight_mx, gemm_mx with the
    compensation): codes and scale bytes bit-exact over the whole arrays, Y on
    sampled rows."""
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
    err = O.rel_fro(host(Y[torch.as_tensor(rows, device=Y.device)]), want)
    log(f"[full] {L.name} (micro-scaled): Y rel err {err:.3g}")
    assert err <= Y_TOL
