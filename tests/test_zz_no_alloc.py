"""The allocation-free select, fp4lin_outlier_select_noalloc, against the
workspace entry point fp4lin_outlier_select through the C ABI: tau, row_ptr
and the COO arrays must be bit-identical. Each case makes two calls in a row
on the same GPU's static scratch, the second with a smaller input, so that
the second call runs on what the first left behind. Also: the largest row
count whose select fits the scratch, and one row more (refused before any
launch)."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import assert_bits_equal, host, log, to_device

pytestmark = pytest.mark.gpu

# rows whose select workspace is exactly the 8 MiB static scratch (bfloat16)
MAX_ROWS_BF16 = 1_865_152


@pytest.fixture(scope="module")
def ql():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_linear_layer_amd as q
    q.lib()
    return q


def noalloc_select(ql, A, q):
    import torch
    M, K = A.shape
    k = ql.quantile_rank(M * K, q)
    tau = torch.full((1,), -1.0, dtype=torch.float32, device=A.device)
    coo = ql.CooBuffers.empty(M, M * K - 1 - k, A.device)
    ql.fp4lin_outlier_select_noalloc(A, q, tau, coo)
    return tau, coo


def assert_same_select(ql, A, q, what):
    import torch
    tau_r, coo_r = ql.outlier_select(A, q)
    tau, coo = noalloc_select(ql, A, q)
    torch.cuda.synchronize()
    assert_bits_equal(host(tau), host(tau_r), f"{what}: tau")
    rp = host(coo.row_ptr)
    assert_bits_equal(rp, host(coo_r.row_ptr), f"{what}: row_ptr")
    nnz = int(rp[-1])
    for name in ("row", "col", "val"):
        assert_bits_equal(host(getattr(coo, name))[:nnz], host(getattr(coo_r, name))[:nnz],
                          f"{what}: {name}")
    return nnz


SEQUENCES = [
    # (dtype, M, K, q) pairs: a larger call, then a smaller one
    [(wl.BF16, 8192, 4096, 0.99), (wl.BF16, 700, 333, 0.9)],
    [(wl.F32, 2000, 600, 0.995), (wl.F32, 130, 77, 0.5)],
    [(wl.BF16, 3000, 1000, 0.999), (wl.F32, 257, 520, 0.97)],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "-".join(f"{d}{m}x{k}" for d, m, k, _ in s))
def test_noalloc_select_matches_workspace_select(ql, seq):
    rng = np.random.default_rng(sum(m * k for _, m, k, _ in seq))
    for i, (dtype, M, K, q) in enumerate(seq):
        log(f"noalloc select call {i}: {dtype} {M}x{K} q={q}")
        A = to_device(wl.random_matrix(rng, M, K, dtype, dist="t3"))
        nnz = assert_same_select(ql, A, q, f"call {i} {dtype} {M}x{K}")
        log(f"  nnz {nnz}, identical")


def test_noalloc_select_at_scratch_limit(ql):
    """The largest bfloat16 row count whose select fits the scratch (K = 16),
    then a small call; one row more is refused with FP4LIN_ERR_SCRATCH."""
    import torch
    rng = np.random.default_rng(21)
    M, K = MAX_ROWS_BF16, 16
    assert ql.select_workspace_bytes(M, K, ql.BF16) == 8 << 20
    assert ql.select_workspace_bytes(M + 1, K, ql.BF16) > 8 << 20
    log(f"noalloc select at the scratch limit: bf16 {M}x{K}")
    A = to_device(wl.random_matrix(rng, M, K, wl.BF16, dist="t3"))
    assert_same_select(ql, A, 0.99, "limit")
    A2 = to_device(wl.random_matrix(rng, 1000, 64, wl.BF16, dist="t3"))
    assert_same_select(ql, A2, 0.95, "after the limit")
    big = torch.zeros((M + 1, K), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ql.Fp4linError) as ei:
        noalloc_select(ql, big, 0.99)
    assert ei.value.status == 9   # FP4LIN_ERR_SCRATCH
