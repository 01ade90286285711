"""Pins for the CPU oracle: checks against facts the pages and mathematics fix,
never against the oracle's own formulas retyped.

Citations are to the FP4 training write-up "微软首创FP4训练框架，训练效果媲美BF16"
(format, granularity, rounding, ScaleShift, outlier-clamp and compensation
paragraphs) unless stated otherwise.
"""
import math
import multiprocessing as mp
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as wl

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


# ---------------------------------------------------------------------------
# E2M1 encoder: exhaustive against a brute-force nearest search
# ---------------------------------------------------------------------------
def _brute_nearest(y32):
    """Nearest grid magnitude by explicit distance search in float64; on a tie
    the larger magnitude wins (round half away from zero); NaN -> index 0."""
    y = y32.astype(np.float64)
    best = np.zeros(y.shape, dtype=np.uint8)
    bestd = np.abs(y - 0.0)
    for idx in range(1, 8):
        d = np.abs(y - GRID[idx])
        with np.errstate(invalid="ignore"):
            take = d <= bestd
        best = np.where(take, np.uint8(idx), best)
        bestd = np.where(take, d, bestd)
    return best


def _check_chunk(start):
    n = 1 << 24
    bits = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32)
    y = bits.view(np.float32)
    got = O.encode_magnitude(y)
    want = _brute_nearest(y)
    # NaN patterns: no midpoint reached, and no distance compares -> 0 both ways
    bad = np.nonzero(got != want)[0]
    return int(bad.size), (int(bits[bad[0]]) if bad.size else None)


@pytest.mark.slow
def test_e2m1_encoder_exhaustive_all_fp32_patterns():
    """Every sign-clear float32 bit pattern y (the encoder sees y = |x|*inv >= 0,
    or NaN): midpoint counting == nearest search (R3). 2^31 patterns."""
    starts = [c << 24 for c in range(128)]
    with mp.get_context("fork").Pool(min(8, mp.cpu_count())) as pool:
        res = pool.map(_check_chunk, starts, chunksize=4)
    nbad = sum(r[0] for r in res)
    first = [r[1] for r in res if r[1] is not None]
    assert nbad == 0, f"{nbad} mismatches, first bit pattern {first[:1]}"


def test_e2m1_encoder_special_points():
    """Grid points map to themselves, midpoints go up, saturation, NaN -> 0."""
    for i, g in enumerate(GRID):
        assert O.encode_magnitude(np.float32(g)) == i
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for i, t in enumerate(mids):
        assert O.encode_magnitude(np.float32(t)) == i + 1          # tie -> larger
        below = np.nextafter(np.float32(t), np.float32(0))
        assert O.encode_magnitude(below) == i                      # just below -> smaller
    assert O.encode_magnitude(np.float32(6.0000005)) == 7
    assert O.encode_magnitude(np.float32(np.inf)) == 7
    assert O.encode_magnitude(np.float32(np.nan)) == 0
    assert O.encode_magnitude(np.float32(1e-45)) == 0
    neg_nan = np.array([0xFF800001, 0xFFC00000, 0xFFFFFFFF], dtype=np.uint32).view(np.float32)
    assert not O.encode_magnitude(neg_nan).any()


# ---------------------------------------------------------------------------
# Scales: exact rounding through Fractions
# ---------------------------------------------------------------------------
def _rn32_fraction(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32, ties to even, by
    comparing exact distances to the two float32 neighbours."""
    approx = np.float32(float(fr))
    cands = {approx, np.nextafter(approx, np.float32(np.inf)),
             np.nextafter(approx, np.float32(-np.inf))}
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - fr)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def test_scales_exactly_rounded_tiny_workload():
    """s = RN32(amax/6) and inv = RN32(6/amax) for every row of the tiny workload."""
    L = wl.make_layer("tiny")
    A = L.A.f32
    amax = np.abs(A).max(axis=1)
    s, inv = O.vector_scales(amax)
    for i in range(A.shape[0]):
        fa = Fraction(float(amax[i]))
        assert s[i] == _rn32_fraction(fa / 6), i
        assert inv[i] == _rn32_fraction(6 / fa), i


def test_power_of_two_metamorphic():
    """Scaling a row by 2^p leaves its codes unchanged and scales s by 2^p."""
    rng = np.random.default_rng(3)
    X = rng.standard_normal((16, 300)).astype(np.float32)
    c0, s0 = O.quantize_rows(X)
    for p in (-20, -3, 1, 7, 30):
        f = np.float32(2.0 ** p)
        c1, s1 = O.quantize_rows(X * f)
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1, s0 * f)


def test_grid_exact_rows_round_trip():
    """Rows that already are s*{grid values} quantize without error (R1, R2)."""
    rng = np.random.default_rng(5)
    R, L = 64, 200
    mags = rng.integers(0, 8, size=(R, L))
    mags[:, 0] = 7                                     # each row's amax is 6*s
    signs = rng.choice([-1.0, 1.0], size=(R, L))
    scale = 2.0 ** rng.integers(-30, 30, size=R)
    X = (np.array(GRID)[mags] * signs * scale[:, None]).astype(np.float32)
    codes, s = O.quantize_rows(X)
    assert np.array_equal(s, scale.astype(np.float32))
    back = O.decode(codes) * s[:, None].astype(np.float64)
    assert np.array_equal(back, X.astype(np.float64))


def test_zero_and_subnormal_rows():
    """amax = 0: every code is +0/-0 with scale 0; subnormal amax: inv = Inf (R3, R4)."""
    X = np.zeros((2, 8), dtype=np.float32)
    X[1, :] = -0.0
    codes, s = O.quantize_rows(X)
    assert np.all(s == 0)
    assert np.all(codes[0] == 0) and np.all(codes[1] == 8)
    tiny = np.array([[1e-45, -1e-45, 0.0, 3e-45]], dtype=np.float32)
    codes, s = O.quantize_rows(tiny)
    assert s[0] == np.float32(3e-45 / 6)  # rounds to 0 or the smallest subnormal
    assert list(codes[0]) == [7, 15, 0, 7]


# ---------------------------------------------------------------------------
# Threshold: full sort and order-statistic invariants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("q", [0.0, 0.5, 0.9, 0.99, 0.999, 1.0])
def test_threshold_against_full_sort(q):
    L = wl.make_layer("tiny")
    A = L.A.f32
    tau, k = O.select_threshold(A, q)
    srt = np.sort(np.abs(A).ravel())
    assert k == min(max(math.ceil(q * A.size) - 1, 0), A.size - 1)
    assert tau == srt[k]
    absA = np.abs(A)
    assert np.count_nonzero(absA < tau) <= k < np.count_nonzero(absA <= tau)
    perm = np.random.default_rng(1).permutation(A.size)
    tau_p, _ = O.select_threshold(A.ravel()[perm].reshape(A.shape), q)
    assert tau_p == tau


def test_quantile_one_clamps_nothing():
    L = wl.make_layer("tiny")
    tau, _ = O.select_threshold(L.A.f32, 1.0)
    assert tau == np.abs(L.A.f32).max()
    _, d = O.clamp_and_residual(L.A.f32, tau)
    assert d.nnz == 0


def test_threshold_bf16_slice_against_sort():
    """A slice of the 1.3B-like workload (bf16 data, many ties at tau)."""
    L = wl.make_layer("llama1.3b_ffn_up", M=256)
    A = L.A.f32
    tau, k = O.select_threshold(A, 0.99)
    assert tau == np.sort(np.abs(A).ravel())[k]


# ---------------------------------------------------------------------------
# Delta A: support, exact reconstruction, rounding of the stored values
# ---------------------------------------------------------------------------
def test_delta_support_and_exact_reconstruction():
    L = wl.make_layer("tiny")
    A = L.A.f32
    tau, k = O.select_threshold(A, L.q)
    A_c, d = O.clamp_and_residual(A, tau)
    C = np.abs(A) > tau
    dense = np.zeros(A.shape, dtype=bool)
    dense[d.row, d.col] = True
    assert np.array_equal(dense, C)                          # non-zero exactly on C
    assert d.nnz <= A.size - 1 - k
    order = d.row.astype(np.int64) * A.shape[1] + d.col
    assert np.all(np.diff(order) > 0)                        # row-major, no duplicates
    assert np.all(np.abs(A_c) <= tau)
    # A_c + Delta A == A exactly, per entry, in rationals
    for r, c, v in zip(d.row[:200], d.col[:200], d.val64[:200]):
        assert Fraction(float(A_c[r, c])) + Fraction(float(v)) == Fraction(float(A[r, c]))
        assert np.sign(v) == np.sign(A[r, c])
    # the float32 values are the correctly rounded differences
    for r, c, v32 in zip(d.row, d.col, d.val32):
        a = Fraction(float(A[r, c]))
        exact = a - (Fraction(float(tau)) if a > 0 else -Fraction(float(tau)))
        assert v32 == _rn32_fraction(exact)
    assert np.array_equal(np.diff(d.row_ptr), np.count_nonzero(C, axis=1))


# ---------------------------------------------------------------------------
# Products: closed forms
# ---------------------------------------------------------------------------
def _grid_exact(rng, R, L, axis):
    """R x L matrix whose rows (axis=1) or columns (axis=0) are power-of-two
    multiples of E2M1 grid values, each vector reaching 6*s."""
    mags = rng.integers(0, 8, size=(R, L))
    if axis == 1:
        mags[:, rng.integers(0, L)] = 7
        sc = 2.0 ** rng.integers(-6, 6, size=(R, 1))
    else:
        mags[rng.integers(0, R), :] = 7
        sc = 2.0 ** rng.integers(-6, 6, size=(1, L))
    signs = rng.choice([-1.0, 1.0], size=(R, L))
    return (np.array(GRID)[mags] * signs * sc).astype(np.float32)


def test_forward_equals_plain_product_on_grid_exact_inputs():
    """q = 1 (nothing clamped) and grid-exact A rows / W columns: Y = A W exactly.
    Non-square shapes catch a transposed operand or swapped scale axis."""
    rng = np.random.default_rng(11)
    M, K, N = 37, 150, 23
    A = _grid_exact(rng, M, K, axis=1)
    W = _grid_exact(rng, K, N, axis=0)
    Y, ops = O.forward(A, W, 1.0)
    assert ops.delta.nnz == 0
    assert np.array_equal(Y, A.astype(np.float64) @ W.astype(np.float64))


def test_integer_product_against_int64():
    rng = np.random.default_rng(2)
    ca = rng.integers(0, 16, size=(20, 333)).astype(np.uint8)
    cb = rng.integers(0, 16, size=(9, 333)).astype(np.uint8)
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12], dtype=np.int64)
    ia = np.where(ca & 8, -1, 1) * twice[ca & 7]
    ib = np.where(cb & 8, -1, 1) * twice[cb & 7]
    ref = np.zeros((20, 9), dtype=np.int64)
    for i in range(20):
        for j in range(9):
            ref[i, j] = int(np.sum(ia[i] * ib[j]))
    assert np.array_equal(O.integer_product(ca, cb) * 4, ref.astype(np.float64))


def test_compensation_equals_dense_residual():
    """The sparse term equals (A - A_clamped) W computed densely."""
    L = wl.make_layer("tiny")
    A, W = L.A.f32, L.W.f32
    Y, ops = O.forward(A, W, L.q)
    dense = (A.astype(np.float64) - ops.A_c.astype(np.float64)) @ W.astype(np.float64)
    sparse = O.sparse_times_dense(ops.delta, W)
    assert O.rel_fro(sparse, dense) < 1e-13
    quant = O.scaled_product(O.integer_product(ops.codesA, ops.codesW), ops.sA, ops.sW)
    assert O.rel_fro(Y, quant + dense) < 1e-13
    # the layer output approximates A W (FP4 error, outliers compensated)
    exact = A.astype(np.float64) @ W.astype(np.float64)
    assert O.rel_fro(Y, exact) < 0.25


def test_dgrad_closed_form():
    """dY rows and W rows grid-exact: Q(dY) Q(W)^T == dY W^T exactly (R9)."""
    rng = np.random.default_rng(4)
    M, N, K = 19, 260, 13
    dY = _grid_exact(rng, M, N, axis=1)
    W = _grid_exact(rng, K, N, axis=1)
    dX, _, _ = O.dgrad(dY, W)
    assert np.array_equal(dX, dY.astype(np.float64) @ W.astype(np.float64).T)


def test_wgrad_closed_form():
    """A and dY columns grid-exact over M: Q(A)^T Q(dY) == A^T dY exactly (R10).
    M = 150 pads the packed columns; K != N catches a swapped operand."""
    rng = np.random.default_rng(9)
    M, K, N = 150, 13, 21
    A = _grid_exact(rng, M, K, axis=0)
    dY = _grid_exact(rng, M, N, axis=0)
    dW, (Aq2, sA2, cA2), (dYq2, sdY2, cdY2) = O.wgrad(A, dY)
    assert dW.shape == (K, N)
    assert np.array_equal(dW, A.astype(np.float64).T @ dY.astype(np.float64))
    assert Aq2.shape == (K, O.packed_ld(M)) and dYq2.shape == (N, O.packed_ld(M))


def test_wgrad_brute_force_tiny():
    """Tiny wgrad by explicit loops: per-column amax, exactly rounded scales,
    y = RN32(|x| * inv), nearest grid value (ties away), then the exact sum
    over M scaled by both column scales (R2-R4, R10)."""
    rng = np.random.default_rng(10)
    M, K, N = 7, 3, 4
    A = (rng.standard_normal((M, K)) * 3).astype(np.float32)
    dY = (rng.standard_normal((M, N)) * 0.01).astype(np.float32)
    A[2, 1] = 0.0
    dY[:, 3] = 0.0   # an all-zero column: s = 0, codes +-0

    def column_codes(X, j):
        col = X[:, j]
        amax = max(abs(float(v)) for v in col)
        if amax == 0.0:
            return [0.0] * len(col), np.float32(0.0), [(np.signbit(v) << 3) for v in col]
        s = _rn32_fraction(Fraction(amax) / 6)
        inv = _rn32_fraction(6 / Fraction(amax))
        vals, codes = [], []
        for v in col:
            y = np.float32(np.float32(abs(v)) * inv)
            m = int(_brute_nearest(np.array([y], np.float32))[0])
            vals.append((-1.0 if np.signbit(v) else 1.0) * GRID[m])
            codes.append((int(np.signbit(v)) << 3) | m)
        return vals, s, codes

    dW, (_, sA2, cA2), (_, sdY2, cdY2) = O.wgrad(A, dY)
    for k in range(K):
        va, sa, ca = column_codes(A, k)
        assert sA2[k] == sa and list(cA2[k]) == ca, k
        for n in range(N):
            vd, sd, cd = column_codes(dY, n)
            if k == 0:
                assert sdY2[n] == sd and list(cdY2[n]) == cd, n
            acc = sum(Fraction(a) * Fraction(b) for a, b in zip(va, vd))
            assert dW[k, n] == float(acc * Fraction(float(sa)) * Fraction(float(sd))), (k, n)


# ---------------------------------------------------------------------------
# A hand-worked example (values derived by hand from the definitions)
# ---------------------------------------------------------------------------
def test_hand_worked_example():
    A = np.array([[1.0, -3.0, 0.5, 12.0],
                  [-0.25, 2.0, -6.0, 0.0]], dtype=np.float32)
    W = np.array([[1.0, 2.0],
                  [0.5, -1.0],
                  [-2.0, 0.25],
                  [3.0, 0.0]], dtype=np.float32)
    q = 0.75
    # n = 8, k = ceil(6) - 1 = 5; sorted |A| = 0,.25,.5,1,2,3,6,12 -> tau = 3
    Y, ops = O.forward(A, W, q)
    assert ops.k == 5 and ops.tau == 3.0
    # strict clamp: -3.0 (== tau) is not clamped; 12 -> 3 (+9), -6 -> -3 (-3)
    assert list(ops.delta.row) == [0, 1] and list(ops.delta.col) == [3, 2]
    assert list(ops.delta.val32) == [9.0, -3.0]
    assert list(ops.delta.row_ptr) == [0, 1, 2]
    # rows: amax 3 -> s = 0.5, inv = 2; y row0 = 2,6,1,6; row1 = .5,4,6,0
    assert list(ops.sA) == [0.5, 0.5]
    assert ops.codesA.tolist() == [[4, 15, 2, 7], [9, 6, 15, 0]]
    # W col0 amax 3 -> y = 2,1,4,6; col1 amax 2 -> inv = 3, y = 6,3,0.75(tie->1),0
    assert ops.sW[0] == 0.5 and ops.sW[1] == np.float32(1.0 / 3.0)
    assert ops.codesW.tolist() == [[4, 2, 14, 7], [7, 13, 2, 0]]
    # packing: even index in the low nibble, rows padded to 64 bytes
    assert ops.Aq.shape == (2, 64) and ops.Wq.shape == (2, 64)
    assert list(ops.Aq[0, :2]) == [0xF4, 0x72] and list(ops.Aq[1, :2]) == [0x69, 0x0F]
    assert list(ops.Wq[0, :2]) == [0x24, 0x7E] and list(ops.Wq[1, :2]) == [0xD7, 0x02]
    assert not ops.Aq[:, 2:].any() and not ops.Wq[:, 2:].any()
    # acc = [[30, 31], [27, -21]]; Y = acc*sA*sW + dA W
    s1 = float(np.float32(1.0 / 3.0))
    want = np.array([[30 * 0.25 + 27.0, 31 * 0.5 * s1 + 0.0],
                     [27 * 0.25 + 6.0, -21 * 0.5 * s1 - 0.75]])
    assert np.array_equal(Y, want)
    # column 0 is quantized without error, so it equals the exact product
    assert Y[0, 0] == 34.5 and Y[1, 0] == 12.75


def test_pack_layout():
    codes = np.arange(16, dtype=np.uint8)[None, :].repeat(3, axis=0)
    p = O.pack_rows(codes)
    assert p.shape == (3, 64)
    assert list(p[0, :8]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(O.unpack_rows(p, 16), codes)
    assert O.packed_ld(1) == 64 and O.packed_ld(128) == 64 and O.packed_ld(129) == 128


def test_quantile_rank_edges():
    assert O.quantile_rank(8, 0.75) == 5
    assert O.quantile_rank(8, 0.0) == 0
    assert O.quantile_rank(8, 1.0) == 7
    assert O.quantile_rank(1, 0.5) == 0
    assert O.quantile_rank(100, 0.99) == 98
    assert O.quantile_rank(131072, 0.99) == 129761


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.00781250, 3e-39, -0.0],
                                 dtype=np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_golden_tiny_fixture():
    """The oracle still reproduces the frozen tiny-workload fixture."""
    import hashlib
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_forward.json")
    g = json.load(open(path))
    L = wl.make_layer("tiny", seed=0)
    Y, ops = O.forward(L.A.f32, L.W.f32, L.q)
    h = lambda a: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
    assert ops.k == g["k"] and ops.delta.nnz == g["nnz"]
    assert int(np.float32(ops.tau).view(np.uint32)) == g["tau_bits"]
    assert h(ops.Aq) == g["Aq_sha256"] and h(ops.Wq) == g["Wq_sha256"]
    assert h(ops.sA.astype(np.float32)) == g["sA_sha256"]
    assert h(ops.sW.astype(np.float32)) == g["sW_sha256"]
    assert h(ops.delta.row_ptr.astype(np.int32)) == g["row_ptr_sha256"]
    assert h(ops.delta.val32.astype(np.float32)) == g["coo_val32_sha256"]
    assert abs(float(np.linalg.norm(Y)) - g["Y_fro"]) <= 1e-9 * g["Y_fro"]


# ---------------------------------------------------------------------------
# Micro-scaled variant (reading R11; "FP4量化训练的硬件挑战：NVIDIA Blackwell架构上
# 的微缩放格式（Micro-scaling）实现", section 3, and the custom-formats section of
# "训练大型语言模型的挑战": one E8M0 scale per block)
# ---------------------------------------------------------------------------
def test_mx_exponent_closed_forms():
    """e is the least integer >= -127 with 6 * 2^e >= amax: worked by hand."""
    f32 = np.float32
    cases = {
        0.0: -127,                       # empty block: byte 0
        6.0: 0, 12.0: 1, 3.0: -1, 1.5: -2, 0.75: -3,   # exactly 6 * 2^e
        1.0: -2,                         # 6/4 = 1.5 >= 1 > 6/8
        float(np.nextafter(f32(6), f32(7))): 1,
        float(np.nextafter(f32(1.5), f32(2))): -1,
        float(np.nextafter(f32(0), f32(1))): -127,     # smallest subnormal
        float(np.finfo(np.float32).tiny): -127,        # 2^-126 <= 6 * 2^-127
        float(np.finfo(np.float32).max): 126,          # < 2^128 <= 6 * 2^126
        float(f32(2.0 ** 100)): 98,                     # 6 * 2^97 < 2^100 <= 6 * 2^98
    }
    e = O.mx_block_exponents(np.array(list(cases.keys())))
    assert e.tolist() == list(cases.values())
    assert O.mx_scale_bytes(e).tolist() == [v + 127 for v in cases.values()]


def test_mx_exponent_is_least_covering_power():
    """Against the definition by search over every candidate exponent."""
    rng = np.random.default_rng(5)
    amax = np.abs(rng.standard_normal(2000) * np.exp2(rng.integers(-140, 120, 2000))).astype(np.float32)
    e = O.mx_block_exponents(amax.astype(np.float64))
    for a, ei in zip(amax.astype(np.float64), e):
        want = next(c for c in range(-127, 200) if 6.0 * 2.0 ** c >= a)
        assert ei == want


def test_mx_round_trip_exact_on_grid_blocks():
    """Blocks made of grid values times a per-block power of two, each holding
    +-6 * 2^e, decode back exactly, with exponent e."""
    rng = np.random.default_rng(6)
    R, L = 5, 256
    grid = np.array(GRID)
    vals = grid[rng.integers(0, 8, (R, L))] * rng.choice([-1.0, 1.0], (R, L))
    ex = rng.integers(-20, 20, (R, L // 32))
    vals.reshape(R, L // 32, 32)[:, :, 7] = 6.0            # each block reaches 6
    X = (vals.reshape(R, L // 32, 32) * np.exp2(ex)[:, :, None]).reshape(R, L).astype(np.float32)
    codes, e = O.quantize_rows_mx(X)
    assert np.array_equal(e[:, : L // 32], ex)
    back = O.decode(codes).reshape(R, L // 32, 32) * np.exp2(e[:, : L // 32])[:, :, None]
    assert np.array_equal(back.reshape(R, L), X.astype(np.float64))


def test_mx_codes_are_nearest_grid_values():
    """Every code is the nearest grid value of x / 2^e (ties away from zero),
    found by brute-force distance search; the block max lands in (3, 6]."""
    rng = np.random.default_rng(7)
    X = (rng.standard_t(3, (64, 200)) * np.exp2(rng.integers(-30, 30, (64, 1)))).astype(np.float32)
    codes, e = O.quantize_rows_mx(X)
    full = np.zeros((64, 256))
    full[:, :200] = X
    y = np.abs(full.reshape(64, 8, 32)) / np.exp2(e)[:, :, None]
    near = _brute_nearest(y.reshape(64, 256)[:, :200].astype(np.float32))
    assert np.array_equal(codes & 7, near)
    assert np.array_equal(codes >> 3, np.signbit(X).astype(np.uint8))
    bmax = y.max(axis=2)
    live = bmax > 0
    assert np.all((bmax[live] > 3.0) & (bmax[live] <= 6.0))
    assert np.all(e[~live] == -127)
    # x / 2^e is exact: no value of y is rounded
    assert np.array_equal(y * np.exp2(e)[:, :, None], np.abs(full.reshape(64, 8, 32)))


def test_mx_product_equals_dequantized_matmul():
    """The block-scaled sum equals the plain product of the dequantized
    operands (v * 2^e expanded over each block), and a triple loop on a tiny case."""
    rng = np.random.default_rng(8)
    M, N, K = 9, 7, 150
    A = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-8, 8, (M, 1)))).astype(np.float32)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    _, _, ca, ea = O.quantize_act_mx(A)
    _, _, cw, ew = O.quantize_weight_mx(W)
    y, mag = O.mx_product(ca, ea, cw, ew)
    Kp = O.packed_ld(K) * 2
    da = np.zeros((M, Kp)); da[:, :K] = O.decode(ca)
    dw = np.zeros((N, Kp)); dw[:, :K] = O.decode(cw)
    da *= np.repeat(np.exp2(ea), 32, axis=1)
    dw *= np.repeat(np.exp2(ew), 32, axis=1)
    ref = da @ dw.T
    assert np.allclose(y, ref, rtol=1e-13, atol=0)
    assert np.all(mag >= np.abs(y) * (1 - 1e-13))
    for i in (0, 4):
        for j in (0, 6):
            s = sum(Fraction(float(da[i, k])) * Fraction(float(dw[j, k])) for k in range(Kp))
            assert float(s) == pytest.approx(y[i, j], rel=1e-14, abs=1e-300)


def test_mx_unit_scales_reduce_to_integer_product():
    """With every exponent 0 the block-scaled product is the plain integer product."""
    rng = np.random.default_rng(9)
    ca = rng.integers(0, 16, (6, 96)).astype(np.uint8)
    cb = rng.integers(0, 16, (5, 96)).astype(np.uint8)
    nb = O.packed_ld(96) // 16
    y, _ = O.mx_product(ca, np.zeros((6, nb), int), cb, np.zeros((5, nb), int))
    assert np.array_equal(y, O.integer_product(ca, cb))


def test_mx_weight_blocks_run_along_k():
    """W's blocks are 32 consecutive k of one column: scaling one column's
    block by 2^s moves only that block's exponent, by s."""
    rng = np.random.default_rng(10)
    W = rng.standard_normal((100, 6)).astype(np.float32)
    _, sb, c0, e0 = O.quantize_weight_mx(W)
    W2 = W.copy(); W2[32:64, 3] *= np.float32(8.0)
    _, _, c1, e1 = O.quantize_weight_mx(W2)
    diff = e1 - e0
    assert diff[3, 1] == 3 and np.count_nonzero(diff) == 1
    assert np.array_equal(c0, c1)
    assert sb.shape == (6, O.packed_ld(100) // 16)


def _mx_grid_exact(rng, R, C, along_rows):
    """Values that the micro-scaled quantizer keeps exactly: grid values times a
    power of two per 32-block along the reduction, each block reaching 6 * 2^e."""
    grid = np.array(GRID)
    v = grid[rng.integers(0, 8, (R, C))] * rng.choice([-1.0, 1.0], (R, C))
    if along_rows:          # blocks along each row (C is the reduction)
        nb = C // 32
        e = rng.integers(-6, 6, (R, nb))
        v.reshape(R, nb, 32)[:, :, 0] = 6.0
        v = (v.reshape(R, nb, 32) * np.exp2(e)[:, :, None]).reshape(R, C)
    else:                   # blocks along each column (R is the reduction)
        nb = R // 32
        e = rng.integers(-6, 6, (nb, C))
        v.reshape(nb, 32, C)[:, 0, :] = 6.0
        v = (v.reshape(nb, 32, C) * np.exp2(e)[:, None, :]).reshape(R, C)
    return v.astype(np.float32)


def test_mx_dgrad_wgrad_exact_on_grid():
    """On block-exact inputs the micro-scaled backward products equal the plain
    float64 products: dX = dY W^T (blocks along N) and dW = A^T dY (blocks along M)."""
    rng = np.random.default_rng(11)
    M, K, N = 64, 40, 96
    dY = _mx_grid_exact(rng, M, N, along_rows=True)
    W = _mx_grid_exact(rng, K, N, along_rows=True)
    dX, _, _, _ = O.dgrad_mx(dY, W)
    assert np.array_equal(dX, dY.astype(np.float64) @ W.astype(np.float64).T)
    A = _mx_grid_exact(rng, M, K, along_rows=False)
    dY2 = _mx_grid_exact(rng, M, N, along_rows=False)
    dW, _, _, _ = O.wgrad_mx(A, dY2)
    assert np.array_equal(dW, A.astype(np.float64).T @ dY2.astype(np.float64))
    assert dW.shape == (K, N) and dX.shape == (M, K)


# ---------------------------------------------------------------------------
# The micro-scaled whole-layer forward: clamp at tau, block quantization of the
# clamped A, the block-scaled product and the compensation term (reading R11
# with the outlier and compensation paragraphs of the FP4 training write-up)
# ---------------------------------------------------------------------------
def _mx_hand_case():
    """2 x 64 A with two outliers, 64 x 2 W, q = 126/128 (worked in the test)."""
    A = np.zeros((2, 64), np.float32)
    A[0, 0], A[0, 1], A[0, 2], A[0, 40] = 10.0, 1.0, -0.75, 2.5
    A[1, 5], A[1, 33], A[1, 63] = -3.0, 0.625, -7.0
    W = np.zeros((64, 2), np.float32)
    for k, (w0, w1) in {0: (1, 2), 1: (0.5, -1), 2: (2, 0.25), 5: (1, 1), 33: (4, -0.5),
                        40: (-1, 3), 63: (0.5, 2)}.items():
        W[k] = (w0, w1)
    return A, W, 126 / 128


def test_mx_clamped_activation_quantizer_by_hand():
    """quantize_act_mx with tau: the block exponents and codes of the clamped
    rows, worked by hand, and how they differ from the unclamped rows."""
    A, _, _ = _mx_hand_case()
    Aq, sb, codes, e = O.quantize_act_mx(A, np.float32(3.0))
    # clamped row 0, block 0: 10 -> 3, so max 3 = 6 * 2^-1 -> e = -1 and
    # y = 2|x|: 3 -> 6 (mag 7), 1 -> 2 (mag 4), -0.75 -> 1.5 (mag 3, sign set);
    # block 1: max 2.5, 6 * 2^-2 = 1.5 < 2.5 <= 3 -> e = -1, y = 5 ties -> 6
    assert e.tolist() == [[-1, -1, -127, -127], [-1, -1, -127, -127]]
    assert sb.tolist() == [[126, 126, 0, 0], [126, 126, 0, 0]]
    assert codes[0, [0, 1, 2, 40]].tolist() == [7, 4, 11, 7]
    # row 1: -3 (== tau, kept) -> y = 6 -> 15; 0.625 -> y = 1.25 ties -> 1.5
    # (mag 3); -7 -> -3 -> 15
    assert codes[1, [5, 33, 63]].tolist() == [15, 3, 15]
    assert np.count_nonzero(codes) == 7
    assert Aq[0, 0] == 0x47 and Aq[0, 1] == 0x0B and Aq[1, 31] == 0xF0
    # unclamped: block 0 of row 0 has max 10 -> e = 1 (6 < 10 <= 12), y = |x|/2:
    # 10 -> 5 ties -> 6 (7), 1 -> 0.5 (1), -0.75 -> 0.375 -> 0.5 (1, sign set)
    _, sb_u, codes_u, e_u = O.quantize_act_mx(A)
    assert e_u[0, 0] == 1 and sb_u[0, 0] == 128
    assert codes_u[0, [0, 1, 2]].tolist() == [7, 1, 9]
    # row 1 block 1 unclamped: max 7 -> e = 1, 0.625 / 2 = 0.3125 -> 0.5 (1),
    # 7 / 2 = 3.5 ties -> 4 (6)
    assert e_u[1, 1] == 1 and codes_u[1, [33, 63]].tolist() == [1, 14]


def test_mx_forward_hand_worked():
    """The whole micro-scaled forward on the 2 x 64 x 2 case, worked by hand:
    n = 128, k = ceil(126) - 1 = 125; sorted |A| is 121 zeros, .625, .75, 1,
    2.5, 3, 7, 10, so tau = 3 and the clamped set is {10, -7} (strict: -3 stays)."""
    A, W, q = _mx_hand_case()
    Y, mag, tau, delta, qa, qw = O.forward_mx(A, W, q)
    assert tau == 3.0
    assert delta.row.tolist() == [0, 1] and delta.col.tolist() == [0, 63]
    assert delta.val64.tolist() == [7.0, -4.0] and delta.row_ptr.tolist() == [0, 1, 2]
    # W is block-exact: column 0 blocks max 2 (e = -1) and 4 (e = 0); column 1
    # max 2 (e = -1) and 3 (e = -1); every value is a grid value times 2^e
    assert qw[3].tolist() == [[-1, 0, -127, -127], [-1, -1, -127, -127]]
    deq_w = O.decode(qw[2]) * np.repeat(np.exp2(qw[3]), 32, axis=1)[:, :64]
    assert np.array_equal(deq_w.T, W.astype(np.float64))
    # Q(A_c): row 0 = 3 (k0), 1 (k1), -0.75 (k2), 3 (k40, 2.5 rounded up);
    # row 1 = -3 (k5), 0.75 (k33), -3 (k63)
    # Y0 row 0: 3*1 + 1*.5 - .75*2 + 3*(-1) = -1;  3*2 - 1 - .1875 + 9 = 13.8125
    # Y0 row 1: -3 + .75*4 - 3*.5 = -1.5;  -3 - .375 - 6 = -9.375
    # dA W: row 0 += 7 * W[0] = (7, 14); row 1 += -4 * W[63] = (-2, -8)
    assert Y.tolist() == [[6.0, 27.8125], [-3.5, -17.375]]
    # the exact product differs by the roundings 2.5 -> 3 (row 0, times W[40])
    # and 0.625 -> 0.75 (row 1, times W[33])
    exact = A.astype(np.float64) @ W.astype(np.float64)
    assert np.array_equal(exact - Y, np.array([[0.5, -1.5], [-0.5, 0.0625]]))
    assert np.all(mag >= np.abs(Y - np.array([[7.0, 14.0], [-2.0, -8.0]])))


def _mx_block_exact_with_outliers(rng, M, K, n_out):
    """M x K values whose clamp at tau = 6 is block-exact for the micro-scaled
    quantizer: grid values times 2^e per 32-block (e <= 0, so nothing but the
    planted outliers exceeds 6), every block holding +-6 * 2^e, and n_out
    outliers (|a| > 6, dyadic) planted in blocks with e = 0."""
    grid = np.array(GRID)
    nb = K // 32
    v = grid[rng.integers(0, 8, (M, K))] * rng.choice([-1.0, 1.0], (M, K))
    e = rng.integers(-5, 1, (M, nb))
    v.reshape(M, nb, 32)[:, :, 3] = 6.0
    pos = rng.choice(M * K, n_out, replace=False)
    r, c = np.divmod(pos, K)
    e[r, c // 32] = 0                       # outlier blocks clamp to +-6 * 2^0
    v = (v.reshape(M, nb, 32) * np.exp2(e)[:, :, None]).reshape(M, K)
    out = (6.0 + rng.integers(1, 400, n_out) / 4.0) * rng.choice([-1.0, 1.0], n_out)
    keep = (c % 32) != 3                    # never overwrite a block's +-6 anchor
    v[r[keep], c[keep]] = out[keep]
    return v.astype(np.float32), int(keep.sum())


@pytest.mark.parametrize("M,K,N,n_out", [(16, 96, 40, 9), (40, 256, 24, 30)])
def test_mx_forward_exact_on_block_exact_clamp(M, K, N, n_out):
    """With tau = 6 placed by q and A_clamped block-exact, Q(A_clamped) is
    A_clamped and Q(W) is W, so Y = A_c W + dA W = A W exactly. Quantizing the
    unclamped A, a tau that differs between the clamp and dA, a dropped or
    negated dA, or a transposed operand each break the equality."""
    rng = np.random.default_rng(M + K + N)
    A, n_clamped = _mx_block_exact_with_outliers(rng, M, K, n_out)
    W = _mx_grid_exact(rng, K, N, along_rows=False)
    n = M * K
    q = (n - n_clamped) / n                 # k = n - n_clamped - 1: the largest |a| <= 6
    Y, _, tau, delta, qa, _ = O.forward_mx(A, W, q)
    assert tau == 6.0
    big = np.abs(A) > 6.0
    assert delta.nnz == n_clamped == int(big.sum())
    assert np.array_equal(delta.row * K + delta.col, np.flatnonzero(big))
    # every outlier block's exponent is that of the clamped block (0), not of
    # the outlier (e >= 1)
    assert np.all(qa[3][np.nonzero(big)[0], np.nonzero(big)[1] // 32] == 0)
    assert np.array_equal(Y, A.astype(np.float64) @ W.astype(np.float64))
    # the clamp matters: without it the outlier blocks get coarser exponents
    Y_noclamp, *_ = O.forward_mx(A, W, 1.0)
    assert not np.array_equal(Y_noclamp, Y)


def test_mx_forward_q1_block_exact_is_plain_product():
    """q = 1 clamps nothing (tau = max |a|, dA empty): block-exact A and W give
    Y = A W exactly, on a non-square shape with a ragged K."""
    rng = np.random.default_rng(12)
    M, K, N = 24, 160, 36
    A = _mx_grid_exact(rng, M, K, along_rows=True)
    W = _mx_grid_exact(rng, K, N, along_rows=False)
    Y, _, tau, delta, _, _ = O.forward_mx(A, W, 1.0)
    assert delta.nnz == 0 and tau == np.abs(A).max()
    assert np.array_equal(Y, A.astype(np.float64) @ W.astype(np.float64))
