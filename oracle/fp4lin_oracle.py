"""CPU oracle for the FP4 quantized linear layer forward (and its dgrad GEMM).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module. The library
(``quantized_linear_layer_amd``) never calls it and shares no code with it.

It is deliberately plain and slow: numpy with float64 wherever a real number is
formed, no blocking or fusion, each step in the order the method states it.

Sources (cited by page title and passage; the pages have no numbered sections):
  [FP4-news]  "微软首创FP4训练框架，训练效果媲美BF16，助力大模型训练更高效"
              (news.movedaos.com write-up of arXiv 2501.17116). Passages used:
              - the FP4 format paragraph (E2M1: 2 exponent, 1 mantissa, 1 sign bit);
              - the granularity paragraph (W quantized per column / channel-wise,
                A per row / token-wise, matched to the GEMM so no transpose);
              - the forward-start paragraph (W and A quantized when each
                linear layer's forward begins);
              - the rounding paragraph (scale + shift into the FP4 range, then
                round to the nearest FP4 value by table lookup);
              - the ScaleShift paragraph (scale to [-1,1], then shift to the
                FP4 range);
              - the outlier paragraph (quantile search finds the largest-magnitude
                entries of A, they are clamped to a threshold giving A_clamped)
                and the compensation paragraph (sparse Delta A = A - A_clamped,
                non-zero only where clamping happened).
  [FP4-abs]   "Optimizing Large Language Model Training Using FP4 Quantization"
              (chatpaper.ai), the abstract: outlier clamping and compensation,
              vector-wise quantization.

Readings where the pages are silent (each is listed in the design notes):
  R1  E2M1 grid: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}; the 3-bit magnitude code is the
      grid index, bit 3 is the sign (sign-magnitude).
  R2  ScaleShift: amax = max |x| over the vector; inv = RN32(6/amax) once per
      vector; y = RN32(|x| * inv) per element; stored scale s = RN32(amax/6).
      "Shift" is read as the multiplicative map of [-1,1] onto [-6,6]; no
      additive offset.
  R3  Round to nearest, ties away from zero: the magnitude code is the number of
      midpoints {0.25,0.75,1.25,1.75,2.5,3.5,5} that y reaches (y >= t). y > 6
      saturates to 6. NaN y (0*Inf when amax = 0) reaches no midpoint -> 0.
  R4  The sign bit is signbit(x): -0 and negative values that round to 0 get 0b1000.
  R5  Quantile: tau is the k-th smallest |a| (0-based) over all M*K entries,
      k = clamp(ceil(q*n) - 1, 0, n-1) evaluated in IEEE double.
  R6  Clamped set C = {|a| > tau} (strict). Delta A holds RN32(a - sign(a)*tau)
      on C, listed in row-major order, with row_ptr[M+1].
  R7  Packing: two codes per byte, the even index in the low nibble; each row
      padded with zero codes to a multiple of 128 codes (row stride
      roundup(L,128)/2 bytes). W is packed N-major (one packed row per output
      column).
  R8  Y = RN32(RN32(acc*s_A[i])*s_W[j]) + sum_k dA[i,k]*W[k,j]; the oracle keeps
      every step in float64 and compares by relative Frobenius error.
  R9  dgrad dX = Q(dY) Q(W)^T: dY quantized per row over N (no clamp), W
      re-quantized per row over N so that its scale leaves the reduction.
  R10 wgrad dW = Q(A)^T Q(dY): A and dY both quantized per column over M (the
      reduction), with no clamp and no compensation term, so that both scales
      leave the reduction; the channel-wise quantizer of W applied to A and dY.
  R11 Micro-scaled variant ([mx] section 3: groups with one scale each taken
      from the group's max, elements divided by it and rounded to FP4;
      [survey] custom-formats section: one E8M0 scale per block beside
      low-precision elements). Blocks are 32 consecutive elements along the
      reduction (K): per row of A, per column of W. A block's scale is 2^e
      with e the smallest integer >= -127 for which 6 * 2^e >= the block's
      max |x| (the max lands inside the FP4 range, none is clipped, and E8M0
      holds only powers of two); it is stored as the byte e + 127. Elements
      are y = |x| / 2^e (exact) rounded as in R3/R4. A is clamped to +-tau
      first, as in the forward. Padding elements are zero; an all-zero block
      has e = -127. Y0[i,j] = sum over blocks b of
      2^(eA[i,b] + eW[j,b]) * sum_{k in b} v(qa[i,k]) v(qw[j,k]), with no
      separate scale epilogue, and Y = Y0 + Delta A . W.

Page tags: [news] "微软首创FP4训练框架，训练效果媲美BF16，助力大模型训练更高效";
[mx] "FP4量化训练的硬件挑战：NVIDIA Blackwell架构上的微缩放格式（Micro-scaling）实现";
[survey] "训练大型语言模型的挑战".
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# [FP4-news], FP4 format paragraph; grid values per reading R1.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
# Midpoints between neighbouring magnitudes (reading R3).
E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
FP4_MAX = 6.0
PACK_ALIGN = 128  # codes per padded row unit (reading R7)


# --------------------------------------------------------------------------
# Rank and threshold ([FP4-news] outlier paragraph; reading R5)
# --------------------------------------------------------------------------
def quantile_rank(n: int, q: float) -> int:
    """0-based rank of the clamp threshold among the n values of |A|."""
    if n <= 0:
        raise ValueError("n must be positive")
    k = math.ceil(float(q) * float(n)) - 1
    return int(min(max(k, 0), n - 1))


def select_threshold(A32: np.ndarray, q: float):
    """tau = k-th smallest |a| over the whole tensor (an element of |A|)."""
    absA = np.abs(np.asarray(A32, dtype=np.float32)).ravel()
    k = quantile_rank(absA.size, q)
    tau = np.partition(absA, k)[k]
    return np.float32(tau), k


# --------------------------------------------------------------------------
# Clamp and sparse compensation ([FP4-news] outlier and compensation
# paragraphs; reading R6)
# --------------------------------------------------------------------------
@dataclasses.dataclass
class SparseDelta:
    row: np.ndarray      # int32, row-major order
    col: np.ndarray      # int32
    val32: np.ndarray    # float32, RN32(a - sign(a) tau)
    val64: np.ndarray    # float64, a - sign(a) tau (exact for the test data)
    row_ptr: np.ndarray  # int32, M+1
    shape: tuple

    @property
    def nnz(self) -> int:
        return int(self.row.size)

    def dense64(self) -> np.ndarray:
        d = np.zeros(self.shape, dtype=np.float64)
        d[self.row, self.col] = self.val64
        return d


def clamp_and_residual(A32: np.ndarray, tau: np.float32):
    """Return (A_clamped float32, SparseDelta)."""
    A32 = np.asarray(A32, dtype=np.float32)
    M, K = A32.shape
    tau = np.float32(tau)
    C = np.abs(A32) > tau
    rows, cols = np.nonzero(C)          # row-major order
    a64 = A32[rows, cols].astype(np.float64)
    # a - sign(a)*tau; float64 difference of two float32 values, then rounded
    # once more to float32 (correctly rounded: 53 >= 2*24 + 2).
    d64 = a64 - np.sign(a64) * np.float64(tau)
    val32 = d64.astype(np.float32)
    A_c = np.where(C, np.copysign(np.float32(tau), A32), A32).astype(np.float32)
    counts = np.bincount(rows, minlength=M) if rows.size else np.zeros(M, np.int64)
    row_ptr = np.zeros(M + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    delta = SparseDelta(rows.astype(np.int32), cols.astype(np.int32), val32, d64,
                        row_ptr.astype(np.int32), (M, K))
    return A_c, delta


# --------------------------------------------------------------------------
# ScaleShift quantizer ([FP4-news] rounding and ScaleShift paragraphs;
# readings R1-R4)
# --------------------------------------------------------------------------
def encode_magnitude(y32: np.ndarray) -> np.ndarray:
    """3-bit E2M1 magnitude code of float32 y >= 0 (or NaN): midpoints reached."""
    y32 = np.asarray(y32, dtype=np.float32)
    m = np.zeros(y32.shape, dtype=np.uint8)
    with np.errstate(invalid="ignore"):
        for t in E2M1_MIDPOINTS:
            m += (y32 >= t).astype(np.uint8)
    return m


def vector_scales(amax32: np.ndarray):
    """Per-vector (stored scale s, encode multiplier inv), both float32."""
    a64 = np.asarray(amax32, dtype=np.float32).astype(np.float64)
    with np.errstate(divide="ignore", over="ignore"):
        s = (a64 / FP4_MAX).astype(np.float32)
        inv = (FP4_MAX / a64).astype(np.float32)
    return s, inv


def quantize_rows(X32: np.ndarray):
    """Token-wise quantization: one scale per row. Returns (codes uint8 MxL, s float32 M)."""
    X32 = np.asarray(X32, dtype=np.float32)
    absX = np.abs(X32)
    amax = absX.max(axis=1) if X32.shape[1] else np.zeros(X32.shape[0], np.float32)
    s, inv = vector_scales(amax)
    with np.errstate(invalid="ignore", over="ignore"):
        y = absX * inv[:, None]          # one float32 multiply, round-to-nearest-even
    mag = encode_magnitude(y)
    sign = np.signbit(X32).astype(np.uint8)
    return (sign << 3) | mag, s


def quantize_cols(X32: np.ndarray):
    """Channel-wise quantization: one scale per column. Returns (codes KxN, s N)."""
    codes_t, s = quantize_rows(np.asarray(X32, dtype=np.float32).T)
    return codes_t.T, s


def decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E2M1 code as float64."""
    codes = np.asarray(codes, dtype=np.uint8)
    v = E2M1_MAGNITUDES[codes & 7]
    return np.where(codes & 8, -v, v)


def packed_ld(L: int) -> int:
    """Bytes per packed row of L codes."""
    return ((int(L) + PACK_ALIGN - 1) // PACK_ALIGN) * PACK_ALIGN // 2


def pack_rows(codes: np.ndarray) -> np.ndarray:
    """Pack a rows x L code matrix, even index in the low nibble, zero padded."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, L = codes.shape
    Lp = packed_ld(L) * 2
    full = np.zeros((R, Lp), dtype=np.uint8)
    full[:, :L] = codes
    return (full[:, 0::2] | (full[:, 1::2] << 4)).astype(np.uint8)


def unpack_rows(packed: np.ndarray, L: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out[:, :L]


# --------------------------------------------------------------------------
# The three library operations, each as the oracle defines it
# --------------------------------------------------------------------------
def quantize_act(X32: np.ndarray, tau=None):
    """Token-wise quantization of (optionally clamped) activations.

    Returns (packed codes M x packed_ld(K), s float32 M, unpacked codes)."""
    X32 = np.asarray(X32, dtype=np.float32)
    if tau is not None:
        tau = np.float32(tau)
        X32 = np.where(np.abs(X32) > tau, np.copysign(tau, X32), X32).astype(np.float32)
    codes, s = quantize_rows(X32)
    return pack_rows(codes), s, codes


def quantize_weight(W32: np.ndarray):
    """Channel-wise quantization of a K x N weight, packed N-major.

    Returns (packed N x packed_ld(K), s float32 N, codes N x K)."""
    codes_kn, s = quantize_cols(np.asarray(W32, dtype=np.float32))
    codes_nk = np.ascontiguousarray(codes_kn.T)
    return pack_rows(codes_nk), s, codes_nk


def integer_product(codesA: np.ndarray, codesB_nmajor: np.ndarray) -> np.ndarray:
    """acc[i,j] = sum_k v(A[i,k]) v(B[j,k]), exact in float64.

    2*v is an integer in [-12,12] and |sum| <= 144*K < 2**53, so the float64
    matrix product is exact whatever order BLAS uses."""
    a2 = 2.0 * decode(codesA)
    b2 = 2.0 * decode(codesB_nmajor)
    return (a2 @ b2.T) / 4.0


def scaled_product(acc: np.ndarray, sA: np.ndarray, sB: np.ndarray) -> np.ndarray:
    """(s_A (x) rows) . acc . (s_B (x) cols) in float64."""
    return acc * np.asarray(sA, np.float64)[:, None] * np.asarray(sB, np.float64)[None, :]


def sparse_times_dense(delta: SparseDelta, W64: np.ndarray, use64: bool = True) -> np.ndarray:
    """Delta A . W as a plain scatter-accumulate over the non-zeros, float64."""
    M = delta.shape[0]
    W64 = np.asarray(W64, dtype=np.float64)
    out = np.zeros((M, W64.shape[1]), dtype=np.float64)
    vals = delta.val64 if use64 else delta.val32.astype(np.float64)
    # group by row (already row-major) and accumulate each row's terms
    for i in range(M):
        lo, hi = int(delta.row_ptr[i]), int(delta.row_ptr[i + 1])
        if hi > lo:
            out[i] = vals[lo:hi] @ W64[delta.col[lo:hi]]
    return out


@dataclasses.dataclass
class ForwardResult:
    k: int
    tau: np.float32
    delta: SparseDelta
    Aq: np.ndarray        # packed, M x packed_ld(K)
    sA: np.ndarray
    codesA: np.ndarray
    Wq: np.ndarray        # packed, N x packed_ld(K)
    sW: np.ndarray
    codesW: np.ndarray    # N x K
    A_c: np.ndarray


def forward_operands(A32: np.ndarray, W32: np.ndarray, q: float) -> ForwardResult:
    """Every intermediate of the forward, in the order the method applies them:
    threshold, clamp + Delta A, token-wise A quantization, channel-wise W."""
    tau, k = select_threshold(A32, q)
    A_c, delta = clamp_and_residual(A32, tau)
    Aq, sA, codesA = quantize_act(A32, tau)
    Wq, sW, codesW = quantize_weight(W32)
    return ForwardResult(k, tau, delta, Aq, sA, codesA, Wq, sW, codesW, A_c)


def forward_output(ops: ForwardResult, W32: np.ndarray, rows=None) -> np.ndarray:
    """Y (float64) for all rows, or for the listed rows only."""
    if rows is None:
        rows = np.arange(ops.codesA.shape[0])
    rows = np.asarray(rows)
    acc = integer_product(ops.codesA[rows], ops.codesW)
    y = scaled_product(acc, ops.sA[rows], ops.sW)
    d = ops.delta
    W64 = np.asarray(W32, dtype=np.float64)
    for t, i in enumerate(rows):
        lo, hi = int(d.row_ptr[i]), int(d.row_ptr[i + 1])
        if hi > lo:
            y[t] += d.val64[lo:hi] @ W64[d.col[lo:hi]]
    return y


def forward(A32: np.ndarray, W32: np.ndarray, q: float):
    """Full forward Y = (s_A . Q(A_c)) (Q(W) . s_W) + Delta A . W in float64."""
    ops = forward_operands(A32, W32, q)
    return forward_output(ops, W32), ops


def dgrad(dY32: np.ndarray, W32: np.ndarray, rows=None):
    """dX = Q(dY) Q(W)^T with dY and W both quantized per row over N (reading R9).

    Returns (dX float64, (dYq, s_dY, codes_dY), (Wq', s_W', codes_W'))."""
    dYq, s_dy, c_dy = quantize_act(dY32, None)
    Wq2, s_w2, c_w2 = quantize_act(W32, None)
    if rows is None:
        rows = np.arange(c_dy.shape[0])
    acc = integer_product(c_dy[rows], c_w2)
    return scaled_product(acc, s_dy[rows], s_w2), (dYq, s_dy, c_dy), (Wq2, s_w2, c_w2)


def wgrad(A32: np.ndarray, dY32: np.ndarray, rows=None):
    """dW = Q(A)^T Q(dY) with A (M x K) and dY (M x N) quantized per column over
    M (reading R10): the weight quantizer applied to A and to dY gives both
    operands packed along M, one packed row per column of A or dY.

    Returns (dW float64 K x N, or its listed rows, (Aq', s_A', codes_A' K x M),
    (dYq', s_dY', codes_dY' N x M))."""
    Aq2, s_a2, c_a2 = quantize_weight(A32)
    dYq2, s_dy2, c_dy2 = quantize_weight(dY32)
    if rows is None:
        rows = np.arange(c_a2.shape[0])
    acc = integer_product(c_a2[rows], c_dy2)
    return scaled_product(acc, s_a2[rows], s_dy2), (Aq2, s_a2, c_a2), (dYq2, s_dy2, c_dy2)


# --------------------------------------------------------------------------
# Micro-scaled variant ([mx] section 3, the principle and the steps of
# micro-scaling; [survey] custom-formats section, per-block E8M0 scales;
# reading R11)
# --------------------------------------------------------------------------
MX_BLOCK = 32          # elements per block along the reduction
E8M0_BIAS = 127
E8M0_MIN_EXP = -127    # byte 0


def mx_block_exponents(amax) -> np.ndarray:
    """Smallest integer e >= -127 with 6 * 2**e >= amax, elementwise (amax >= 0)."""
    a = np.asarray(amax, dtype=np.float64)
    e = np.full(a.shape, E8M0_MIN_EXP, dtype=np.int64)
    nz = a > 0
    with np.errstate(divide="ignore"):
        guess = np.ceil(np.log2(np.where(nz, a, 1.0) / FP4_MAX)).astype(np.int64)
    e = np.where(nz, guess, e)
    # log2 is rounded: move to the exact boundary (6 * 2**e is exact in float64)
    for _ in range(3):
        e = np.where(nz & (np.ldexp(FP4_MAX, e) < a), e + 1, e)
    for _ in range(3):
        e = np.where(nz & (np.ldexp(FP4_MAX, e - 1) >= a), e - 1, e)
    return np.maximum(e, E8M0_MIN_EXP)


def quantize_rows_mx(X32: np.ndarray):
    """Blocks of 32 along each row. Returns (codes uint8 R x L, exponents
    int64 R x (packed_ld(L)/16)); the blocks cover the zero padding too."""
    X32 = np.asarray(X32, dtype=np.float32)
    R, L = X32.shape
    Lp = packed_ld(L) * 2
    full = np.zeros((R, Lp), dtype=np.float64)
    full[:, :L] = X32
    nb = Lp // MX_BLOCK
    blocks = np.abs(full).reshape(R, nb, MX_BLOCK)
    e = mx_block_exponents(blocks.max(axis=2))
    y = np.ldexp(blocks, -e[:, :, None]).reshape(R, Lp)[:, :L]   # exact
    mag = np.zeros((R, L), dtype=np.uint8)
    for t in E2M1_MIDPOINTS.astype(np.float64):
        mag += (y >= t).astype(np.uint8)
    sign = np.signbit(X32).astype(np.uint8)
    return (sign << 3) | mag, e


def mx_scale_bytes(e: np.ndarray) -> np.ndarray:
    """E8M0 byte of each block exponent."""
    return (np.asarray(e, dtype=np.int64) + E8M0_BIAS).astype(np.uint8)


def quantize_act_mx(X32: np.ndarray, tau=None):
    """Micro-scaled quantization of (optionally clamped) activations.

    Returns (packed codes M x packed_ld(K), scale bytes M x packed_ld(K)/16,
    codes M x K, exponents)."""
    X32 = np.asarray(X32, dtype=np.float32)
    if tau is not None:
        tau = np.float32(tau)
        X32 = np.where(np.abs(X32) > tau, np.copysign(tau, X32), X32).astype(np.float32)
    codes, e = quantize_rows_mx(X32)
    return pack_rows(codes), mx_scale_bytes(e), codes, e


def quantize_weight_mx(W32: np.ndarray):
    """Micro-scaled quantization of a K x N weight along K, packed N-major.

    Returns (packed N x packed_ld(K), scale bytes N x packed_ld(K)/16,
    codes N x K, exponents)."""
    codes_nk, e = quantize_rows_mx(np.ascontiguousarray(np.asarray(W32, dtype=np.float32).T))
    return pack_rows(codes_nk), mx_scale_bytes(e), codes_nk, e


def mx_product(codesA, eA, codesB_nmajor, eB):
    """Y0[i,j] = sum_b 2^(eA[i,b]+eB[j,b]) sum_{k in b} v(A[i,k]) v(B[j,k]).

    Each block's sum is exact in float64 (integers / 4); the blocks are added
    in ascending order. Returns (Y0, sum over blocks of |term|), both float64."""
    codesA = np.asarray(codesA, dtype=np.uint8)
    codesB = np.asarray(codesB_nmajor, dtype=np.uint8)
    K = codesA.shape[1]
    Kp = packed_ld(K) * 2
    a2 = np.zeros((codesA.shape[0], Kp))
    b2 = np.zeros((codesB.shape[0], Kp))
    a2[:, :K] = 2.0 * decode(codesA)
    b2[:, :K] = 2.0 * decode(codesB)
    y = np.zeros((a2.shape[0], b2.shape[0]))
    mag = np.zeros_like(y)
    for b in range(Kp // MX_BLOCK):
        blk = slice(b * MX_BLOCK, (b + 1) * MX_BLOCK)
        acc = (a2[:, blk] @ b2[:, blk].T) / 4.0
        term = np.ldexp(acc, np.asarray(eA)[:, b][:, None] + np.asarray(eB)[:, b][None, :])
        y += term
        mag += np.abs(term)
    return y, mag


def forward_mx(A32: np.ndarray, W32: np.ndarray, q: float, rows=None):
    """Micro-scaled forward Y = Q_mx(A_c) Q_mx(W) + Delta A . W (reading R11).

    Returns (Y float64 for all or the listed rows, |term| sums, tau, delta,
    (Aq, As, codesA, eA), (Wq, Ws, codesW, eW))."""
    tau, _ = select_threshold(A32, q)
    _, delta = clamp_and_residual(A32, tau)
    qa = quantize_act_mx(A32, tau)
    qw = quantize_weight_mx(W32)
    if rows is None:
        rows = np.arange(qa[2].shape[0])
    rows = np.asarray(rows)
    y, mag = mx_product(qa[2][rows], qa[3][rows], qw[2], qw[3])
    W64 = np.asarray(W32, dtype=np.float64)
    for t, i in enumerate(rows):
        lo, hi = int(delta.row_ptr[i]), int(delta.row_ptr[i + 1])
        if hi > lo:
            y[t] += delta.val64[lo:hi] @ W64[delta.col[lo:hi]]
    return y, mag, tau, delta, qa, qw


def dgrad_mx(dY32: np.ndarray, W32: np.ndarray, rows=None):
    """Micro-scaled dX = Q(dY) Q(W)^T: dY and W both in blocks of 32 along N,
    the reduction (readings R9 and R11), no clamp.

    Returns (dX float64 or its listed rows, |term| sums, dY's and W's
    (packed, scale bytes, codes, exponents))."""
    qd = quantize_act_mx(dY32, None)
    qw = quantize_act_mx(W32, None)
    if rows is None:
        rows = np.arange(qd[2].shape[0])
    y, mag = mx_product(qd[2][rows], qd[3][rows], qw[2], qw[3])
    return y, mag, qd, qw


def wgrad_mx(A32: np.ndarray, dY32: np.ndarray, rows=None):
    """Micro-scaled dW = Q(A)^T Q(dY): A and dY both in blocks of 32 along M,
    the reduction (readings R10 and R11), no clamp.

    Returns (dW float64 K x N or its listed rows, |term| sums, A's and dY's
    (packed, scale bytes, codes, exponents), each packed along M)."""
    qa = quantize_weight_mx(A32)
    qd = quantize_weight_mx(dY32)
    if rows is None:
        rows = np.arange(qa[2].shape[0])
    y, mag = mx_product(qa[2][rows], qa[3][rows], qd[2], qd[3])
    return y, mag, qa, qd


def rel_fro(x: np.ndarray, ref: np.ndarray) -> float:
    """Relative Frobenius error ||x - ref|| / ||ref|| (0 when both are zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
