// Micro-scaled (MXFP4) quantization: E2M1 codes in blocks of 32 consecutive
// elements along the reduction dimension K, one power-of-two scale per block
// stored as an E8M0 byte.
//
// Method: the micro-scaling lecture ("FP4量化训练的硬件挑战：NVIDIA Blackwell架构上
// 的微缩放格式（Micro-scaling）实现", section 3) splits a tensor into small groups,
// gives each group its own scale taken from the group's maximum magnitude,
// divides the elements by it and rounds them to FP4; the survey of number
// formats ("训练大型语言模型的挑战", custom-formats section) pairs such blocks with
// an E8M0 scale. A block's scale is 2^e with e the least integer >= -127 for
// which 6 * 2^e covers the block's max |x| (so nothing is clipped), stored as
// e + 127; each element is y = |x| / 2^e, exact, rounded to the nearest E2M1
// value with ties away from zero, as in the token-wise quantizer. Activations
// are clamped to +-tau first. The GEMM takes the bytes as the matrix core's
// block-scale operands (gemm.hip).
//
// Scale layout (step-major): for each K step of 128 codes, one 32-bit word per
// row (per column of W) holds the bytes of its blocks 4s .. 4s+3, low byte
// first, and the words of consecutive rows are adjacent: the byte of block b
// of row i (of R rows) is at (b / 4) * 4R + 4i + b % 4. The GEMM then reads the
// scales of 64 consecutive rows for one step as 256 contiguous bytes.
//
// The block exponent and the element encoder (mx_exponent, mx_magnitude) are
// in device_common.hpp, shared with the forward's compaction kernel, which
// block-quantizes the rows of A it already holds; the column pass is
// quantize_cols_mx_body (colquant.hpp), which the forward pairs with the
// select's row count.
//
// Rows (activations): one thread per 8-code chunk of a padded row, so four
//   consecutive lanes hold one block and its max is two lane exchanges away;
//   each thread writes its 8 codes as one 32-bit word and the first lane of a
//   block writes the scale byte. No block needs more than its own 32 values, so
//   rows of any length stream through once.
// Columns (weights, K x N row-major): the 128 x 128 tiles of the channel-wise
//   encode pass; a thread holds 8 consecutive rows of 8 columns, so the four
//   lanes with the same columns and consecutive row groups hold one block of
//   each of those columns.
#include "colquant.hpp"
#include "device_common.hpp"
#include "internal.hpp"

namespace fp4lin {

namespace {

constexpr int kMxThreads = 256;

// Workgroup (bx, by) takes rows by, by + gridDim.y, ... and in each the chunks
// c = bx * 256 + t, c + 256 * gridDim.x, ... (cpr = ldq / 4 chunks of 8 codes
// per padded row, a multiple of 16). Four consecutive t hold one block and sit
// on four consecutive lanes, and the chunk stride is a multiple of 4, so a
// block's lanes are active together.
template <class In, bool kFast>
__global__ __launch_bounds__(kMxThreads) void quantize_rows_mx_kernel(
    const typename In::T* __restrict__ X, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ tau_p, uint8_t* __restrict__ Xq, int64_t ldq,
    uint8_t* __restrict__ Xs) {
  const float tau = tau_p ? *tau_p : __builtin_huge_valf();
  const int64_t cpr = ldq / 4;
  for (int64_t r = blockIdx.y; r < M; r += gridDim.y)
  for (int64_t c = int64_t(blockIdx.x) * kMxThreads + threadIdx.x; c < cpr;
       c += int64_t(gridDim.x) * kMxThreads) {
    Vec8<In> v;
    load_chunk<In, kFast>(X + r * ldx, c * 8, K, v);
    float ax[8];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ax[i] = fminf(fabsf(In::widen(v.v[i])), tau);
      m = fmaxf(m, ax[i]);
    }
    const int e = mx_exponent(quad_max(m));
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      word |= (mx_magnitude(ax[i], e) | (In::sign_bit(v.v[i]) << 3)) << (4 * i);
    *reinterpret_cast<uint32_t*>(Xq + r * ldq + c * 4) = word;
    // chunk c: block c / 4 = 4 * (c / 16) + (c / 4) % 4
    if ((c & 3) == 0) Xs[(c / 16) * 4 * M + 4 * r + ((c / 4) & 3)] = uint8_t(e + 127);
  }
}

// One workgroup per 128 x 128 tile of W (quantize_cols_mx_body).
template <class In, bool kAligned>
__global__ __launch_bounds__(kMxThreads) void quantize_cols_mx_kernel(
    const typename In::T* __restrict__ W, int64_t K, int64_t N, int64_t ldw,
    uint8_t* __restrict__ Wq, int64_t ldq, uint8_t* __restrict__ Ws) {
  quantize_cols_mx_body<In, kAligned>(blockIdx.x, blockIdx.y, W, K, N, ldw, Wq, ldq, Ws);
}

// chunks of a row across x (at most 64 workgroups), rows across y (at most 65535)
dim3 mx_row_grid(int64_t M, int64_t cpr) {
  const int64_t bx = (cpr + kMxThreads - 1) / kMxThreads;
  return dim3(unsigned(bx < 64 ? bx : 64), unsigned(M < 65535 ? M : 65535));
}

template <class In>
hipError_t run_rows_mx(const void* X, int64_t M, int64_t K, int64_t ldx, const float* tau,
                       uint8_t* Xq, int64_t ldq, uint8_t* Xs, hipStream_t stream) {
  using T = typename In::T;
  const T* x = static_cast<const T*>(X);
  const bool fast = (reinterpret_cast<uintptr_t>(X) % 16 == 0) &&
                    ((ldx * In::kBytes) % 16 == 0) && (K % 8 == 0);
  const dim3 grid = mx_row_grid(M, ldq / 4);
  if (fast)
    quantize_rows_mx_kernel<In, true><<<grid, kMxThreads, 0, stream>>>(x, M, K, ldx, tau, Xq, ldq,
                                                                       Xs);
  else
    quantize_rows_mx_kernel<In, false><<<grid, kMxThreads, 0, stream>>>(x, M, K, ldx, tau, Xq,
                                                                        ldq, Xs);
  return hipGetLastError();
}

template <class In>
hipError_t run_cols_mx(const void* Wp, int64_t K, int64_t N, int64_t ldw, uint8_t* Wq,
                       int64_t ldq, uint8_t* Ws, hipStream_t stream) {
  using T = typename In::T;
  const T* W = static_cast<const T*>(Wp);
  const bool aligned = (reinterpret_cast<uintptr_t>(Wp) % 16 == 0) &&
                       ((ldw * In::kBytes) % 16 == 0);
  const dim3 grid(unsigned((N + kMxTN - 1) / kMxTN), unsigned((ldq * 2) / kMxTK));
  if (aligned)
    quantize_cols_mx_kernel<In, true><<<grid, kMxThreads, 0, stream>>>(W, K, N, ldw, Wq, ldq, Ws);
  else
    quantize_cols_mx_kernel<In, false><<<grid, kMxThreads, 0, stream>>>(W, K, N, ldw, Wq, ldq,
                                                                        Ws);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows_mx(const void* X, bool bf16, int64_t M, int64_t K, int64_t ldx,
                                   const float* tau, uint8_t* Xq, int64_t ldq, uint8_t* Xs,
                                   hipStream_t stream) {
  return bf16 ? run_rows_mx<BF16In>(X, M, K, ldx, tau, Xq, ldq, Xs, stream)
              : run_rows_mx<F32In>(X, M, K, ldx, tau, Xq, ldq, Xs, stream);
}

hipError_t launch_quantize_cols_mx(const void* W, bool bf16, int64_t K, int64_t N, int64_t ldw,
                                   uint8_t* Wq, int64_t ldq, uint8_t* Ws, hipStream_t stream) {
  return bf16 ? run_cols_mx<BF16In>(W, K, N, ldw, Wq, ldq, Ws, stream)
              : run_cols_mx<F32In>(W, K, N, ldw, Wq, ldq, Ws, stream);
}

}  // namespace fp4lin
