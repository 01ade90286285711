// Launchers behind the C ABI. Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp4lin {

size_t select_workspace_bytes(bool bf16, int64_t M);
size_t weight_workspace_bytes(int64_t N);

// The two passes of launch_quantize_weight for bf16 W with 16-byte aligned rows,
// with colmax (N words) already zero.
hipError_t launch_quantize_weight_cleared(const uint16_t* W, int64_t K, int64_t N, int64_t ldw,
                                          uint8_t* Wq, int64_t ldq, float* sW, uint32_t* colmax,
                                          hipStream_t stream);

// With quantized set, rows that allow it are also quantized token-wise (Xq
// with row stride ldq, scales sX, clamped to tau) by the compaction, and
// *quantized says whether that happened; with quantized null, Xq is ignored.
// With Xs set, that quantization is the micro-scaled one instead (block
// scales into the step-major array Xs; sX unused).
hipError_t launch_outlier_select(const void* A, bool bf16, int64_t M, int64_t K, int64_t lda,
                                 int64_t k, float* tau, int64_t capacity, int32_t* row,
                                 int32_t* col, float* val, int32_t* row_ptr, void* ws,
                                 hipStream_t stream, uint8_t* Xq = nullptr, int64_t ldq = 0,
                                 float* sX = nullptr, bool* quantized = nullptr,
                                 uint8_t* Xs = nullptr);

// Whole-layer forward, front half (select, quantization of A and of W) for
// bf16 A and W with 16-byte aligned rows, K % 8 == 0 and K up to 8192
// (forward_front_supported): the select of launch_outlier_select with the
// token-wise quantization of A in its compaction; colmax (N words of
// workspace apart from ws) is cleared by the select's first pass. For K up to
// 4096 the channel-wise quantization of W shares launches with the select's
// row kernels and *w_done is set; otherwise the caller runs
// launch_quantize_weight_cleared.
bool forward_front_supported(const void* A, const void* W, bool bf16, int64_t K, int64_t lda,
                             int64_t ldw);
hipError_t launch_forward_front(const void* A, int64_t M, int64_t K, int64_t lda, int64_t k,
                                float* tau, int64_t capacity, int32_t* row, int32_t* col,
                                float* val, int32_t* row_ptr, void* ws, uint8_t* Aq, int64_t ldq,
                                float* sA, const void* W, int64_t N, int64_t ldw, uint8_t* Wq,
                                float* sW, uint32_t* colmax, bool* w_done, hipStream_t stream);

hipError_t launch_quantize_rows(const void* X, bool bf16, int64_t M, int64_t K, int64_t ldx,
                                const float* tau, uint8_t* Xq, int64_t ldq, float* sX,
                                hipStream_t stream);

hipError_t launch_quantize_weight(const void* W, bool bf16, int64_t K, int64_t N, int64_t ldw,
                                  uint8_t* Wq, int64_t ldq, float* sW, void* ws,
                                  hipStream_t stream);

struct SparseArgs {
  const int32_t* row_ptr;  // nullptr: no compensation term
  const int32_t* col;
  const float* val;
  const void* W;
  bool w_bf16;
  int64_t ldw;
  int64_t w_rows;  // K: rows of W (W is addressed with 32-bit byte offsets)
};

// Y[i, :] += sum over row i's non-zeros of val * W[col, :] (ascending col).
hipError_t launch_sparse_add(const SparseArgs& sp, int64_t M, int64_t N, float* Y, int64_t ldy,
                             hipStream_t stream);

hipError_t launch_fp4_gemm(const uint8_t* Aq, const float* sA, const uint8_t* Bq, const float* sB,
                           int64_t M, int64_t N, int64_t ldq, const SparseArgs& sp, float* Y,
                           int64_t ldy, hipStream_t stream);

// Micro-scaled operands: E2M1 codes with one E8M0 byte per 32 codes along K
// (rows of ldq / 16 bytes). Xs / Ws / As / Bs are those scale rows.
hipError_t launch_quantize_rows_mx(const void* X, bool bf16, int64_t M, int64_t K, int64_t ldx,
                                   const float* tau, uint8_t* Xq, int64_t ldq, uint8_t* Xs,
                                   hipStream_t stream);
hipError_t launch_quantize_cols_mx(const void* W, bool bf16, int64_t K, int64_t N, int64_t ldw,
                                   uint8_t* Wq, int64_t ldq, uint8_t* Ws, hipStream_t stream);
hipError_t launch_fp4_gemm_mx(const uint8_t* Aq, const uint8_t* As, const uint8_t* Bq,
                              const uint8_t* Bs, int64_t M, int64_t N, int64_t ldq,
                              const SparseArgs& sp, float* Y, int64_t ldy, hipStream_t stream);

}  // namespace fp4lin
