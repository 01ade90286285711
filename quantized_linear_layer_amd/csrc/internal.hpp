// Launchers behind the C ABI. Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp4lin {

size_t select_workspace_bytes(bool bf16, int64_t M);
size_t weight_workspace_bytes(int64_t N);

// With quantized set, rows that allow it are also quantized token-wise (Xq
// with row stride ldq, scales sX, clamped to tau) by the compaction, and
// *quantized says whether that happened; with quantized null, Xq is ignored.
hipError_t launch_outlier_select(const void* A, bool bf16, int64_t M, int64_t K, int64_t lda,
                                 int64_t k, float* tau, int64_t capacity, int32_t* row,
                                 int32_t* col, float* val, int32_t* row_ptr, void* ws,
                                 hipStream_t stream, uint8_t* Xq = nullptr, int64_t ldq = 0,
                                 float* sX = nullptr, bool* quantized = nullptr);

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

}  // namespace fp4lin
