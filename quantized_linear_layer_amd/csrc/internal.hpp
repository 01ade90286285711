// Launchers behind the C ABI. Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp4lin {

size_t select_workspace_bytes(bool bf16, int64_t M);
size_t weight_workspace_bytes(int64_t N);

hipError_t launch_outlier_select(const void* A, bool bf16, int64_t M, int64_t K, int64_t lda,
                                 int64_t k, float* tau, int64_t capacity, int32_t* row,
                                 int32_t* col, float* val, int32_t* row_ptr, void* ws,
                                 hipStream_t stream);

// Whole-layer forward, front half: the select of launch_outlier_select (rank
// k, workspace ws of select_workspace_bytes) with the quantization of A
// clamped to tau done by its compaction, and the quantization of W (same
// dtype as A) in launches shared with the select's row kernels. Token-wise:
// sA and sW are float scales and colmax (N words apart from ws) is cleared by
// the select's first pass; micro-scaled (mx): sA and sW are the step-major
// E8M0 arrays and colmax is unused. Any K, alignment and leading dimensions.
struct FrontArgs {
  const void* A;
  bool bf16, mx;
  int64_t M, K, lda, k;
  float* tau;
  int64_t capacity;
  int32_t *row, *col;
  float* val;
  int32_t* row_ptr;
  void* ws;
  uint8_t* Aq;
  int64_t ldq;
  void* sA;
  const void* W;
  int64_t N, ldw;
  uint8_t* Wq;
  void* sW;
  uint32_t* colmax;
};
hipError_t launch_forward_front(const FrontArgs& f, hipStream_t stream);

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
  int64_t capacity;  // COO entries allocated: bounds the non-zeros (picks the GEMM's schedule)
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
