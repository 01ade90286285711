// C ABI of libfp4lin.so: argument checks, workspace layout and launches.
// Every check runs on the host before anything is enqueued; no call allocates,
// frees, synchronises or reads device memory.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "fp4lin.h"
#include "internal.hpp"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 31;

bool bad_dtype(fp4lin_dtype dt) { return dt != FP4LIN_F32 && dt != FP4LIN_BF16; }
// histogram bins count in 32 bits
constexpr int64_t kMaxCount = int64_t(1) << 32;
bool ok_dim(int64_t x) { return x >= 1 && x < kMaxDim; }
bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// HIP error behind the calling thread's last launch check (for
// fp4lin_last_hip_error).
thread_local hipError_t t_last_hip = hipSuccess;

fp4lin_status launch_status(hipError_t e) {
  t_last_hip = e;
  return e == hipSuccess ? FP4LIN_OK : FP4LIN_ERR_LAUNCH;
}

// The micro-scaled column quantizer launches one workgroup row per 128 codes
// of K along the grid's second dimension, which holds at most 65535; the
// token-wise one keeps the same limit.
constexpr int64_t kMaxColK = int64_t(65535) * 128;

// The column quantizers' one-dimensional grids (128-column tiles by 64 rows at
// the finest, plus the select's row workgroups when they share a launch) fit
// the 32-bit workgroup count.
bool col_grids_fit(int64_t K, int64_t N) {
  return ((N + 127) / 128) * ((K + 63) / 64) < (int64_t(1) << 32) - 4096;
}

// COO entries the select can produce for rank k: #{|a| > tau} <= n - 1 - k.
int64_t needed_capacity(int64_t n, int64_t k) { return n - 1 - k; }

size_t weight_ws(int64_t N) { return round_up(fp4lin::weight_workspace_bytes(N), 256); }

// The compensation kernel addresses W with 32-bit byte offsets.
bool weight_addressable(int64_t K, int64_t ldw, fp4lin_dtype wdt) {
  return K * ldw * (wdt == FP4LIN_BF16 ? 2 : 4) < kMaxDim;
}

size_t select_ws(int64_t M, fp4lin_dtype dt) {
  return round_up(fp4lin::select_workspace_bytes(dt == FP4LIN_BF16, M), 256);
}

}  // namespace

extern "C" {

int64_t fp4lin_quantile_rank(int64_t n, double q) {
  if (n < 1 || !(q >= 0.0 && q <= 1.0)) return -1;
  const double c = std::ceil(q * double(n));
  int64_t k = int64_t(c) - 1;
  if (k < 0) k = 0;
  if (k > n - 1) k = n - 1;
  return k;
}

int64_t fp4lin_packed_ld(int64_t L) {
  if (L < 1) return -1;
  return (L + 127) / 128 * 64;
}

size_t fp4lin_select_workspace_bytes(int64_t M, int64_t K, fp4lin_dtype dt) {
  if (!ok_dim(M) || !ok_dim(K) || bad_dtype(dt)) return 0;
  return select_ws(M, dt);
}

size_t fp4lin_weight_workspace_bytes(int64_t K, int64_t N) {
  if (!ok_dim(K) || !ok_dim(N)) return 0;
  return weight_ws(N);
}

}  // extern "C"

namespace {

// The forward's workspace: tau, the COO, the packed operands with their
// scales (fp32 vectors, or with mx the step-major E8M0 block scales), then
// scratch.
fp4lin_status forward_layout(int64_t M, int64_t K, int64_t N, fp4lin_dtype dt, double q, bool mx,
                             fp4lin_forward_offsets* out) {
  if (out == nullptr) return FP4LIN_ERR_NULL;
  if (!ok_dim(M) || !ok_dim(K) || !ok_dim(N)) return FP4LIN_ERR_SHAPE;
  if (bad_dtype(dt)) return FP4LIN_ERR_DTYPE;
  const int64_t n = M * K;
  if (n >= kMaxCount) return FP4LIN_ERR_SHAPE;
  const int64_t k = fp4lin_quantile_rank(n, q);
  if (k < 0) return FP4LIN_ERR_QUANTILE;
  const int64_t cap = needed_capacity(n, k);
  if (cap >= kMaxDim) return FP4LIN_ERR_SHAPE;
  const size_t slots = size_t(cap > 0 ? cap : 1);
  const size_t ldq = size_t(fp4lin_packed_ld(K));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  fp4lin_forward_offsets o{};
  o.tau = take(4);
  o.coo_row = take(slots * 4);
  o.coo_col = take(slots * 4);
  o.coo_val = take(slots * 4);
  o.row_ptr = take(size_t(M + 1) * 4);
  const size_t nblk = ldq / 16;
  o.Aq = take(size_t(M) * ldq);
  o.sA = take(size_t(M) * (mx ? nblk : 4));
  o.Wq = take(size_t(N) * ldq);
  o.sW = take(size_t(N) * (mx ? nblk : 4));
  // the select's workspace, then (token-wise) the column maxima of W's
  // quantization: the forward keeps both live at once
  o.scratch = take(select_ws(M, dt) + (mx ? 0 : weight_ws(N)));
  o.capacity = cap;
  o.total = off;
  *out = o;
  return FP4LIN_OK;
}

}  // namespace

extern "C" {

fp4lin_status fp4lin_forward_layout(int64_t M, int64_t K, int64_t N, fp4lin_dtype dt, double q,
                                    fp4lin_forward_offsets* out) {
  return forward_layout(M, K, N, dt, q, false, out);
}

fp4lin_status fp4lin_forward_layout_mx(int64_t M, int64_t K, int64_t N, fp4lin_dtype dt,
                                       double q, fp4lin_forward_offsets* out) {
  return forward_layout(M, K, N, dt, q, true, out);
}

size_t fp4lin_workspace_bytes(int64_t M, int64_t K, int64_t N, fp4lin_dtype dt, double q) {
  fp4lin_forward_offsets o;
  if (fp4lin_forward_layout(M, K, N, dt, q, &o) != FP4LIN_OK) return 0;
  return o.total;
}

size_t fp4lin_workspace_bytes_mx(int64_t M, int64_t K, int64_t N, fp4lin_dtype dt, double q) {
  fp4lin_forward_offsets o;
  if (fp4lin_forward_layout_mx(M, K, N, dt, q, &o) != FP4LIN_OK) return 0;
  return o.total;
}

int fp4lin_last_hip_error(void) { return int(t_last_hip); }

const char* fp4lin_last_hip_error_name(void) { return hipGetErrorName(t_last_hip); }

const char* fp4lin_status_str(fp4lin_status s) {
  switch (s) {
    case FP4LIN_OK: return "ok";
    case FP4LIN_ERR_NULL: return "a required pointer is NULL";
    case FP4LIN_ERR_SHAPE: return "invalid shape or leading dimension";
    case FP4LIN_ERR_DTYPE: return "unsupported dtype";
    case FP4LIN_ERR_QUANTILE: return "quantile q must be in [0, 1]";
    case FP4LIN_ERR_CAPACITY: return "COO capacity below M*K - 1 - k";
    case FP4LIN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FP4LIN_ERR_WORKSPACE: return "workspace too small";
    case FP4LIN_ERR_LAUNCH: return "kernel launch failed";
    case FP4LIN_ERR_SCRATCH: return "input needs more than the static scratch of the allocation-free call";
  }
  return "unknown status";
}

}  // extern "C"

namespace {

// The select's argument checks apart from the workspace.
fp4lin_status select_check(const void* A, fp4lin_dtype dt, int64_t M, int64_t K, int64_t lda,
                           double q, const float* tau, const fp4lin_coo& dA) {
  if (A == nullptr || tau == nullptr || dA.row == nullptr || dA.col == nullptr ||
      dA.val == nullptr || dA.row_ptr == nullptr)
    return FP4LIN_ERR_NULL;
  if (bad_dtype(dt)) return FP4LIN_ERR_DTYPE;
  if (!ok_dim(M) || !ok_dim(K) || lda < K) return FP4LIN_ERR_SHAPE;
  const int64_t n = M * K;
  if (n >= kMaxCount) return FP4LIN_ERR_SHAPE;
  const int64_t k = fp4lin_quantile_rank(n, q);
  if (k < 0) return FP4LIN_ERR_QUANTILE;
  const int64_t cap = needed_capacity(n, k);
  if (cap >= kMaxDim) return FP4LIN_ERR_SHAPE;
  if (dA.capacity < cap) return FP4LIN_ERR_CAPACITY;
  return FP4LIN_OK;
}

// fp4lin_outlier_select; with quantized set, the forward path's token-wise
// quantization of A (Xq, sX) is done by the same kernels where the rows allow
// it, and *quantized says whether it was.
fp4lin::FrontArgs front_args(const void* A, fp4lin_dtype dt, bool mx, int64_t M, int64_t K,
                             int64_t lda, double q, float* tau, const fp4lin_coo& coo,
                             void* scratch, uint8_t* Aq, int64_t ldq, void* sA, const void* W,
                             int64_t N, int64_t ldw, uint8_t* Wq, void* sW, uint32_t* colmax) {
  fp4lin::FrontArgs f;
  f.A = A;
  f.bf16 = dt == FP4LIN_BF16;
  f.mx = mx;
  f.M = M;
  f.K = K;
  f.lda = lda;
  f.k = fp4lin_quantile_rank(M * K, q);
  f.tau = tau;
  f.capacity = coo.capacity;
  f.row = coo.row;
  f.col = coo.col;
  f.val = coo.val;
  f.row_ptr = coo.row_ptr;
  f.ws = scratch;
  f.Aq = Aq;
  f.ldq = ldq;
  f.sA = sA;
  f.W = W;
  f.N = N;
  f.ldw = ldw;
  f.Wq = Wq;
  f.sW = sW;
  f.colmax = colmax;
  return f;
}
fp4lin_status select_impl(const void* A, fp4lin_dtype dt, int64_t M, int64_t K, int64_t lda,
                          double q, float* tau, fp4lin_coo dA, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  if (ws == nullptr) return FP4LIN_ERR_NULL;
  const fp4lin_status c = select_check(A, dt, M, K, lda, q, tau, dA);
  if (c != FP4LIN_OK) return c;
  if (!aligned16(ws)) return FP4LIN_ERR_ALIGN;
  if (ws_bytes < select_ws(M, dt)) return FP4LIN_ERR_WORKSPACE;
  return launch_status(fp4lin::launch_outlier_select(
      A, dt == FP4LIN_BF16, M, K, lda, fp4lin_quantile_rank(M * K, q), tau, dA.capacity,
      dA.row, dA.col, dA.val, dA.row_ptr, ws, stream));
}

// ---- allocation-free select ---------------------------------------------------
// fp4lin_outlier_select_noalloc keeps the select's scratch (selection state,
// histograms, per-row counts) in this array: one copy per GPU the library
// runs on, held until the process ends. In host code its name is only a
// host-side stand-in; the device address of each GPU's copy is looked up once
// per device, with that device current, and only that address is used.
// None of the select's kernels relies on the scratch being cleared, so the
// contents a previous call left are harmless.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices];

// This GPU's copy of the scratch: the device of `stream` (the current device
// for the null stream), looked up on the first call for that device.
hipError_t scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_addr[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev) {
      e = hipSetDevice(dev);
      if (e != hipSuccess) return e;
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

fp4lin_status fp4lin_outlier_select(const void* A, fp4lin_dtype dt, int64_t M, int64_t K,
                                    int64_t lda, double q, float* tau, fp4lin_coo dA, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  return select_impl(A, dt, M, K, lda, q, tau, dA, ws, ws_bytes, stream);
}

fp4lin_status fp4lin_outlier_select_noalloc(const void* A, fp4lin_dtype dt, int64_t M,
                                            int64_t K, int64_t lda, double q, float* tau,
                                            fp4lin_coo dA, hipStream_t stream) {
  const fp4lin_status c = select_check(A, dt, M, K, lda, q, tau, dA);
  if (c != FP4LIN_OK) return c;
  if (select_ws(M, dt) > kNoAllocScratchBytes) return FP4LIN_ERR_SCRATCH;
  void* ws = nullptr;
  const hipError_t e = scratch_address(stream, &ws);
  if (e != hipSuccess) return launch_status(e);
  return select_impl(A, dt, M, K, lda, q, tau, dA, ws, kNoAllocScratchBytes, stream);
}

fp4lin_status fp4lin_quantize_act(const void* X, fp4lin_dtype dt, int64_t M, int64_t K,
                                  int64_t ldx, const float* tau, uint8_t* Xq, float* sX,
                                  hipStream_t stream) {
  if (X == nullptr || Xq == nullptr || sX == nullptr) return FP4LIN_ERR_NULL;
  if (bad_dtype(dt)) return FP4LIN_ERR_DTYPE;
  if (!ok_dim(M) || !ok_dim(K) || ldx < K) return FP4LIN_ERR_SHAPE;
  if (!aligned16(Xq)) return FP4LIN_ERR_ALIGN;
  return launch_status(fp4lin::launch_quantize_rows(X, dt == FP4LIN_BF16, M, K, ldx, tau, Xq,
                                                    fp4lin_packed_ld(K), sX, stream));
}

fp4lin_status fp4lin_quantize_weight(const void* W, fp4lin_dtype dt, int64_t K, int64_t N,
                                     int64_t ldw, uint8_t* Wq, float* sW, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  if (W == nullptr || Wq == nullptr || sW == nullptr || ws == nullptr) return FP4LIN_ERR_NULL;
  if (bad_dtype(dt)) return FP4LIN_ERR_DTYPE;
  if (!ok_dim(K) || !ok_dim(N) || ldw < N || K > kMaxColK || !col_grids_fit(K, N))
    return FP4LIN_ERR_SHAPE;
  if (!aligned16(Wq) || !aligned16(ws)) return FP4LIN_ERR_ALIGN;
  if (ws_bytes < weight_ws(N)) return FP4LIN_ERR_WORKSPACE;
  return launch_status(fp4lin::launch_quantize_weight(W, dt == FP4LIN_BF16, K, N, ldw, Wq,
                                                      fp4lin_packed_ld(K), sW, ws, stream));
}

fp4lin_status fp4lin_gemm(const uint8_t* Aq, const float* sA, const uint8_t* Bq, const float* sB,
                          int64_t M, int64_t N, int64_t K, const fp4lin_coo* dA, const void* W,
                          fp4lin_dtype wdt, int64_t ldw, float* Y, int64_t ldy,
                          hipStream_t stream) {
  if (Aq == nullptr || sA == nullptr || Bq == nullptr || sB == nullptr || Y == nullptr)
    return FP4LIN_ERR_NULL;
  if (!ok_dim(M) || !ok_dim(N) || !ok_dim(K) || ldy < N) return FP4LIN_ERR_SHAPE;
  fp4lin::SparseArgs sp{nullptr, nullptr, nullptr, nullptr, false, 0, 0, 0};
  if (dA != nullptr) {
    if (dA->row_ptr == nullptr || dA->col == nullptr || dA->val == nullptr || W == nullptr)
      return FP4LIN_ERR_NULL;
    if (bad_dtype(wdt)) return FP4LIN_ERR_DTYPE;
    if (ldw < N || !weight_addressable(K, ldw, wdt)) return FP4LIN_ERR_SHAPE;
    sp = fp4lin::SparseArgs{dA->row_ptr, dA->col, dA->val, W, wdt == FP4LIN_BF16, ldw, K,
                            dA->capacity};
  }
  // packed operands are addressed with 32-bit byte offsets
  const int64_t ldq = fp4lin_packed_ld(K);
  if ((M + 1) * ldq >= kMaxDim || (N + 1) * ldq >= kMaxDim) return FP4LIN_ERR_SHAPE;
  if (!aligned16(Aq) || !aligned16(Bq)) return FP4LIN_ERR_ALIGN;
  return launch_status(
      fp4lin::launch_fp4_gemm(Aq, sA, Bq, sB, M, N, fp4lin_packed_ld(K), sp, Y, ldy, stream));
}

fp4lin_status fp4lin_sparse_add(const fp4lin_coo* dA, const void* W, fp4lin_dtype wdt,
                                int64_t K, int64_t ldw, int64_t M, int64_t N, float* Y,
                                int64_t ldy, hipStream_t stream) {
  if (dA == nullptr || dA->row_ptr == nullptr || dA->col == nullptr || dA->val == nullptr ||
      W == nullptr || Y == nullptr)
    return FP4LIN_ERR_NULL;
  if (bad_dtype(wdt)) return FP4LIN_ERR_DTYPE;
  if (!ok_dim(M) || !ok_dim(N) || !ok_dim(K) || ldw < N || ldy < N ||
      !weight_addressable(K, ldw, wdt))
    return FP4LIN_ERR_SHAPE;
  const fp4lin::SparseArgs sp{dA->row_ptr, dA->col, dA->val, W, wdt == FP4LIN_BF16,
                              ldw,         K,       dA->capacity};
  return launch_status(fp4lin::launch_sparse_add(sp, M, N, Y, ldy, stream));
}

int64_t fp4lin_mx_scales_ld(int64_t L) {
  if (L < 1) return -1;
  return fp4lin_packed_ld(L) / 16;
}

fp4lin_status fp4lin_quantize_act_mx(const void* X, fp4lin_dtype dt, int64_t M, int64_t K,
                                     int64_t ldx, const float* tau, uint8_t* Xq, uint8_t* Xs,
                                     hipStream_t stream) {
  if (X == nullptr || Xq == nullptr || Xs == nullptr) return FP4LIN_ERR_NULL;
  if (bad_dtype(dt)) return FP4LIN_ERR_DTYPE;
  if (!ok_dim(M) || !ok_dim(K) || ldx < K) return FP4LIN_ERR_SHAPE;
  if (!aligned16(Xq) || !aligned16(Xs)) return FP4LIN_ERR_ALIGN;
  return launch_status(fp4lin::launch_quantize_rows_mx(X, dt == FP4LIN_BF16, M, K, ldx, tau, Xq,
                                                       fp4lin_packed_ld(K), Xs, stream));
}

fp4lin_status fp4lin_quantize_weight_mx(const void* W, fp4lin_dtype dt, int64_t K, int64_t N,
                                        int64_t ldw, uint8_t* Wq, uint8_t* Ws,
                                        hipStream_t stream) {
  if (W == nullptr || Wq == nullptr || Ws == nullptr) return FP4LIN_ERR_NULL;
  if (bad_dtype(dt)) return FP4LIN_ERR_DTYPE;
  if (!ok_dim(K) || !ok_dim(N) || ldw < N || K > kMaxColK || !col_grids_fit(K, N))
    return FP4LIN_ERR_SHAPE;
  if (!aligned16(Wq) || !aligned16(Ws)) return FP4LIN_ERR_ALIGN;
  return launch_status(fp4lin::launch_quantize_cols_mx(W, dt == FP4LIN_BF16, K, N, ldw, Wq,
                                                       fp4lin_packed_ld(K), Ws, stream));
}

fp4lin_status fp4lin_gemm_mx(const uint8_t* Aq, const uint8_t* As, const uint8_t* Bq,
                             const uint8_t* Bs, int64_t M, int64_t N, int64_t K,
                             const fp4lin_coo* dA, const void* W, fp4lin_dtype wdt,
                             int64_t ldw, float* Y, int64_t ldy, hipStream_t stream) {
  if (Aq == nullptr || As == nullptr || Bq == nullptr || Bs == nullptr || Y == nullptr)
    return FP4LIN_ERR_NULL;
  if (!ok_dim(M) || !ok_dim(N) || !ok_dim(K) || ldy < N) return FP4LIN_ERR_SHAPE;
  fp4lin::SparseArgs sp{nullptr, nullptr, nullptr, nullptr, false, 0, 0, 0};
  if (dA != nullptr) {
    if (dA->row_ptr == nullptr || dA->col == nullptr || dA->val == nullptr || W == nullptr)
      return FP4LIN_ERR_NULL;
    if (bad_dtype(wdt)) return FP4LIN_ERR_DTYPE;
    if (ldw < N || !weight_addressable(K, ldw, wdt)) return FP4LIN_ERR_SHAPE;
    sp = fp4lin::SparseArgs{dA->row_ptr, dA->col, dA->val, W, wdt == FP4LIN_BF16, ldw, K,
                            dA->capacity};
  }
  // packed operands and scale rows are addressed with 32-bit byte offsets
  const int64_t ldq = fp4lin_packed_ld(K);
  if ((M + 1) * ldq >= kMaxDim || (N + 1) * ldq >= kMaxDim) return FP4LIN_ERR_SHAPE;
  if (!aligned16(Aq) || !aligned16(Bq) || !aligned16(As) || !aligned16(Bs))
    return FP4LIN_ERR_ALIGN;
  return launch_status(fp4lin::launch_fp4_gemm_mx(Aq, As, Bq, Bs, M, N, ldq, sp, Y, ldy, stream));
}

fp4lin_status fp4lin_forward(const void* A, const void* W, fp4lin_dtype dt, int64_t M, int64_t K,
                             int64_t N, int64_t lda, int64_t ldw, double q, float* Y, int64_t ldy,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  if (A == nullptr || W == nullptr || Y == nullptr || ws == nullptr) return FP4LIN_ERR_NULL;
  if (bad_dtype(dt)) return FP4LIN_ERR_DTYPE;
  if (!ok_dim(M) || !ok_dim(K) || !ok_dim(N) || lda < K || ldw < N || ldy < N)
    return FP4LIN_ERR_SHAPE;
  fp4lin_forward_offsets o;
  const fp4lin_status ls = fp4lin_forward_layout(M, K, N, dt, q, &o);
  if (ls != FP4LIN_OK) return ls;
  if (!aligned16(ws)) return FP4LIN_ERR_ALIGN;
  if (ws_bytes < o.total) return FP4LIN_ERR_WORKSPACE;
  // the limits of the GEMM and of W's quantizer, checked before anything is
  // enqueued
  const int64_t ldq = fp4lin_packed_ld(K);
  if ((M + 1) * ldq >= kMaxDim || (N + 1) * ldq >= kMaxDim || !weight_addressable(K, ldw, dt) ||
      K > kMaxColK)
    return FP4LIN_ERR_SHAPE;
  char* base = static_cast<char*>(ws);
  float* tau = reinterpret_cast<float*>(base + o.tau);
  fp4lin_coo coo;
  coo.row = reinterpret_cast<int32_t*>(base + o.coo_row);
  coo.col = reinterpret_cast<int32_t*>(base + o.coo_col);
  coo.val = reinterpret_cast<float*>(base + o.coo_val);
  coo.row_ptr = reinterpret_cast<int32_t*>(base + o.row_ptr);
  coo.capacity = o.capacity;
  uint8_t* Aq = reinterpret_cast<uint8_t*>(base + o.Aq);
  float* sA = reinterpret_cast<float*>(base + o.sA);
  uint8_t* Wq = reinterpret_cast<uint8_t*>(base + o.Wq);
  float* sW = reinterpret_cast<float*>(base + o.sW);
  void* scratch = base + o.scratch;
  // select, quantization of A (in the select's compaction) and of W (in the
  // select's row launches); W's column maxima follow the select's workspace
  const fp4lin::FrontArgs f = front_args(A, dt, false, M, K, lda, q, tau, coo, scratch, Aq, ldq, sA,
                                         W, N, ldw, Wq, sW,
                                         reinterpret_cast<uint32_t*>(static_cast<char*>(scratch) +
                                                                     select_ws(M, dt)));
  const fp4lin_status s = launch_status(fp4lin::launch_forward_front(f, stream));
  if (s != FP4LIN_OK) return s;
  return fp4lin_gemm(Aq, sA, Wq, sW, M, N, K, &coo, W, dt, ldw, Y, ldy, stream);
}

fp4lin_status fp4lin_forward_mx(const void* A, const void* W, fp4lin_dtype dt, int64_t M,
                                int64_t K, int64_t N, int64_t lda, int64_t ldw, double q,
                                float* Y, int64_t ldy, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  if (A == nullptr || W == nullptr || Y == nullptr || ws == nullptr) return FP4LIN_ERR_NULL;
  if (bad_dtype(dt)) return FP4LIN_ERR_DTYPE;
  if (!ok_dim(M) || !ok_dim(K) || !ok_dim(N) || lda < K || ldw < N || ldy < N)
    return FP4LIN_ERR_SHAPE;
  fp4lin_forward_offsets o;
  const fp4lin_status ls = fp4lin_forward_layout_mx(M, K, N, dt, q, &o);
  if (ls != FP4LIN_OK) return ls;
  if (!aligned16(ws)) return FP4LIN_ERR_ALIGN;
  if (ws_bytes < o.total) return FP4LIN_ERR_WORKSPACE;
  // the limits of the GEMM and of W's quantizer, checked before anything is
  // enqueued
  const int64_t ldq = fp4lin_packed_ld(K);
  if ((M + 1) * ldq >= kMaxDim || (N + 1) * ldq >= kMaxDim || !weight_addressable(K, ldw, dt) ||
      K > kMaxColK)
    return FP4LIN_ERR_SHAPE;
  char* base = static_cast<char*>(ws);
  float* tau = reinterpret_cast<float*>(base + o.tau);
  fp4lin_coo coo;
  coo.row = reinterpret_cast<int32_t*>(base + o.coo_row);
  coo.col = reinterpret_cast<int32_t*>(base + o.coo_col);
  coo.val = reinterpret_cast<float*>(base + o.coo_val);
  coo.row_ptr = reinterpret_cast<int32_t*>(base + o.row_ptr);
  coo.capacity = o.capacity;
  uint8_t* Aq = reinterpret_cast<uint8_t*>(base + o.Aq);
  uint8_t* As = reinterpret_cast<uint8_t*>(base + o.sA);
  uint8_t* Wq = reinterpret_cast<uint8_t*>(base + o.Wq);
  uint8_t* Ws = reinterpret_cast<uint8_t*>(base + o.sW);
  void* scratch = base + o.scratch;
  // select, micro-scaled quantization of A (in the select's compaction) and
  // of W (in the select's row-count launch)
  const fp4lin::FrontArgs f = front_args(A, dt, true, M, K, lda, q, tau, coo, scratch, Aq, ldq, As,
                                         W, N, ldw, Wq, Ws, nullptr);
  const fp4lin_status s = launch_status(fp4lin::launch_forward_front(f, stream));
  if (s != FP4LIN_OK) return s;
  return fp4lin_gemm_mx(Aq, As, Wq, Ws, M, N, K, &coo, W, dt, ldw, Y, ldy, stream);
}

}  // extern "C"
