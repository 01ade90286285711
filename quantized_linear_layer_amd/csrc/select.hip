// Outlier selection: exact per-tensor |A| quantile by multi-pass radix select,
// then row-major stream compaction of the clamped entries into COO.
//
// Method: the outlier paragraph of the FP4 training write-up ("微软首创FP4训练框架")
// finds the largest-magnitude activations by a quantile search and clamps them to
// a threshold; the compensation paragraph keeps A - A_clamped as a sparse matrix
// that is non-zero only at clamped positions.
//
// |a| of a finite float is ordered like its bit pattern with the sign cleared,
// so the k-th smallest |a| is the k-th smallest integer key. The key is found
// digit by digit from the top: each pass histograms one digit of the keys whose
// higher digits equal the prefix found so far (LDS histogram per workgroup,
// merged with global atomics), and a one-workgroup pick kernel finds the digit
// that holds the remaining rank. Everything stays on the device; the host never
// reads the histogram.
#include "device_common.hpp"
#include "internal.hpp"

namespace fp4lin {

namespace {

constexpr int kHistBins = 2048;  // widest digit: 11 bits

struct SelState {
  uint32_t prefix;   // key bits decided so far (right-aligned)
  uint32_t tau_key;  // final key after the last pass
  int64_t krem;      // rank still to find inside the current prefix
};

template <class In>
struct DigitPlan;
template <>
struct DigitPlan<BF16In> {  // 15-bit keys: 11 + 4
  static constexpr int kPasses = 2;
  static constexpr int kKeyBits = 15;
  __host__ __device__ static constexpr int shift(int p) { return p == 0 ? 4 : 0; }
  __host__ __device__ static constexpr int width(int p) { return p == 0 ? 11 : 4; }
};
template <>
struct DigitPlan<F32In> {  // 31-bit keys: 11 + 11 + 9
  static constexpr int kPasses = 3;
  static constexpr int kKeyBits = 31;
  __host__ __device__ static constexpr int shift(int p) { return p == 0 ? 20 : (p == 1 ? 9 : 0); }
  __host__ __device__ static constexpr int width(int p) { return p == 0 ? 11 : (p == 1 ? 11 : 9); }
};

__global__ void select_init_kernel(SelState* st, uint32_t* hist, int nwords, int64_t k) {
  for (int i = threadIdx.x; i < nwords; i += blockDim.x) hist[i] = 0u;
  if (threadIdx.x == 0) {
    st->prefix = 0u;
    st->tau_key = 0u;
    st->krem = k;
  }
}

// One radix pass: histogram digit (key >> shift) & mask of the keys whose bits
// above hi_shift equal the current prefix.
template <class In, bool kAligned>
__global__ __launch_bounds__(256) void select_hist_kernel(
    const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda,
    const SelState* __restrict__ st, int shift, int width, int hi_shift,
    uint32_t* __restrict__ ghist) {
  __shared__ uint32_t h[kHistBins];
  const int nb = 1 << width;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  const uint32_t prefix = st->prefix;
  const uint32_t mask = uint32_t(nb - 1);
  for (int64_t r = blockIdx.x; r < M; r += gridDim.x) {
    const typename In::T* row = A + r * lda;
    for (int64_t c = int64_t(threadIdx.x) * 8; c < K; c += int64_t(blockDim.x) * 8) {
      Vec8<In> v;
      const int64_t valid = K - c;
      load8<In, kAligned>(row + c, valid, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t key = In::key(v.v[i]);
        const bool in_prefix = (hi_shift >= 32 ? 0u : (key >> hi_shift)) == prefix;
        if (i < valid && in_prefix) atomicAdd(&h[(key >> shift) & mask], 1u);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += blockDim.x) {
    const uint32_t c = h[i];
    if (c) atomicAdd(&ghist[i], c);
  }
}

// Find the digit whose cumulative count passes the remaining rank.
__global__ __launch_bounds__(256) void select_pick_kernel(SelState* st,
                                                          const uint32_t* __restrict__ hist,
                                                          int width, int last, int key_is_bf16,
                                                          float* __restrict__ tau) {
  __shared__ uint64_t part[256];
  const int nb = 1 << width;
  const int per = (nb + 255) / 256;
  const int t = threadIdx.x;
  const int lo = t * per;
  uint64_t s = 0;
  for (int i = 0; i < per; ++i)
    if (lo + i < nb) s += hist[lo + i];
  part[t] = s;
  __syncthreads();
  // inclusive scan over 256 partial sums (Hillis-Steele, 8 steps)
  for (int off = 1; off < 256; off <<= 1) {
    uint64_t add = (t >= off) ? part[t - off] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  const int64_t krem = st->krem;
  const uint64_t before = (t == 0) ? 0 : part[t - 1];
  const uint64_t upto = part[t];
  __syncthreads();
  if (uint64_t(krem) >= before && uint64_t(krem) < upto) {
    uint64_t acc = before;
    for (int i = 0; i < per; ++i) {
      const int b = lo + i;
      const uint64_t c = (b < nb) ? hist[b] : 0;
      if (uint64_t(krem) < acc + c) {
        const uint32_t prefix = (st->prefix << width) | uint32_t(b);
        st->prefix = prefix;
        st->krem = krem - int64_t(acc);
        if (last) {
          st->tau_key = prefix;
          *tau = key_is_bf16 ? __uint_as_float(prefix << 16) : __uint_as_float(prefix);
        }
        break;
      }
      acc += c;
    }
  }
}

// Per-row count of |a| > tau, written to row_ptr[i+1]. One wave per row.
template <class In, bool kAligned>
__global__ __launch_bounds__(256) void count_rows_kernel(const typename In::T* __restrict__ A,
                                                         int64_t M, int64_t K, int64_t lda,
                                                         const SelState* __restrict__ st,
                                                         int32_t* __restrict__ row_ptr) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (blockIdx.x == 0 && threadIdx.x == 0) row_ptr[0] = 0;
  if (r >= M) return;
  const uint32_t tkey = st->tau_key;
  const typename In::T* row = A + r * lda;
  uint32_t cnt = 0;
  for (int64_t c = int64_t(lane) * 8; c < K; c += kWave * 8) {
    Vec8<In> v;
    const int64_t valid = K - c;
    load8<In, kAligned>(row + c, valid, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) cnt += (i < valid && In::key(v.v[i]) > tkey) ? 1u : 0u;
  }
  cnt = wave_sum_u32(cnt);
  if (lane == 0) row_ptr[r + 1] = int32_t(cnt);
}

// In-place inclusive scan of row_ptr[1..M] (one workgroup of 1024 threads).
__global__ __launch_bounds__(1024) void scan_rows_kernel(int32_t* __restrict__ row_ptr, int64_t M) {
  __shared__ int32_t buf[1024];
  __shared__ int32_t carry;
  const int t = threadIdx.x;
  if (t == 0) carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < M; base += 1024) {
    const int64_t i = base + t;
    int32_t v = (i < M) ? row_ptr[i + 1] : 0;
    buf[t] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int32_t add = (t >= off) ? buf[t - off] : 0;
      __syncthreads();
      buf[t] += add;
      __syncthreads();
    }
    const int32_t c = carry;
    if (i < M) row_ptr[i + 1] = buf[t] + c;
    __syncthreads();
    if (t == 1023) carry = c + buf[1023];
    __syncthreads();
  }
}

// Write every |a| > tau entry of a row, ascending column, at row_ptr[i] + rank.
template <class In, bool kAligned>
__global__ __launch_bounds__(256) void compact_rows_kernel(
    const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda,
    const SelState* __restrict__ st, const float* __restrict__ tau_p,
    const int32_t* __restrict__ row_ptr, int64_t capacity, int32_t* __restrict__ out_row,
    int32_t* __restrict__ out_col, float* __restrict__ out_val) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (r >= M) return;
  const uint32_t tkey = st->tau_key;
  const float tau = *tau_p;
  const typename In::T* row = A + r * lda;
  int64_t pos = row_ptr[r];
  for (int64_t c0 = 0; c0 < K; c0 += kWave * 8) {
    const int64_t c = c0 + int64_t(lane) * 8;
    Vec8<In> v;
    const int64_t valid = K - c;
    uint32_t cnt = 0;
    if (valid > 0) {
      load8<In, kAligned>(row + c, valid, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) cnt += (i < valid && In::key(v.v[i]) > tkey) ? 1u : 0u;
    }
    uint32_t total;
    const uint32_t off = wave_exclusive_scan(cnt, total);
    if (cnt) {
      int64_t p = pos + off;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // p < capacity always holds when tau is the true order statistic
        // (nnz <= n-1-k); the test only keeps a wrong tau from writing out of bounds.
        if (i < valid && In::key(v.v[i]) > tkey && p < capacity) {
          const float a = In::widen(v.v[i]);
          out_row[p] = int32_t(r);
          out_col[p] = int32_t(c + i);
          out_val[p] = __fsub_rn(a, copysignf(tau, a));
          ++p;
        }
      }
    }
    pos += total;
  }
}

template <class In>
size_t hist_words() {
  return size_t(DigitPlan<In>::kPasses) * kHistBins;
}

template <class In, bool kAligned>
hipError_t run_select(const void* Ap, int64_t M, int64_t K, int64_t lda, int64_t k, float* tau,
                      int64_t capacity,
                      int32_t* row, int32_t* col, float* val, int32_t* row_ptr, void* ws,
                      hipStream_t stream) {
  using T = typename In::T;
  const T* A = static_cast<const T*>(Ap);
  SelState* st = static_cast<SelState*>(ws);
  uint32_t* hist = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + 256);
  const int nwords = int(hist_words<In>());
  select_init_kernel<<<1, 256, 0, stream>>>(st, hist, nwords, k);
  // Enough workgroups to fill the chip, each with a few tens of thousands of
  // elements so that the per-group histogram merge stays small.
  const int64_t n = M * K;
  int64_t g = n / 65536;
  g = g < 1 ? 1 : (g > 1024 ? 1024 : g);
  g = g > M ? M : g;
  for (int p = 0; p < DigitPlan<In>::kPasses; ++p) {
    const int shift = DigitPlan<In>::shift(p);
    const int width = DigitPlan<In>::width(p);
    const int hi = shift + width;
    select_hist_kernel<In, kAligned><<<dim3(unsigned(g)), 256, 0, stream>>>(
        A, M, K, lda, st, shift, width, hi >= DigitPlan<In>::kKeyBits ? 32 : hi,
        hist + size_t(p) * kHistBins);
    select_pick_kernel<<<1, 256, 0, stream>>>(st, hist + size_t(p) * kHistBins, width,
                                               p == DigitPlan<In>::kPasses - 1 ? 1 : 0,
                                               In::kBytes == 2 ? 1 : 0, tau);
  }
  const unsigned rows_blocks = unsigned((M + 3) / 4);
  count_rows_kernel<In, kAligned><<<rows_blocks, 256, 0, stream>>>(A, M, K, lda, st, row_ptr);
  scan_rows_kernel<<<1, 1024, 0, stream>>>(row_ptr, M);
  compact_rows_kernel<In, kAligned><<<rows_blocks, 256, 0, stream>>>(A, M, K, lda, st, tau,
                                                                     row_ptr, capacity, row, col,
                                                                     val);
  return hipGetLastError();
}

}  // namespace

size_t select_workspace_bytes(bool bf16) {
  const size_t words = bf16 ? hist_words<BF16In>() : hist_words<F32In>();
  return 256 + words * 4;
}

hipError_t launch_outlier_select(const void* A, bool bf16, int64_t M, int64_t K, int64_t lda,
                                 int64_t k, float* tau, int64_t capacity, int32_t* row,
                                 int32_t* col, float* val, int32_t* row_ptr, void* ws,
                                 hipStream_t stream) {
  const int esz = bf16 ? 2 : 4;
  const bool aligned = (reinterpret_cast<uintptr_t>(A) % 16 == 0) && ((lda * esz) % 16 == 0);
  if (bf16)
    return aligned ? run_select<BF16In, true>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws, stream)
                   : run_select<BF16In, false>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws, stream);
  return aligned ? run_select<F32In, true>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws, stream)
                 : run_select<F32In, false>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws, stream);
}

}  // namespace fp4lin
