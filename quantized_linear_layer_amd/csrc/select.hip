// Outlier selection: exact per-tensor |A| quantile by radix select, then
// row-major stream compaction of the clamped entries into COO.
//
// Method: the outlier paragraph of the FP4 training write-up ("微软首创FP4训练框架")
// finds the largest-magnitude activations by a quantile search and clamps them to
// a threshold; the compensation paragraph keeps A - A_clamped as a sparse matrix
// that is non-zero only at clamped positions.
//
// |a| of a finite float is ordered like its bit pattern with the sign cleared,
// so the k-th smallest |a| is the k-th smallest integer key, found digit by
// digit from the top: each pass histograms one digit of the keys whose higher
// digits equal the prefix found so far, and a one-workgroup pick kernel finds
// the digit that holds the remaining rank. Everything stays on the device; the
// host never reads a histogram.
//
// bfloat16 keys (15 bits) take two passes over A. Pass 1 builds a full
// 32768-bin histogram per workgroup in LDS (one 16-wave workgroup per CU),
// which spreads the densely populated magnitudes over many bins so that few
// lanes of an LDS atomic meet on one address, but merges only its 128 coarse
// sums (256 keys each) into global memory: merging every non-zero fine bin with
// device-wide atomics costs several times the pass itself. Pass 2 histograms
// the 256 keys of the chosen coarse bin. float32 keys (31 bits) take three
// passes of 11, 11 and 9 bits with a 2048-bin histogram.
//
// Then the entries with |a| > tau are counted per row, the counts scanned into
// row_ptr, and the entries written in row-major order.
#include "device_common.hpp"
#include "internal.hpp"

namespace fp4lin {

namespace {

struct SelState {
  uint32_t prefix;   // key bits decided so far (right-aligned)
  uint32_t tau_key;  // final key after the last pass
  int64_t krem;      // rank still to find inside the current prefix
};

// Find the digit whose cumulative count passes the remaining rank and append
// it to the prefix; after the last pass the prefix is the key of tau, whose
// float bits are key << key_shift. One workgroup of 256 threads.
__global__ __launch_bounds__(256) void select_pick_kernel(SelState* st,
                                                          const uint32_t* __restrict__ hist,
                                                          int width, int last, int key_shift,
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
          *tau = __uint_as_float(prefix << key_shift);
        }
        break;
      }
      acc += c;
    }
  }
}

// ---------------------------------------------------------------------------
// float32: digit histograms of 11, 11 and 9 bits.
// ---------------------------------------------------------------------------
constexpr int kHistBins = 2048;
constexpr int kHistThreads = 256;
constexpr int kHistCh = 2;  // chunks per thread per slab

struct F32Digits {
  static constexpr int kPasses = 3;
  static constexpr int kKeyBits = 31;
  __host__ __device__ static constexpr int shift(int p) { return p == 0 ? 20 : (p == 1 ? 9 : 0); }
  __host__ __device__ static constexpr int width(int p) { return p == 0 ? 11 : (p == 1 ? 11 : 9); }
};

// The matrix is cut into slabs of kHistCh chunks per thread (a slab never
// crosses a row); workgroups stride over slabs and load the next slab before
// counting the current one.
template <class In, bool kFast>
__device__ inline void load_slab(const typename In::T* __restrict__ A, int64_t lda, int64_t K,
                                 int64_t spr, int64_t s, Vec8<In> (&v)[kHistCh], int64_t& c0) {
  const int64_t r = s / spr;
  c0 = (s - r * spr) * (int64_t(kHistThreads) * kHistCh * 8);
  const typename In::T* row = A + r * lda;
#pragma unroll
  for (int j = 0; j < kHistCh; ++j)
    load_chunk<In, kFast>(row, c0 + (int64_t(j) * kHistThreads + threadIdx.x) * 8, K, v[j]);
}

// Histogram digit (key >> shift) & mask of the keys whose bits at and above
// hi_shift equal the current prefix (hi_shift >= 32: all keys).
template <class In, bool kFast>
__global__ __launch_bounds__(kHistThreads) void select_hist_kernel(
    const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda,
    const SelState* __restrict__ st, int shift, int width, int hi_shift,
    uint32_t* __restrict__ ghist) {
  __shared__ uint32_t h[kHistBins];
  const int nb = 1 << width;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  const uint32_t prefix = st->prefix;
  const uint32_t mask = uint32_t(nb - 1);
  const int64_t slab = int64_t(kHistThreads) * kHistCh * 8;
  const int64_t spr = (K + slab - 1) / slab;
  const int64_t total = M * spr;
  int64_t s = blockIdx.x;
  Vec8<In> cur[kHistCh];
  int64_t c_cur = 0;
  if (s < total) load_slab<In, kFast>(A, lda, K, spr, s, cur, c_cur);
  for (; s < total; s += gridDim.x) {
    Vec8<In> nxt[kHistCh];
    int64_t c_nxt = 0;
    if (s + gridDim.x < total) load_slab<In, kFast>(A, lda, K, spr, s + gridDim.x, nxt, c_nxt);
#pragma unroll
    for (int j = 0; j < kHistCh; ++j) {
      const int64_t c = c_cur + (int64_t(j) * kHistThreads + threadIdx.x) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t key = In::key(cur[j].v[i]);
        const bool in_prefix = (hi_shift >= 32 ? 0u : (key >> hi_shift)) == prefix;
        if (c + i < K && in_prefix) atomicAdd(&h[(key >> shift) & mask], 1u);
      }
    }
#pragma unroll
    for (int j = 0; j < kHistCh; ++j) cur[j] = nxt[j];
    c_cur = c_nxt;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += blockDim.x) {
    const uint32_t c = h[i];
    if (c) atomicAdd(&ghist[i], c);
  }
}

// ---------------------------------------------------------------------------
// bfloat16: coarse pass (7-bit digit from a full 15-bit LDS histogram), fine
// pass (8-bit digit).
// ---------------------------------------------------------------------------
constexpr int kKeyBins16 = 1 << 15;
constexpr int kFineBits = 8;
constexpr int kCoarseBits = 15 - kFineBits;
constexpr int kCoarseBins = 1 << kCoarseBits;
constexpr int kFineBins = 1 << kFineBits;
constexpr int kH16Threads = 1024;
constexpr int kH16Waves = kH16Threads / kWave;

// Both bfloat16 passes. Each workgroup (16 waves sharing one LDS histogram)
// takes a contiguous range of rows, one wave per row as in the row kernels
// below (CH chunks per lane issued together).
//   kFine = false: every key into a 32768-bin LDS histogram; the merge adds
//                  each group of 256 bins to coarse[key >> 8].
//   kFine = true:  keys with key >> 8 == prefix into a 256-bin LDS histogram,
//                  merged bin by bin into fine[].
template <bool kFast, bool kFine, int CH>
__global__ __launch_bounds__(kH16Threads) void select_hist16_kernel(
    const uint16_t* __restrict__ A, int64_t M, int64_t K, int64_t lda, int64_t rows_per_wg,
    const SelState* __restrict__ st, uint32_t* __restrict__ out) {
  constexpr int kBins = kFine ? kFineBins : kKeyBins16;
  __shared__ uint32_t h[kBins];
  const int t = threadIdx.x;
  for (int i = t; i < kBins / 4; i += kH16Threads)
    reinterpret_cast<uint4*>(h)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  const uint32_t prefix = kFine ? st->prefix : 0u;
  const int lane = t & (kWave - 1);
  const int64_t slab = int64_t(kWave) * CH * 8;
  const int64_t r0 = int64_t(blockIdx.x) * rows_per_wg;
  const int64_t r1 = (r0 + rows_per_wg < M) ? r0 + rows_per_wg : M;
  for (int64_t r = r0 + t / kWave; r < r1; r += kH16Waves) {
    const uint16_t* row = A + r * lda;
    for (int64_t c0 = 0; c0 < K; c0 += slab) {
      Vec8<BF16In> v[CH];
      load_wave_slab<BF16In, kFast, CH>(row, c0, K, v);
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        // K < 2^31: column offsets fit 32 bits. kFast: a chunk is wholly
        // inside the row or wholly past it.
        const int c = int(c0) + (j * kWave + lane) * 8;
        if (kFast && c >= int(K)) continue;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t key = BF16In::key(v[j].v[i]);
          if (kFast || c + i < int(K)) {
            if constexpr (kFine) {
              if ((key >> kFineBits) == prefix) atomicAdd(&h[key & (kFineBins - 1)], 1u);
            } else {
              atomicAdd(&h[key], 1u);
            }
          }
        }
      }
    }
  }
  __syncthreads();
  if constexpr (kFine) {
    for (int b = t; b < kFineBins; b += kH16Threads) {
      const uint32_t x = h[b];
      if (x) atomicAdd(&out[b], x);
    }
  } else {
    // Thread t sums bins [32t, 32t + 32), reading 16-byte words in a rotated
    // order to spread LDS banks; the 8 threads of one coarse bin are adjacent
    // lanes and reduce with shuffles before one atomic.
    constexpr int kPer = kKeyBins16 / kH16Threads;
    static_assert((kPer * 8) == kFineBins, "8 threads per coarse bin");
    uint32_t part = 0;
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i) {
      const int q4 = (i + t) & (kPer / 4 - 1);
      const uint4 x = *reinterpret_cast<const uint4*>(&h[t * kPer + q4 * 4]);
      part += x.x + x.y + x.z + x.w;
    }
    part += __shfl_xor(part, 1, kWave);
    part += __shfl_xor(part, 2, kWave);
    part += __shfl_xor(part, 4, kWave);
    if ((t & 7) == 0 && part) atomicAdd(&out[t >> 3], part);
  }
}

// ---------------------------------------------------------------------------
// Rows: count, scan, compact. One wave per row.
// ---------------------------------------------------------------------------
template <class In, int CH>
__device__ inline uint32_t count_above(const Vec8<In> (&v)[CH], uint32_t tkey) {
  // chunks past K are zero and a zero key never exceeds tkey
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) cnt += In::key(v[j].v[i]) > tkey ? 1u : 0u;
  return cnt;
}

// Per-row count of |a| > tau, written to row_ptr[i+1].
template <class In, bool kFast, int CH>
__global__ __launch_bounds__(kRowWaves * kWave) void count_rows_kernel(
    const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda,
    const SelState* __restrict__ st, int32_t* __restrict__ row_ptr) {
  if (blockIdx.x == 0 && threadIdx.x == 0) row_ptr[0] = 0;
  const uint32_t tkey = st->tau_key;
  const int64_t slab = int64_t(kWave) * CH * 8;
  const int64_t stride = int64_t(gridDim.x) * kRowWaves;
  for (int64_t r = int64_t(blockIdx.x) * kRowWaves + threadIdx.x / kWave; r < M; r += stride) {
    const typename In::T* row = A + r * lda;
    uint32_t cnt = 0;
    for (int64_t c0 = 0; c0 < K; c0 += slab) {
      Vec8<In> v[CH];
      load_wave_slab<In, kFast, CH>(row, c0, K, v);
      cnt += count_above<In, CH>(v, tkey);
    }
    cnt = wave_sum_u32(cnt);
    if ((threadIdx.x & (kWave - 1)) == 0) row_ptr[r + 1] = int32_t(cnt);
  }
}

// In-place inclusive scan of row_ptr[1..M] by one workgroup of 1024 threads,
// in tiles of kScanPer * 1024 rows: thread t owns rows kScanPer*t .. +kScanPer-1
// of a tile (loaded together, scanned serially), the thread totals are scanned
// across the wave with shuffles and across the 16 waves through LDS, and the
// carry of earlier tiles is added.
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 8;

__global__ __launch_bounds__(kScanThreads) void scan_rows_kernel(int32_t* __restrict__ row_ptr,
                                                                 int64_t M) {
  constexpr int kW = kScanThreads / kWave;
  __shared__ uint32_t wsum[kW];
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), w = t / kWave;
  int32_t* v = row_ptr + 1;
  uint32_t carry = 0;
  for (int64_t base = 0; base < M; base += int64_t(kScanPer) * kScanThreads) {
    const int64_t i0 = base + int64_t(t) * kScanPer;
    uint32_t x[kScanPer];
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) x[j] = (i0 + j < M) ? uint32_t(v[i0 + j]) : 0u;
#pragma unroll
    for (int j = 1; j < kScanPer; ++j) x[j] += x[j - 1];
    uint32_t wtot;
    const uint32_t wex = wave_exclusive_scan(x[kScanPer - 1], wtot);
    if (lane == 0) wsum[w] = wtot;
    __syncthreads();
    uint32_t before = carry + wex, all = 0;
    for (int y = 0; y < kW; ++y) {
      const uint32_t s = wsum[y];
      before += (y < w) ? s : 0u;
      all += s;
    }
    carry += all;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j)
      if (i0 + j < M) v[i0 + j] = int32_t(before + x[j]);
    __syncthreads();  // wsum is rewritten by the next tile
  }
}

// Write every |a| > tau entry of a row, ascending column, at row_ptr[i] + rank.
// The entries of chunk (j, lane) follow those of all chunks (j', *) with
// j' < j and (j, lane') with lane' < lane; per element position i of a chunk
// a wave ballot of the predicate gives, through mbcnt, how many entries the
// lower lanes hold at that position, so the rank needs no LDS and no barrier.
template <class In, bool kFast, int CH>
__global__ __launch_bounds__(kRowWaves * kWave) void compact_rows_kernel(
    const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda,
    const SelState* __restrict__ st, const float* __restrict__ tau_p,
    const int32_t* __restrict__ row_ptr, int64_t capacity, int32_t* __restrict__ out_row,
    int32_t* __restrict__ out_col, float* __restrict__ out_val) {
  const uint32_t tkey = st->tau_key;
  const float tau = *tau_p;
  const int lane = threadIdx.x & (kWave - 1);
  const int cap = int(capacity < INT32_MAX ? capacity : INT32_MAX);
  const int64_t slab = int64_t(kWave) * CH * 8;
  const int64_t stride = int64_t(gridDim.x) * kRowWaves;
  for (int64_t r = int64_t(blockIdx.x) * kRowWaves + threadIdx.x / kWave; r < M; r += stride) {
    const typename In::T* row = A + r * lda;
    int pos = row_ptr[r];
    for (int64_t c0 = 0; c0 < K; c0 += slab) {
      Vec8<In> v[CH];
      load_wave_slab<In, kFast, CH>(row, c0, K, v);
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        uint32_t lower = 0, total = 0, mine = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bool p = In::key(v[j].v[i]) > tkey;
          const uint64_t b = __ballot(p);
          lower = __builtin_amdgcn_mbcnt_hi(uint32_t(b >> 32),
                                            __builtin_amdgcn_mbcnt_lo(uint32_t(b), lower));
          total += uint32_t(__popcll(b));
          mine |= uint32_t(p) << i;
        }
        if (mine) {
          // positions and columns fit 32 bits (capacity < 2^31, K < 2^31)
          int p = pos + int(lower);
          const int c = int(c0) + (j * kWave + lane) * 8;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            // p < capacity always holds when tau is the true order statistic
            // (nnz <= n-1-k); the test only keeps a wrong tau from writing out of bounds.
            if (((mine >> i) & 1u) && p < cap) {
              const float a = In::widen(v[j].v[i]);
              out_row[p] = int32_t(r);
              out_col[p] = c + i;
              out_val[p] = __fsub_rn(a, copysignf(tau, a));
              ++p;
            }
          }
        }
        pos += int(total);
      }
    }
  }
}

// Histogram words after the 256-byte state: bfloat16 128 coarse + 256 fine
// bins; float32 one 2048-bin histogram per pass.
template <class In>
constexpr size_t hist_words() {
  if constexpr (In::kBytes == 2)
    return size_t(kCoarseBins + kFineBins);
  else
    return size_t(F32Digits::kPasses) * kHistBins;
}

__global__ void select_init_kernel(SelState* st, uint32_t* hist, int64_t nwords, int64_t k) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < nwords;
       i += int64_t(gridDim.x) * blockDim.x)
    hist[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    st->prefix = 0u;
    st->tau_key = 0u;
    st->krem = k;
  }
}

template <class In, bool kFast, int CH>
void launch_rows(const typename In::T* A, int64_t M, int64_t K, int64_t lda, SelState* st,
                 const float* tau, int64_t capacity, int32_t* row, int32_t* col, float* val,
                 int32_t* row_ptr, hipStream_t stream) {
  const unsigned blocks = row_blocks(M);
  count_rows_kernel<In, kFast, CH><<<blocks, kRowWaves * kWave, 0, stream>>>(A, M, K, lda, st,
                                                                            row_ptr);
  scan_rows_kernel<<<1, kScanThreads, 0, stream>>>(row_ptr, M);
  compact_rows_kernel<In, kFast, CH><<<blocks, kRowWaves * kWave, 0, stream>>>(
      A, M, K, lda, st, tau, row_ptr, capacity, row, col, val);
}

template <class In, bool kFast>
hipError_t run_select(const void* Ap, int64_t M, int64_t K, int64_t lda, int64_t k, float* tau,
                      int64_t capacity, int32_t* row, int32_t* col, float* val,
                      int32_t* row_ptr, void* ws, hipStream_t stream) {
  using T = typename In::T;
  const T* A = static_cast<const T*>(Ap);
  SelState* st = static_cast<SelState*>(ws);
  uint32_t* hist = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + 256);
  const int64_t nwords = int64_t(hist_words<In>());
  select_init_kernel<<<1, 256, 0, stream>>>(st, hist, nwords, k);
  if constexpr (In::kBytes == 2) {
    // one workgroup per CU (MI355X: 256), at least one row per wave
    int64_t wgs = (M + kH16Waves - 1) / kH16Waves;
    wgs = wgs < 256 ? wgs : 256;
    const int64_t per = (M + wgs - 1) / wgs;
    uint32_t* coarse = hist;
    uint32_t* fine = hist + kCoarseBins;
    const dim3 g(static_cast<unsigned>(wgs));
    switch (chunks_per_lane(K, 16)) {
#define FP4LIN_H16(CH)                                                                            \
  case CH:                                                                                        \
    select_hist16_kernel<kFast, false, CH><<<g, kH16Threads, 0, stream>>>(A, M, K, lda, per, st,  \
                                                                         coarse);                 \
    select_pick_kernel<<<1, 256, 0, stream>>>(st, coarse, kCoarseBits, 0, 16, tau);               \
    select_hist16_kernel<kFast, true, CH><<<g, kH16Threads, 0, stream>>>(A, M, K, lda, per, st,   \
                                                                        fine);                    \
    select_pick_kernel<<<1, 256, 0, stream>>>(st, fine, kFineBits, 1, 16, tau);                   \
    break;
      FP4LIN_H16(1)
      FP4LIN_H16(2)
      FP4LIN_H16(4)
      FP4LIN_H16(8)
      FP4LIN_H16(16)
#undef FP4LIN_H16
      default:
        return hipErrorInvalidValue;
    }
  } else {
    // Enough workgroups to fill the chip, each with several slabs so that the
    // per-group histogram merge stays small.
    const int64_t slab = int64_t(kHistThreads) * kHistCh * 8;
    const int64_t slabs = M * ((K + slab - 1) / slab);
    const int64_t g = slabs < 1024 ? slabs : 1024;
    for (int p = 0; p < F32Digits::kPasses; ++p) {
      const int shift = F32Digits::shift(p);
      const int width = F32Digits::width(p);
      const int hi = shift + width;
      select_hist_kernel<In, kFast><<<dim3(unsigned(g)), kHistThreads, 0, stream>>>(
          A, M, K, lda, st, shift, width, hi >= F32Digits::kKeyBits ? 32 : hi,
          hist + size_t(p) * kHistBins);
      select_pick_kernel<<<1, 256, 0, stream>>>(st, hist + size_t(p) * kHistBins, width,
                                                 p == F32Digits::kPasses - 1 ? 1 : 0, 0, tau);
    }
  }
  // rows up to 512 * CH columns in one slab (bfloat16: 8192, float32: 4096)
  constexpr int kMaxCh = In::kBytes == 2 ? 16 : 8;
  switch (chunks_per_lane(K, kMaxCh)) {
    case 1: launch_rows<In, kFast, 1>(A, M, K, lda, st, tau, capacity, row, col, val, row_ptr, stream); break;
    case 2: launch_rows<In, kFast, 2>(A, M, K, lda, st, tau, capacity, row, col, val, row_ptr, stream); break;
    case 4: launch_rows<In, kFast, 4>(A, M, K, lda, st, tau, capacity, row, col, val, row_ptr, stream); break;
    case 8: launch_rows<In, kFast, 8>(A, M, K, lda, st, tau, capacity, row, col, val, row_ptr, stream); break;
    case 16:
      if constexpr (kMaxCh >= 16) {
        launch_rows<In, kFast, 16>(A, M, K, lda, st, tau, capacity, row, col, val, row_ptr, stream);
        break;
      }
      return hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
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
  const bool fast = (reinterpret_cast<uintptr_t>(A) % 16 == 0) && ((lda * esz) % 16 == 0) &&
                    (K % 8 == 0);
  if (bf16)
    return fast ? run_select<BF16In, true>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws, stream)
                : run_select<BF16In, false>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws, stream);
  return fast ? run_select<F32In, true>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws, stream)
              : run_select<F32In, false>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws, stream);
}

}  // namespace fp4lin
