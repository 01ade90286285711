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
// digits equal the prefix found so far, and the digit that holds the remaining
// rank is appended to the prefix. Everything stays on the device; the host
// never reads a histogram.
//
// bfloat16 keys (15 bits): pass 1 builds a full 32768-bin histogram per
// workgroup in LDS (one 16-wave workgroup per CU), which spreads the densely
// populated magnitudes over many bins so that few lanes of an LDS atomic meet
// on one address, and writes only its 128 coarse sums (256 keys each), one row
// of partial sums per workgroup: merging every non-zero fine bin with
// device-wide atomics costs several times the pass itself. From its own rows
// the workgroup also estimates the coarse bin of rank k and saves the exact
// fine counts of that bin and its two neighbours. Pass 2 adds the partial rows
// up in every workgroup and finds the coarse bin that holds rank k. When every
// workgroup saved that bin or has no key in it, the fine histogram is the sum
// of the saved counts and A is not read again; otherwise pass 2 histograms the
// 256 keys of that bin from A. The row count that follows finds tau's key from
// the fine histogram in every wave. No kernel needs a cleared buffer on entry,
// so no launch is spent on set-up.
// float32 keys (31 bits) take three passes of 11, 11 and 9 bits with a
// 2048-bin histogram and a one-workgroup pick kernel after each.
//
// Then the entries with |a| > tau are counted per row, with one total per
// workgroup of rows; the compaction adds up the totals of the workgroups before
// its own, which gives row_ptr and the row-major positions without a separate
// scan. In the whole-layer forward, bfloat16 rows that fit one slab are also
// quantized token-wise by the compaction kernel, from the same registers.
#include "colquant.hpp"
#include "device_common.hpp"
#include "internal.hpp"

namespace fp4lin {

namespace {

struct SelState {
  uint32_t prefix;   // key bits decided so far (right-aligned)
  uint32_t tau_key;  // final key after the last pass
  int64_t krem;      // rank still to find inside the current prefix
};

// float32 passes: find the digit whose cumulative count passes the remaining
// rank and append it to the prefix; after the last pass the prefix is the key
// of tau, whose float bits are key << key_shift. One workgroup of 256 threads.
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
constexpr int kMaxH16Groups = 256;  // workgroups of the bfloat16 passes (one per CU)

// The coarse bin (key >> 8) that holds rank k. Thread t adds, for the four
// bins 4q .. 4q+3 (q = t % 32), the partial rows s, s+32, ... (s = t / 32);
// wave 0 adds the 32 sets up, two bins per lane, scans the 128 totals, and
// the lane whose range holds k names the bin. Workgroup 0 records the bin and
// the rank left inside it for the row count. All kH16Threads threads call it.
__device__ inline uint32_t coarse_pick(const uint32_t* __restrict__ part, int nparts,
                                       uint32_t k, SelState* __restrict__ st) {
  constexpr int kQuads = kCoarseBins / 4;
  constexpr int kSets = kH16Threads / kQuads;
  __shared__ uint4 red[kSets][kQuads];
  __shared__ uint32_t pick;
  const int t = threadIdx.x;
  const int q = t % kQuads, s = t / kQuads;
  if (t == 0) pick = 0u;
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  for (int p = s; p < nparts; p += kSets) {
    const uint4 x = reinterpret_cast<const uint4*>(part)[p * kQuads + q];
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  red[s][q] = acc;
  __syncthreads();
  if (t < kWave) {
    const uint32_t* r = reinterpret_cast<const uint32_t*>(&red[0][0]);
    uint32_t a = 0, b = 0;
    for (int y = 0; y < kSets; ++y) {
      a += r[y * kCoarseBins + 2 * t];
      b += r[y * kCoarseBins + 2 * t + 1];
    }
    // totals and ranks are below M*K < 2^32
    uint32_t total;
    const uint32_t ex = wave_exclusive_scan(a + b, total);
    if (k >= ex && k - ex < a + b) {
      const bool lo = k - ex < a;
      const uint32_t bin = uint32_t(2 * t) + (lo ? 0u : 1u);
      pick = bin;
      if (blockIdx.x == 0) {
        st->prefix = bin;
        st->krem = int64_t(lo ? k - ex : k - ex - a);
      }
    }
  }
  __syncthreads();
  return uint32_t(__builtin_amdgcn_readfirstlane(int(pick)));
}

// Both bfloat16 passes. Each workgroup (16 waves sharing one LDS histogram)
// takes a contiguous range of rows, one wave per row as in the row kernels
// below (CH chunks per lane issued together).
//   kFine = false: every key into a 32768-bin LDS histogram; workgroup b
//                  writes the sums of its 128 groups of 256 bins to
//                  part[b][0 .. 128), and workgroup 0 clears fine[]. The
//                  workgroup also estimates the coarse bin of rank k from its
//                  own rows (the bin where its cumulative count passes
//                  k * n_b / (M*K)) and saves the exact fine counts of that
//                  bin and its two neighbours: win[b] = first of the three,
//                  fwin[b][0 .. 768) = their 256-bin histograms.
//   kFine = true:  the workgroup finds the coarse bin from the nparts partial
//                  rows. If every coarse workgroup saved that bin or has no
//                  key in it, the saved counts add up to its whole fine
//                  histogram: workgroup 0 writes that sum to fine[] and A is
//                  not read again. Otherwise every workgroup histograms the
//                  keys of that bin (key >> 8 equal to it) in a 256-bin LDS
//                  histogram, merged bin by bin into fine[].
constexpr int kWinBins = 3;                     // coarse bins saved per workgroup
constexpr int kWinWords = kWinBins * kFineBins;

template <bool kFast, bool kFine, int CH>
__global__ __launch_bounds__(kH16Threads) void select_hist16_kernel(
    const uint16_t* __restrict__ A, int64_t M, int64_t K, int64_t lda, int64_t rows_per_wg,
    uint32_t* __restrict__ part, int nparts, uint32_t k, SelState* __restrict__ st,
    uint32_t* __restrict__ fine, uint32_t* __restrict__ win, uint32_t* __restrict__ fwin,
    uint32_t* __restrict__ clear, int64_t nclear) {
  constexpr int kBins = kFine ? kFineBins : kKeyBins16;
  __shared__ uint32_t h[kBins];
  const int t = threadIdx.x;
  for (int i = t; i < kBins / 4; i += kH16Threads)
    reinterpret_cast<uint4*>(h)[i] = make_uint4(0, 0, 0, 0);
  uint32_t prefix = 0u;
  if constexpr (kFine) {
    prefix = coarse_pick(part, nparts, k, st);
    int miss = 0;
    for (int w = t; w < nparts; w += kH16Threads)
      if (prefix - win[w] >= uint32_t(kWinBins) && part[size_t(w) * kCoarseBins + prefix] != 0u)
        miss = 1;
    if (!__syncthreads_or(miss)) {
      // fine[i] = sum over the coarse workgroups of their saved counts of
      // key (prefix << 8) | i; workgroup b forms bins b, b + gridDim.x, ...
      // and thread t reads coarse workgroup t's count.
      static_assert(kMaxH16Groups <= kH16Threads, "one coarse workgroup per thread");
      __shared__ uint32_t wred[kH16Waves];
      const uint32_t d = (t < nparts) ? prefix - win[t] : uint32_t(kWinBins);
      const int lane = t & (kWave - 1);
      for (int i = blockIdx.x; i < kFineBins; i += gridDim.x) {
        uint32_t x = (d < uint32_t(kWinBins)) ? fwin[size_t(t) * kWinWords + d * kFineBins + i] : 0u;
        x = wave_sum_u32(x);
        if (lane == 0) wred[t / kWave] = x;
        __syncthreads();
        if (t == 0) {
          uint32_t y = 0;
#pragma unroll
          for (int w = 0; w < kH16Waves; ++w) y += wred[w];
          fine[i] = y;
        }
        __syncthreads();
      }
      return;
    }
  } else {
    if (blockIdx.x == 0)
      for (int i = t; i < kFineBins; i += kH16Threads) fine[i] = 0u;
    // forward: the column maxima of W's quantization start from zero
    for (int64_t i = int64_t(blockIdx.x) * kH16Threads + t; i < nclear;
         i += int64_t(gridDim.x) * kH16Threads)
      clear[i] = 0u;
  }
  __syncthreads();
  const int lane = t & (kWave - 1);
  const int64_t slab = int64_t(kWave) * CH * 8;
  const int64_t r0 = int64_t(blockIdx.x) * rows_per_wg;
  const int64_t r1 = (r0 + rows_per_wg < M) ? r0 + rows_per_wg : M;
  for (int64_t r = r0 + __builtin_amdgcn_readfirstlane(t / kWave); r < r1; r += kH16Waves) {
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
      if (x) atomicAdd(&fine[b], x);
    }
  } else {
    // Thread t sums bins [32t, 32t + 32), reading 16-byte words in a rotated
    // order to spread LDS banks; the 8 threads of one coarse bin are adjacent
    // lanes and reduce with shuffles before one store.
    constexpr int kPer = kKeyBins16 / kH16Threads;
    static_assert((kPer * 8) == kFineBins, "8 threads per coarse bin");
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i) {
      const int q4 = (i + t) & (kPer / 4 - 1);
      const uint4 x = *reinterpret_cast<const uint4*>(&h[t * kPer + q4 * 4]);
      sum += x.x + x.y + x.z + x.w;
    }
    sum += __shfl_xor(sum, 1, kWave);
    sum += __shfl_xor(sum, 2, kWave);
    sum += __shfl_xor(sum, 4, kWave);
    __shared__ uint32_t csum[kCoarseBins];
    __shared__ uint32_t wbase;
    if ((t & 7) == 0) {
      part[size_t(blockIdx.x) * kCoarseBins + (t >> 3)] = sum;
      csum[t >> 3] = sum;
    }
    __syncthreads();
    if (t < kWave) {
      // this workgroup's estimate of the coarse bin of rank k (lane t owns
      // bins 2t and 2t+1); its counts are below M*K < 2^32
      const uint32_t a = csum[2 * t], b = csum[2 * t + 1];
      uint32_t nb;
      const uint32_t ex = wave_exclusive_scan(a + b, nb);
      const uint32_t target = uint32_t(uint64_t(k) * nb / uint64_t(M * K));
      const uint64_t hit = __ballot(target >= ex && target - ex < a + b);
      uint32_t bin = 0u;
      if (hit) {
        const int l = __builtin_ctzll(hit);
        const uint32_t exl = uint32_t(__shfl(int(ex), l, kWave));
        const uint32_t al = uint32_t(__shfl(int(a), l, kWave));
        bin = uint32_t(2 * l) + (target - exl < al ? 0u : 1u);
      }
      const uint32_t first =
          bin < 1u ? 0u : (bin + kWinBins - 1 > kCoarseBins ? kCoarseBins - kWinBins : bin - 1u);
      if (t == 0) {
        wbase = first;
        win[blockIdx.x] = first;
      }
    }
    __syncthreads();
    const uint32_t first = wbase;
    for (int i = t; i < kWinWords; i += kH16Threads)
      fwin[size_t(blockIdx.x) * kWinWords + i] = h[first * kFineBins + i];
  }
}

// tau's key in every wave: the coarse bin recorded in st followed by the fine
// bin that holds the rank left inside it. Lane l owns fine bins 4l .. 4l+3.
__device__ inline uint32_t fine_pick(const SelState* st, const uint32_t* __restrict__ fine) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint4 h = reinterpret_cast<const uint4*>(fine)[lane];
  const uint32_t s = h.x + h.y + h.z + h.w;
  uint32_t total;
  const uint32_t ex = wave_exclusive_scan(s, total);
  const uint32_t krem = uint32_t(st->krem);
  const uint32_t prefix = st->prefix;
  const uint32_t r = krem - ex;  // meaningful in the lane that holds krem
  uint32_t j = 3;
  if (r < h.x)
    j = 0;
  else if (r - h.x < h.y)
    j = 1;
  else if (r - h.x - h.y < h.z)
    j = 2;
  const uint64_t mine = __ballot(krem >= ex && r < s);
  const int src = mine ? __builtin_ctzll(mine) : 0;
  const uint32_t key = (prefix << kFineBits) | (uint32_t(4 * lane) + j);
  // uniform: kept in a scalar register for the compares
  return uint32_t(__builtin_amdgcn_readfirstlane(__shfl(int(key), src, kWave)));
}

// ---------------------------------------------------------------------------
// Rows: count, compact. One wave per row. Workgroup g owns the rows
// [g*R, min(M, (g+1)*R)), R = kRowWaves * rpw; wave w takes rows
// g*R + w + kRowWaves*i, so the workgroup walks its range in batches of
// kRowWaves consecutive rows.
// ---------------------------------------------------------------------------
constexpr int64_t kMaxRowGroups = 2048;

__host__ inline int64_t rows_per_wave(int64_t M) {
  return (M + kRowWaves * kMaxRowGroups - 1) / (kRowWaves * kMaxRowGroups);
}

__host__ inline int64_t row_groups(int64_t M) {
  const int64_t R = kRowWaves * rows_per_wave(M);
  return (M + R - 1) / R;
}

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

// Per-row count of |a| > tau into cnt[r], and the workgroup's total into
// gsum[blockIdx.x]. kPick (bfloat16): tau's key comes from the fine histogram
// and workgroup 0 records it in st and tau; otherwise it is read from st.
// (Looking the key up between the first row's loads and their use measured
// slower: it costs registers.)
template <class In, bool kFast, int CH, bool kPick>
__device__ __attribute__((always_inline)) inline void count_rows_body(
    int64_t bid, const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda,
    int64_t rpw, SelState* st, const uint32_t* __restrict__ fine, float* __restrict__ tau,
    uint32_t* __restrict__ cnt, uint32_t* __restrict__ gsum) {
  __shared__ uint32_t wsum[kRowWaves];
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);  // wave-uniform
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t R = int64_t(kRowWaves) * rpw;
  const int64_t r0 = bid * R;
  const int64_t r1 = (r0 + R < M) ? r0 + R : M;
  const int64_t slab = int64_t(kWave) * CH * 8;
  uint32_t tkey;
  if constexpr (kPick) {
    tkey = fine_pick(st, fine);
    if (bid == 0 && threadIdx.x == 0) {
      st->tau_key = tkey;
      *tau = In::key_to_float(tkey);
    }
  } else {
    tkey = st->tau_key;
  }
  uint32_t total = 0;
  for (int64_t r = r0 + w; r < r1; r += kRowWaves) {
    const typename In::T* row = A + r * lda;
    uint32_t c = 0;
    for (int64_t c0 = 0; c0 < K; c0 += slab) {
      Vec8<In> v[CH];
      load_wave_slab<In, kFast, CH>(row, c0, K, v);
      c += count_above<In, CH>(v, tkey);
    }
    c = wave_sum_u32(c);
    total += c;
    if (lane == 0) cnt[r] = c;
  }
  if (lane == 0) wsum[w] = total;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < kRowWaves; ++i) s += wsum[i];
    gsum[bid] = s;
  }
}

template <class In, bool kFast, int CH, bool kPick>
__global__ __launch_bounds__(kRowWaves * kWave) void count_rows_kernel(
    const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda, int64_t rpw,
    SelState* st, const uint32_t* __restrict__ fine, float* __restrict__ tau,
    uint32_t* __restrict__ cnt, uint32_t* __restrict__ gsum) {
  count_rows_body<In, kFast, CH, kPick>(blockIdx.x, A, M, K, lda, rpw, st, fine, tau, cnt, gsum);
}

// Write every |a| > tau entry of a row, ascending column, from position pos.
// The entries of chunk (j, lane) follow those of all chunks (j', *) with
// j' < j and (j, lane') with lane' < lane; per element position i of a chunk
// a wave ballot of the predicate gives, through mbcnt, how many entries the
// lower lanes hold at that position, so the rank needs no LDS and no barrier.
template <class In, int CH>
__device__ inline void compact_slab(const Vec8<In> (&v)[CH], int64_t c0, int64_t r, uint32_t tkey,
                                    float tau, uint32_t& pos, uint32_t cap,
                                    int32_t* __restrict__ out_row, int32_t* __restrict__ out_col,
                                    float* __restrict__ out_val) {
  const int lane = threadIdx.x & (kWave - 1);
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
    // One store per array for each set bit of the lane, lowest first: a lane
    // rarely holds more than one entry of a chunk, so the wave usually
    // stores once instead of once per element position.
    uint32_t p = pos + lower;  // positions below capacity < 2^31, columns below K < 2^31
    const int c = int(c0) + (j * kWave + lane) * 8;
    while (mine) {
      const int i = __builtin_ctz(mine);
      mine &= mine - 1u;
      typename In::T x = v[j].v[0];
#pragma unroll
      for (int q = 1; q < 8; ++q) x = (i == q) ? v[j].v[q] : x;
      // p < cap always holds when tau is the true order statistic
      // (nnz <= n-1-k); the test only keeps a wrong tau from writing out of bounds.
      if (p < cap) {
        const float a = In::widen(x);
        out_row[p] = int32_t(r);
        out_col[p] = c + i;
        out_val[p] = __fsub_rn(a, copysignf(tau, a));
      }
      ++p;
    }
    pos += total;
  }
}

// Row-major COO and row_ptr. The workgroup's first position is the sum of the
// totals of the workgroups before it; within a batch of kRowWaves rows a wave
// adds the counts of the lower rows of the batch, so waves need no barrier
// after the first.
template <class In, bool kFast, int CH>
__global__ __launch_bounds__(kRowWaves * kWave) void compact_rows_kernel(
    const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda, int64_t rpw,
    const SelState* __restrict__ st, const float* __restrict__ tau_p,
    const uint32_t* __restrict__ cnt, const uint32_t* __restrict__ gsum, int64_t capacity,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ out_row, int32_t* __restrict__ out_col,
    float* __restrict__ out_val) {
  __shared__ uint32_t wsum[kRowWaves];
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);  // wave-uniform
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t R = int64_t(kRowWaves) * rpw;
  const int64_t r0 = int64_t(blockIdx.x) * R;
  const int64_t r1 = (r0 + R < M) ? r0 + R : M;
  const int64_t slab = int64_t(kWave) * CH * 8;
  const uint32_t tkey = st->tau_key;
  const float tau = *tau_p;
  const uint32_t cap = uint32_t(capacity < INT32_MAX ? capacity : INT32_MAX);
  if (blockIdx.x == 0 && threadIdx.x == 0) row_ptr[0] = 0;
  // entries of the workgroups before this one
  uint32_t base = 0;
  {
    uint32_t s = 0;
    for (int64_t g = threadIdx.x; g < int64_t(blockIdx.x); g += kRowWaves * kWave) s += gsum[g];
    s = wave_sum_u32(s);
    if (lane == 0) wsum[w] = s;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRowWaves; ++i) base += wsum[i];
  }
  for (int64_t rb = r0; rb < r1; rb += kRowWaves) {
    const int64_t r = rb + w;
    uint32_t before = 0, all = 0, own = 0;
#pragma unroll
    for (int j = 0; j < kRowWaves; ++j) {
      const uint32_t cj = (rb + j < r1) ? cnt[rb + j] : 0u;
      before += (j < w) ? cj : 0u;
      own = (j == w) ? cj : own;
      all += cj;
    }
    if (r < r1) {
      const typename In::T* row = A + r * lda;
      uint32_t pos = base + before;
      for (int64_t c0 = 0; c0 < K; c0 += slab) {
        Vec8<In> v[CH];
        load_wave_slab<In, kFast, CH>(row, c0, K, v);
        compact_slab<In, CH>(v, c0, r, tkey, tau, pos, cap, out_row, out_col, out_val);
      }
      if (lane == 0) row_ptr[r + 1] = int32_t(base + before + own);
    }
    base += all;
  }
}

// Compaction from a bfloat16 row held as raw 16-byte words (element i of a
// chunk is the low half of word i / 2 for even i, the high half for odd i),
// ranked as in compact_slab.
template <int CH>
__device__ inline void compact_words(const uint4 (&wv)[CH], int64_t r, uint32_t tkey, float tau,
                                     uint32_t& pos, uint32_t cap, int32_t* __restrict__ out_row,
                                     int32_t* __restrict__ out_col, float* __restrict__ out_val) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const uint32_t q[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
    uint32_t lower = 0, total = 0, mine = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t key = ((i & 1) ? (q[i >> 1] >> 16) : q[i >> 1]) & 0x7fffu;
      const bool p = key > tkey;
      const uint64_t b = __ballot(p);
      lower = __builtin_amdgcn_mbcnt_hi(uint32_t(b >> 32),
                                        __builtin_amdgcn_mbcnt_lo(uint32_t(b), lower));
      total += uint32_t(__popcll(b));
      mine |= uint32_t(p) << i;
    }
    uint32_t p = pos + lower;  // positions below capacity < 2^31, columns below K < 2^31
    const int c = (j * kWave + lane) * 8;
    while (mine) {
      const int i = __builtin_ctz(mine);
      mine &= mine - 1u;
      const int h = i >> 1;
      const uint32_t word = h == 0 ? q[0] : (h == 1 ? q[1] : (h == 2 ? q[2] : q[3]));
      // p < cap always holds when tau is the true order statistic
      if (p < cap) {
        const float a = __uint_as_float((i & 1) ? (word & 0xffff0000u) : (word << 16));
        out_row[p] = int32_t(r);
        out_col[p] = c + i;
        out_val[p] = __fsub_rn(a, copysignf(tau, a));
      }
      ++p;
    }
    pos += total;
  }
}

// Forward path, 16-byte aligned bfloat16 rows with K % 8 == 0 whose padded
// length fits one slab: the compaction of compact_rows_kernel and the
// token-wise quantization of the row clamped to tau (quantize_bf16_row) from
// one read of A; with kMx, its micro-scaled quantization instead
// (quantize_bf16_row_mx, block scales into the step-major array Xs).
template <int CH, bool kMx = false>
__device__ __attribute__((always_inline)) inline void compact_quantize_rows_body(
    int64_t bid, const uint16_t* __restrict__ A, int64_t M, int64_t K, int64_t lda, int64_t rpw,
    const SelState* __restrict__ st, const float* __restrict__ tau_p,
    const uint32_t* __restrict__ cnt, const uint32_t* __restrict__ gsum, int64_t capacity,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ out_row, int32_t* __restrict__ out_col,
    float* __restrict__ out_val, uint8_t* __restrict__ Xq, int64_t ldq, float* __restrict__ sX,
    uint8_t* __restrict__ Xs = nullptr) {
  __shared__ uint32_t wsum[kRowWaves];
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);  // wave-uniform
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t R = int64_t(kRowWaves) * rpw;
  const int64_t r0 = bid * R;
  const int64_t r1 = (r0 + R < M) ? r0 + R : M;
  const uint32_t tkey = st->tau_key;
  const float tau = *tau_p;
  const uint32_t cap = uint32_t(capacity < INT32_MAX ? capacity : INT32_MAX);
  if (bid == 0 && threadIdx.x == 0) row_ptr[0] = 0;
  // entries of the workgroups before this one
  uint32_t base = 0;
  {
    uint32_t s = 0;
    for (int64_t g = threadIdx.x; g < bid; g += kRowWaves * kWave) s += gsum[g];
    s = wave_sum_u32(s);
    if (lane == 0) wsum[w] = s;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRowWaves; ++i) base += wsum[i];
  }
  for (int64_t rb = r0; rb < r1; rb += kRowWaves) {
    const int64_t r = rb + w;
    uint32_t before = 0, all = 0, own = 0;
#pragma unroll
    for (int j = 0; j < kRowWaves; ++j) {
      const uint32_t cj = (rb + j < r1) ? cnt[rb + j] : 0u;
      before += (j < w) ? cj : 0u;
      own = (j == w) ? cj : own;
      all += cj;
    }
    if (r < r1) {
      const uint16_t* row = A + r * lda;
      uint4 wv[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int64_t c = (int64_t(j) * kWave + lane) * 8;
        wv[j] = *reinterpret_cast<const uint4*>(row + (c < K ? c : K - 8));
        if (c >= K) wv[j] = make_uint4(0, 0, 0, 0);
      }
      uint32_t pos = base + before;
      compact_words<CH>(wv, r, tkey, tau, pos, cap, out_row, out_col, out_val);
      if constexpr (kMx)
        quantize_bf16_row_mx<CH>(wv, ldq * 2, tau, Xq + r * ldq, Xs, M, r);
      else
        quantize_bf16_row<CH>(wv, ldq * 2, tau, Xq + r * ldq, sX + r);
      if (lane == 0) row_ptr[r + 1] = int32_t(base + before + own);
    }
    base += all;
  }
}

template <int CH, bool kMx = false>
__global__ __launch_bounds__(kRowWaves * kWave) void compact_quantize_rows_kernel(
    const uint16_t* __restrict__ A, int64_t M, int64_t K, int64_t lda, int64_t rpw,
    const SelState* __restrict__ st, const float* __restrict__ tau_p,
    const uint32_t* __restrict__ cnt, const uint32_t* __restrict__ gsum, int64_t capacity,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ out_row, int32_t* __restrict__ out_col,
    float* __restrict__ out_val, uint8_t* __restrict__ Xq, int64_t ldq, float* __restrict__ sX,
    uint8_t* __restrict__ Xs) {
  compact_quantize_rows_body<CH, kMx>(blockIdx.x, A, M, K, lda, rpw, st, tau_p, cnt, gsum,
                                      capacity, row_ptr, out_row, out_col, out_val, Xq, ldq, sX,
                                      Xs);
}

// ---------------------------------------------------------------------------
// Whole-layer forward, bfloat16 with aligned rows: the quantization of W has
// no dependence on the select, so its two passes share launches with the
// select's row kernels (the column maxima with the row count, the codes with
// the compaction), and its cleared maxima come from the coarse pass.
// ---------------------------------------------------------------------------
// Launch index b of a pair launch of na + nb workgroups belongs to the first
// body when floor((b+1)*na/(na+nb)) > floor(b*na/(na+nb)); the two kinds are
// interleaved in proportion, and each gets the indexes 0 .. n-1 once.
__device__ inline bool pair_first(int64_t b, int64_t na, int64_t nb, int64_t& idx) {
  const int64_t t = na + nb;
  const int64_t lo = b * na / t, hi = (b + 1) * na / t;
  idx = hi > lo ? lo : b - lo;
  return hi > lo;
}

struct ColQuantArgs {
  const uint16_t* W;
  int64_t K, N, ldw;
  uint32_t* colmax;
  uint8_t* Wq;
  int64_t ldq;
  float* sW;
};

template <int CH>
__global__ __launch_bounds__(kRowWaves * kWave) void count_colmax_kernel(
    const uint16_t* __restrict__ A, int64_t M, int64_t K, int64_t lda, int64_t rpw, SelState* st,
    const uint32_t* __restrict__ fine, float* __restrict__ tau, uint32_t* __restrict__ cnt,
    uint32_t* __restrict__ gsum, int64_t na, ColQuantArgs cq, int64_t gx, int64_t nb) {
  int64_t i;
  if (pair_first(blockIdx.x, na, nb, i))
    count_rows_body<BF16In, true, CH, true>(i, A, M, K, lda, rpw, st, fine, tau, cnt, gsum);
  else
    colmax_body<BF16In, true>(i % gx, i / gx, cq.W, cq.K, cq.N, cq.ldw, cq.colmax);
}

template <int CH>
__global__ __launch_bounds__(kRowWaves * kWave) void compact_qcols_kernel(
    const uint16_t* __restrict__ A, int64_t M, int64_t K, int64_t lda, int64_t rpw,
    const SelState* __restrict__ st, const float* __restrict__ tau_p,
    const uint32_t* __restrict__ cnt, const uint32_t* __restrict__ gsum, int64_t capacity,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ out_row, int32_t* __restrict__ out_col,
    float* __restrict__ out_val, uint8_t* __restrict__ Xq, int64_t ldq, float* __restrict__ sX,
    int64_t na, ColQuantArgs cq, int64_t gx, int64_t nb) {
  int64_t i;
  if (pair_first(blockIdx.x, na, nb, i))
    compact_quantize_rows_body<CH>(i, A, M, K, lda, rpw, st, tau_p, cnt, gsum, capacity, row_ptr,
                                   out_row, out_col, out_val, Xq, ldq, sX);
  else
    quantize_cols_body<BF16In, true>(i % gx, i / gx, cq.W, cq.K, cq.N, cq.ldw, cq.colmax, cq.Wq,
                                     cq.ldq, cq.sW);
}

// Words after the 256-byte state: bfloat16 has the coarse partial rows, the
// fine histogram, and per coarse workgroup its first saved bin and its saved
// fine counts; float32 one 2048-bin histogram per pass. Both then hold the
// row-group totals and the per-row counts.
template <class In>
constexpr size_t hist_words() {
  if constexpr (In::kBytes == 2)
    return size_t(kMaxH16Groups) * (kCoarseBins + 1 + kWinWords) + kFineBins;
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

// Quantization outputs of the forward path: when Xq is set and the rows
// qualify, the compaction also quantizes A and sets *done; token-wise into sX,
// or micro-scaled into the block scales Xs when Xs is set.
struct RowQuant {
  uint8_t* Xq;
  int64_t ldq;
  float* sX;
  bool* done;
  uint8_t* Xs;
};

template <class In, bool kFast, int CH, bool kPick>
void launch_rows(const typename In::T* A, int64_t M, int64_t K, int64_t lda, SelState* st,
                 const uint32_t* fine, float* tau, uint32_t* gsum, uint32_t* cnt,
                 int64_t capacity, int32_t* row, int32_t* col, float* val, int32_t* row_ptr,
                 const RowQuant& rq, hipStream_t stream) {
  const int64_t rpw = rows_per_wave(M);
  const dim3 g(static_cast<unsigned>(row_groups(M)));
  count_rows_kernel<In, kFast, CH, kPick><<<g, kRowWaves * kWave, 0, stream>>>(
      A, M, K, lda, rpw, st, fine, tau, cnt, gsum);
  if constexpr (In::kBytes == 2 && kFast) {
    // padded row length within one slab of 16 chunks per lane
    if (rq.Xq != nullptr && rq.ldq * 2 <= int64_t(kWave) * 16 * 8) {
      const uint16_t* A16 = reinterpret_cast<const uint16_t*>(A);
      switch (chunks_per_lane(rq.ldq * 2, 16)) {
#define FP4LIN_CQ(CQ)                                                                            \
  case CQ:                                                                                       \
    if (rq.Xs != nullptr)                                                                        \
      compact_quantize_rows_kernel<CQ, true><<<g, kRowWaves * kWave, 0, stream>>>(               \
          A16, M, K, lda, rpw, st, tau, cnt, gsum, capacity, row_ptr, row, col, val, rq.Xq,      \
          rq.ldq, rq.sX, rq.Xs);                                                                 \
    else                                                                                         \
      compact_quantize_rows_kernel<CQ><<<g, kRowWaves * kWave, 0, stream>>>(                     \
          A16, M, K, lda, rpw, st, tau, cnt, gsum, capacity, row_ptr, row, col, val, rq.Xq,      \
          rq.ldq, rq.sX, nullptr);                                                               \
    *rq.done = true;                                                                             \
    return;
        FP4LIN_CQ(1)
        FP4LIN_CQ(2)
        FP4LIN_CQ(4)
        FP4LIN_CQ(8)
        FP4LIN_CQ(16)
#undef FP4LIN_CQ
        default:
          break;
      }
    }
  }
  compact_rows_kernel<In, kFast, CH><<<g, kRowWaves * kWave, 0, stream>>>(
      A, M, K, lda, rpw, st, tau, cnt, gsum, capacity, row_ptr, row, col, val);
}

template <class In, bool kFast, bool kPick>
hipError_t rows_dispatch(const typename In::T* A, int64_t M, int64_t K, int64_t lda,
                         SelState* st, const uint32_t* fine, float* tau, uint32_t* gsum,
                         uint32_t* cnt, int64_t capacity, int32_t* row, int32_t* col, float* val,
                         int32_t* row_ptr, const RowQuant& rq, hipStream_t stream) {
  // rows up to 512 * CH columns in one slab (bfloat16: 8192, float32: 4096)
  constexpr int kMaxCh = In::kBytes == 2 ? 16 : 8;
  switch (chunks_per_lane(K, kMaxCh)) {
#define FP4LIN_ROWS(CH)                                                                          \
  case CH:                                                                                       \
    launch_rows<In, kFast, CH, kPick>(A, M, K, lda, st, fine, tau, gsum, cnt, capacity, row,    \
                                      col, val, row_ptr, rq, stream);                            \
    return hipSuccess;
    FP4LIN_ROWS(1)
    FP4LIN_ROWS(2)
    FP4LIN_ROWS(4)
    FP4LIN_ROWS(8)
#undef FP4LIN_ROWS
    case 16:
      if constexpr (kMaxCh >= 16) {
        launch_rows<In, kFast, 16, kPick>(A, M, K, lda, st, fine, tau, gsum, cnt, capacity, row,
                                          col, val, row_ptr, rq, stream);
        return hipSuccess;
      }
      return hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
}

// The bfloat16 select's workspace: state, then the coarse partial rows, the
// fine histogram, the saved windows, the row-group totals and the row counts.
struct H16Work {
  SelState* st;
  uint32_t *part, *fine, *win, *fwin, *gsum, *cnt;
  explicit H16Work(void* ws) {
    st = static_cast<SelState*>(ws);
    part = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + 256);
    fine = part + size_t(kMaxH16Groups) * kCoarseBins;
    win = fine + kFineBins;
    fwin = win + kMaxH16Groups;
    gsum = part + hist_words<BF16In>();
    cnt = gsum + kMaxRowGroups;
  }
};

// The two bfloat16 histogram passes (the coarse one also clears nclear words
// at clear).
template <bool kFast>
hipError_t launch_hist16(const uint16_t* A, int64_t M, int64_t K, int64_t lda, int64_t k,
                         const H16Work& w, uint32_t* clear, int64_t nclear, hipStream_t stream) {
  // one workgroup per CU (MI355X: 256), at least one row per wave
  int64_t wgs = (M + kH16Waves - 1) / kH16Waves;
  wgs = wgs < kMaxH16Groups ? wgs : kMaxH16Groups;
  const int64_t per = (M + wgs - 1) / wgs;
  const dim3 g(static_cast<unsigned>(wgs));
  // k < M*K < 2^32
  const uint32_t k32 = uint32_t(k);
  switch (chunks_per_lane(K, 16)) {
#define FP4LIN_H16(CH)                                                                           \
  case CH:                                                                                       \
    select_hist16_kernel<kFast, false, CH><<<g, kH16Threads, 0, stream>>>(                       \
        A, M, K, lda, per, w.part, 0, k32, w.st, w.fine, w.win, w.fwin, clear, nclear);          \
    select_hist16_kernel<kFast, true, CH><<<g, kH16Threads, 0, stream>>>(                        \
        A, M, K, lda, per, w.part, int(wgs), k32, w.st, w.fine, w.win, w.fwin, nullptr, 0);      \
    return hipSuccess;
    FP4LIN_H16(1)
    FP4LIN_H16(2)
    FP4LIN_H16(4)
    FP4LIN_H16(8)
    FP4LIN_H16(16)
#undef FP4LIN_H16
    default:
      return hipErrorInvalidValue;
  }
}

template <class In, bool kFast>
hipError_t run_select(const void* Ap, int64_t M, int64_t K, int64_t lda, int64_t k, float* tau,
                      int64_t capacity, int32_t* row, int32_t* col, float* val,
                      int32_t* row_ptr, void* ws, const RowQuant& rq, hipStream_t stream) {
  using T = typename In::T;
  const T* A = static_cast<const T*>(Ap);
  SelState* st = static_cast<SelState*>(ws);
  uint32_t* hist = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + 256);
  uint32_t* gsum = hist + hist_words<In>();
  uint32_t* cnt = gsum + kMaxRowGroups;
  hipError_t e = hipSuccess;
  if constexpr (In::kBytes == 2) {
    const H16Work w(ws);
    e = launch_hist16<kFast>(A, M, K, lda, k, w, nullptr, 0, stream);
    if (e != hipSuccess) return e;
    e = rows_dispatch<In, kFast, true>(A, M, K, lda, st, w.fine, tau, gsum, cnt, capacity, row,
                                       col, val, row_ptr, rq, stream);
  } else {
    select_init_kernel<<<1, 256, 0, stream>>>(st, hist, int64_t(hist_words<In>()), k);
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
    e = rows_dispatch<In, kFast, false>(A, M, K, lda, st, nullptr, tau, gsum, cnt, capacity, row,
                                        col, val, row_ptr, rq, stream);
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace

size_t select_workspace_bytes(bool bf16, int64_t M) {
  const size_t words = (bf16 ? hist_words<BF16In>() : hist_words<F32In>()) +
                       size_t(kMaxRowGroups) + size_t(M);
  return 256 + words * 4;
}

hipError_t launch_outlier_select(const void* A, bool bf16, int64_t M, int64_t K, int64_t lda,
                                 int64_t k, float* tau, int64_t capacity, int32_t* row,
                                 int32_t* col, float* val, int32_t* row_ptr, void* ws,
                                 hipStream_t stream, uint8_t* Xq, int64_t ldq, float* sX,
                                 bool* quantized, uint8_t* Xs) {
  bool done = false;
  const RowQuant rq{quantized != nullptr ? Xq : nullptr, ldq, sX, &done, Xs};
  const int esz = bf16 ? 2 : 4;
  const bool fast = (reinterpret_cast<uintptr_t>(A) % 16 == 0) && ((lda * esz) % 16 == 0) &&
                    (K % 8 == 0);
  hipError_t e;
  if (bf16)
    e = fast ? run_select<BF16In, true>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws, rq, stream)
             : run_select<BF16In, false>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws, rq, stream);
  else
    e = fast ? run_select<F32In, true>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws, rq, stream)
             : run_select<F32In, false>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws, rq, stream);
  if (quantized != nullptr) *quantized = done && e == hipSuccess;
  return e;
}

namespace {

template <int CH>
hipError_t forward_front(const uint16_t* A, int64_t M, int64_t K, int64_t lda, int64_t k,
                         float* tau, int64_t capacity, int32_t* row, int32_t* col, float* val,
                         int32_t* row_ptr, void* ws, uint8_t* Aq, int64_t ldq, float* sA,
                         const ColQuantArgs& cq, bool* w_done, hipStream_t stream) {
  const H16Work w(ws);
  hipError_t e = launch_hist16<true>(A, M, K, lda, k, w, cq.colmax, cq.N, stream);
  if (e != hipSuccess) return e;
  const int64_t rpw = rows_per_wave(M);
  const int64_t na = row_groups(M);
  if constexpr (CH > 8) {
    // the 16-chunk row kernels need up to 162 VGPRs (three waves per SIMD),
    // which would hold the paired column passes to the same occupancy (measured
    // slower): the row kernels run alone and W is quantized afterwards
    count_rows_kernel<BF16In, true, CH, true><<<dim3(unsigned(na)), kRowWaves * kWave, 0,
                                                stream>>>(A, M, K, lda, rpw, w.st, w.fine, tau,
                                                          w.cnt, w.gsum);
    compact_quantize_rows_kernel<CH><<<dim3(unsigned(na)), kRowWaves * kWave, 0, stream>>>(
        A, M, K, lda, rpw, w.st, tau, w.cnt, w.gsum, capacity, row_ptr, row, col, val, Aq, ldq,
        sA, nullptr);
    *w_done = false;
    return hipGetLastError();
  } else {
    // column maxima: 512-column strips x 64-row splits
    const int64_t gx1 = (cq.N + kColStrip - 1) / kColStrip;
    const int64_t nb1 = gx1 * ((cq.K + kColRows - 1) / kColRows);
    count_colmax_kernel<CH><<<dim3(unsigned(na + nb1)), kRowWaves * kWave, 0, stream>>>(
        A, M, K, lda, rpw, w.st, w.fine, tau, w.cnt, w.gsum, na, cq, gx1, nb1);
    // codes: 128-column x 128-row tiles
    const int64_t gx2 = (cq.N + kTN - 1) / kTN;
    const int64_t nb2 = gx2 * ((cq.ldq * 2) / kTK);
    compact_qcols_kernel<CH><<<dim3(unsigned(na + nb2)), kRowWaves * kWave, 0, stream>>>(
        A, M, K, lda, rpw, w.st, tau, w.cnt, w.gsum, capacity, row_ptr, row, col, val, Aq, ldq,
        sA, na, cq, gx2, nb2);
    *w_done = true;
    return hipGetLastError();
  }
}

}  // namespace

bool forward_front_supported(const void* A, const void* W, bool bf16, int64_t K, int64_t lda,
                             int64_t ldw) {
  const bool a_fast = (reinterpret_cast<uintptr_t>(A) % 16 == 0) && ((lda * 2) % 16 == 0) &&
                      (K % 8 == 0);
  const bool w_aligned = (reinterpret_cast<uintptr_t>(W) % 16 == 0) && ((ldw * 2) % 16 == 0);
  // the padded row fits one slab of 16 chunks per lane
  const int64_t kp = (K + 127) / 128 * 128;
  return bf16 && a_fast && w_aligned && kp <= int64_t(kWave) * 16 * 8;
}

hipError_t launch_forward_front(const void* A, int64_t M, int64_t K, int64_t lda, int64_t k,
                                float* tau, int64_t capacity, int32_t* row, int32_t* col,
                                float* val, int32_t* row_ptr, void* ws, uint8_t* Aq, int64_t ldq,
                                float* sA, const void* W, int64_t N, int64_t ldw, uint8_t* Wq,
                                float* sW, uint32_t* colmax, bool* w_done, hipStream_t stream) {
  const uint16_t* A16 = static_cast<const uint16_t*>(A);
  const ColQuantArgs cq{static_cast<const uint16_t*>(W), K, N, ldw, colmax, Wq, ldq, sW};
  // the padded row length (a multiple of 128) needs no more chunks than K:
  // 512 * CH is a multiple of 128
  const int ch = chunks_per_lane(K, 16);
  if (chunks_per_lane(ldq * 2, 16) != ch) return hipErrorInvalidValue;
  switch (ch) {
#define FP4LIN_FF(CH)                                                                            \
  case CH:                                                                                       \
    return forward_front<CH>(A16, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws, Aq,   \
                             ldq, sA, cq, w_done, stream);
    FP4LIN_FF(1)
    FP4LIN_FF(2)
    FP4LIN_FF(4)
    FP4LIN_FF(8)
    FP4LIN_FF(16)
#undef FP4LIN_FF
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fp4lin
