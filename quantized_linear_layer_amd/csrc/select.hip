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
// scan. In the whole-layer forward the count also records each row's amax
// clamped to tau and the compaction quantizes A from the slabs it holds, while
// W's quantization runs in the same launches.
#include <type_traits>

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

template <bool kFast, bool kFine, int CH, bool kStream>
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
  // The wave's slabs in order (its rows r0 + w, r0 + w + 16, ..., each in
  // slabs of CH chunk sweeps), two register buffers used in turn: the loads
  // of the next slab are issued before the current one is counted, so they
  // are in flight while its atomics run. Past the wave's last slab the
  // prefetch repeats the current one and is not counted.
  auto hist = [&](int64_t c0, const Vec8<BF16In>(&v)[CH]) __attribute__((always_inline)) {
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
  };
  // the slab after (r, c0), or (r, c0) itself past the wave's last one
  auto next = [&](int64_t r, int64_t c0, int64_t& rn, int64_t& cn) __attribute__((always_inline)) {
    rn = r;
    cn = c0 + slab;
    if (cn >= K) {
      cn = 0;
      rn = r + kH16Waves;
    }
    return rn < r1;
  };
  int64_t r = r0 + __builtin_amdgcn_readfirstlane(t / kWave), c0 = 0;
  Vec8<BF16In> va[CH], vb[CH];
  if (r < r1) load_wave_slab<BF16In, kFast, CH, kStream>(A + r * lda, c0, K, va);
  while (r < r1) {
    int64_t rb, cb;
    const bool more = next(r, c0, rb, cb);
    load_wave_slab<BF16In, kFast, CH, kStream>(A + (more ? rb : r) * lda, more ? cb : c0, K, vb);
    hist(c0, va);
    if (!more) break;
    int64_t ra, ca;
    const bool more2 = next(rb, cb, ra, ca);
    load_wave_slab<BF16In, kFast, CH, kStream>(A + (more2 ? ra : rb) * lda, more2 ? ca : cb, K, va);
    hist(cb, vb);
    r = ra;
    c0 = ca;
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
//
// A row streams through in slabs (for_row_slabs): slabs of 8 chunks of 8
// elements per lane while they fit, then one slab each of 4, 2 and 1 chunks
// where it fits, then one 1-chunk slab over the ragged end. Only that last
// slab reaches past K, so only its loads need bounds, and all loads of a slab
// are issued before the first is used.
//
// In the whole-layer forward the count also takes each row's amax clamped to
// tau, and the compaction encodes every slab it compacts with the scale that
// follows from that amax: A is read once by each kernel and its quantization
// needs no pass of its own, for any K, dtype and row alignment. The
// micro-scaled format needs no row amax (a block lies inside one chunk sweep).
// ---------------------------------------------------------------------------
constexpr int64_t kMaxRowGroups = 2048;

__host__ inline int64_t rows_per_wave(int64_t M) {
  return (M + kRowWaves * kMaxRowGroups - 1) / (kRowWaves * kMaxRowGroups);
}

__host__ inline int64_t row_groups(int64_t M) {
  const int64_t R = kRowWaves * rows_per_wave(M);
  return (M + R - 1) / R;
}

template <int N>
struct Ch {
  static constexpr int value = N;
};
template <bool B>
using Full = std::integral_constant<bool, B>;

// f(Ch<CH>, Full<inside>, c0) for each slab of a row of K elements.
template <class F>
__device__ __attribute__((always_inline)) inline void for_row_slabs(int64_t K, F&& f) {
  constexpr int64_t S = int64_t(kWave) * 8;  // columns of one chunk sweep
  int64_t c0 = 0;
  for (; c0 + 8 * S <= K; c0 += 8 * S) f(Ch<8>{}, Full<true>{}, c0);
  if (c0 + 4 * S <= K) {
    f(Ch<4>{}, Full<true>{}, c0);
    c0 += 4 * S;
  }
  if (c0 + 2 * S <= K) {
    f(Ch<2>{}, Full<true>{}, c0);
    c0 += 2 * S;
  }
  if (c0 + S <= K) {
    f(Ch<1>{}, Full<true>{}, c0);
    c0 += S;
  }
  if (c0 < K) f(Ch<1>{}, Full<false>{}, c0);
}

// A chunk of 8 consecutive elements as loaded: bfloat16 as its raw 16-byte
// word (element i is the low half of 32-bit word i / 2 for even i, the high
// half for odd i), float32 as 8 floats.
template <class In>
struct RowChunk;
template <>
struct RowChunk<BF16In> {
  using T = uint4;
};
template <>
struct RowChunk<F32In> {
  using T = Vec8<F32In>;
};

// Chunk c (elements c .. c+7) of a row of K elements, zero past K. kFast: the
// row is 16-byte aligned and K % 8 == 0 (vector loads; a chunk is wholly inside
// the row or wholly past it). kFull: the chunk lies inside the row.
template <bool kFast, bool kFull, bool kStream>
__device__ inline void load_row_chunk(const uint16_t* __restrict__ row, int64_t c, int64_t K,
                                      uint4& w) {
  if constexpr (kFast) {
    if constexpr (kFull) {
      w = load16<kStream>(row + c);
    } else {
      w = load16<kStream>(row + (c < K ? c : K - 8));
      if (c >= K) w = make_uint4(0, 0, 0, 0);
    }
  } else {
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (kFull || c + i < K) ? uint32_t(row[c + i]) : 0u;
    w = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                   h[6] | (h[7] << 16));
  }
}

template <bool kFast, bool kFull, bool kStream>
__device__ inline void load_row_chunk(const float* __restrict__ row, int64_t c, int64_t K,
                                      Vec8<F32In>& v) {
  if constexpr (kFull)
    load8<F32In, kFast, kStream>(row + c, 8, v);
  else
    load_chunk<F32In, kFast, kStream>(row, c, K, v);
}

// Chunk j of lane l starts at column c0 + (64j + l) * 8.
template <class In, bool kFast, bool kFull, int CH, bool kStream>
__device__ inline void load_row_slab(const typename In::T* __restrict__ row, int64_t c0,
                                     int64_t K, typename RowChunk<In>::T (&v)[CH]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int j = 0; j < CH; ++j)
    load_row_chunk<kFast, kFull, kStream>(row, c0 + (int64_t(j) * kWave + lane) * 8, K, v[j]);
}

// Count of the entries of a chunk with |a| > tau (chunks past K are zero, and
// a zero key never exceeds tau's) added to n, and with kMax the running
// maximum of the magnitude keys folded into m. bfloat16, two keys per 32-bit
// word: adding bias = 0x7fff - tkey to each 15-bit key sets bit 15 of its half
// exactly when key > tkey (no carry crosses the halves), so one population
// count covers both; m holds two 16-bit maxima (one packed integer max per
// word).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <bool kMax>
__device__ inline void count_fold(const uint4& w, uint32_t bias2, uint32_t& n, uint32_t& m) {
  const uint32_t q[4] = {w.x, w.y, w.z, w.w};
  u16x2 m2 = __builtin_bit_cast(u16x2, m);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t k2 = q[i] & 0x7fff7fffu;
    n += uint32_t(__popc((k2 + bias2) & 0x80008000u));
    if constexpr (kMax) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, k2));
  }
  m = __builtin_bit_cast(uint32_t, m2);
}

// float32: adding bias = 0x7fffffff - tkey to a 31-bit key sets bit 31 exactly
// when key > tkey.
template <bool kMax>
__device__ inline void count_fold(const Vec8<F32In>& v, uint32_t bias, uint32_t& n,
                                  uint32_t& m) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t k = F32In::key(v.v[i]);
    n += (k + bias) >> 31;
    if constexpr (kMax) m = m > k ? m : k;
  }
}

// The bias of count_fold for tau's key (bfloat16: in both halves).
template <class In>
__device__ inline uint32_t count_bias(uint32_t tkey) {
  if constexpr (In::kBytes == 2)
    return (0x7fffu - tkey) * 0x00010001u;
  else
    return 0x7fffffffu - tkey;
}

// The row's largest key, from every lane's running maximum.
template <class In>
__device__ inline uint32_t row_key_max(uint32_t m) {
  if constexpr (In::kBytes == 2) {
    const uint32_t lo = m & 0xffffu, hi = m >> 16;
    m = lo > hi ? lo : hi;
  }
  return wave_max_u32(m);
}

// Value of element i (0 .. 7, not a compile-time constant) of a chunk, taken
// from the chunk's 64-bit halves with shifts and selects of whole values, so
// that the chunk is never indexed through memory.
__device__ inline float chunk_value(const uint4& w, int i) {
  const uint64_t lo = (uint64_t(w.y) << 32) | w.x, hi = (uint64_t(w.w) << 32) | w.z;
  const uint64_t d = (i & 4) ? hi : lo;
  return __uint_as_float(uint32_t(d >> (16 * (i & 3))) << 16);
}

__device__ inline float chunk_value(const Vec8<F32In>& v, int i) {
  uint64_t q[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    q[u] = (uint64_t(__float_as_uint(v.v[2 * u + 1])) << 32) | __float_as_uint(v.v[2 * u]);
  const uint64_t d = (i & 4) ? ((i & 2) ? q[3] : q[2]) : ((i & 2) ? q[1] : q[0]);
  return __uint_as_float(uint32_t(d >> (32 * (i & 1))));
}

// Element mask of a chunk: bit i set when element i's magnitude key exceeds
// tau's. bfloat16: as in count_fold, adding bias = 0x7fff - tkey to both
// 15-bit keys of a word sets bit 15 of a half exactly when its key exceeds
// tkey; the flags of word i (elements 2i and 2i+1, bits 15 and 31) are moved
// to bits 2i and 2i+16, and the upper ones then down to 2i+1.
__device__ inline uint32_t chunk_mask(const uint4& w, uint32_t, uint32_t bias2) {
  const uint32_t q[4] = {w.x, w.y, w.z, w.w};
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) x |= (((q[i] & 0x7fff7fffu) + bias2) & 0x80008000u) >> (15 - 2 * i);
  return (x | (x >> 15)) & 0xffu;
}

__device__ inline uint32_t chunk_mask(const Vec8<F32In>& v, uint32_t tkey, uint32_t) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m |= uint32_t(F32In::key(v.v[i]) > tkey) << i;
  return m;
}

// Write every |a| > tau entry of a slab, ascending column, from position pos.
// The entries of chunk (j, lane) follow those of all chunks (j', *) with
// j' < j and (j, lane') with lane' < lane. A lane's count n of entries in its
// chunk is at most 8; the entries of the lower lanes number the sum over
// t >= 1 of how many lower lanes have n >= t, one wave ballot and mbcnt per t,
// stopping at the first t no lane reaches (entries are sparse: usually after
// t = 2, and at once for a chunk sweep without any). No LDS, no barrier.
template <class C, int CH>
__device__ inline void compact_slab(const C (&v)[CH], int64_t c0, int64_t r, uint32_t tkey,
                                    uint32_t bias, float tau, uint32_t& pos, uint32_t cap,
                                    int32_t* __restrict__ out_row, int32_t* __restrict__ out_col,
                                    float* __restrict__ out_val) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    uint32_t mine = chunk_mask(v[j], tkey, bias);
    const uint32_t n = uint32_t(__popc(mine));
    uint64_t b = __ballot(n != 0u);
    if (b == 0) continue;  // wave-uniform: no entry in this chunk sweep
    uint32_t lower = __builtin_amdgcn_mbcnt_hi(uint32_t(b >> 32),
                                               __builtin_amdgcn_mbcnt_lo(uint32_t(b), 0u));
    uint32_t total = uint32_t(__popcll(b));
    for (uint32_t t = 2; t <= 8; ++t) {
      b = __ballot(n >= t);
      if (b == 0) break;
      lower = __builtin_amdgcn_mbcnt_hi(uint32_t(b >> 32),
                                        __builtin_amdgcn_mbcnt_lo(uint32_t(b), lower));
      total += uint32_t(__popcll(b));
    }
    // One store per array for each set bit of the lane, lowest first: a lane
    // rarely holds more than one entry of a chunk, so the wave usually
    // stores once instead of once per element position.
    uint32_t p = pos + lower;  // positions below capacity < 2^31, columns below K < 2^31
    const int c = int(c0) + (j * kWave + lane) * 8;
    while (mine) {
      const int i = __builtin_ctz(mine);
      mine &= mine - 1u;
      // p < cap always holds when tau is the true order statistic
      // (nnz <= n-1-k); the test only keeps a wrong tau from writing out of bounds.
      if (p < cap) {
        const float a = chunk_value(v[j], i);
        out_row[p] = int32_t(r);
        out_col[p] = c + i;
        out_val[p] = __fsub_rn(a, copysignf(tau, a));
      }
      ++p;
    }
    pos += total;
  }
}

// Token-wise codes of a chunk clamped to tau, 8 per 32-bit word (low nibble
// first). bfloat16 with quick (4 * inv finite): two codes per word of the
// chunk from y4 = RN32(|x| * 4inv) (bf16_chunk_code); otherwise, and for
// float32, the generic encoder.
__device__ inline uint32_t encode_chunk(const uint4& w, float tau, float inv, float inv4,
                                        float cap4, bool quick) {
  if (quick) return bf16_chunk_code(w, inv4, cap4);
  return bf16_pair_code_slow(w.x, tau, inv) | (bf16_pair_code_slow(w.y, tau, inv) << 8) |
         (bf16_pair_code_slow(w.z, tau, inv) << 16) | (bf16_pair_code_slow(w.w, tau, inv) << 24);
}

__device__ inline uint32_t encode_chunk(const Vec8<F32In>& v, float tau, float inv, float,
                                        float, bool) {
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    word |= (e2m1_magnitude(fminf(fabsf(v.v[i]), tau), inv) | (F32In::sign_bit(v.v[i]) << 3))
            << (4 * i);
  return word;
}

// Micro-scaled codes of a chunk clamped to tau and the exponent of its block
// (four consecutive lanes; every lane of the wave takes part in the exchange).
__device__ inline uint32_t encode_chunk_mx(const uint4& w, float tau, int& e) {
  const uint32_t q[4] = {w.x, w.y, w.z, w.w};
  float ax[8];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ax[2 * i] = fminf(fabsf(__uint_as_float(q[i] << 16)), tau);
    ax[2 * i + 1] = fminf(fabsf(__uint_as_float(q[i] & 0xffff0000u)), tau);
    m = fmaxf(m, fmaxf(ax[2 * i], ax[2 * i + 1]));
  }
  e = mx_exponent(quad_max(m));
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    word |= (mx_magnitude(ax[2 * i], e) | ((q[i] >> 12) & 0x8u)) << (8 * i);
    word |= (mx_magnitude(ax[2 * i + 1], e) | ((q[i] >> 28) & 0x8u)) << (8 * i + 4);
  }
  return word;
}

__device__ inline uint32_t encode_chunk_mx(const Vec8<F32In>& v, float tau, int& e) {
  float ax[8];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ax[i] = fminf(fabsf(v.v[i]), tau);
    m = fmaxf(m, ax[i]);
  }
  e = mx_exponent(quad_max(m));
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    word |= (mx_magnitude(ax[i], e) | (F32In::sign_bit(v.v[i]) << 3)) << (4 * i);
  return word;
}

// Per-row count of |a| > tau into cnt[r], and the workgroup's total into
// gsum[blockIdx.x]. kPick (bfloat16): tau's key comes from the fine histogram
// and workgroup 0 records it in st and tau; otherwise it is read from st.
// (Looking the key up between the first row's loads and their use measured
// slower: it costs registers.) kAmax: also the row's amax clamped to tau into
// amax[r].
template <class In, bool kFast, bool kPick, bool kAmax, bool kStream>
__device__ __attribute__((always_inline)) inline void count_rows_body(
    int64_t bid, const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda,
    int64_t rpw, SelState* st, const uint32_t* __restrict__ fine, float* __restrict__ tau,
    uint32_t* __restrict__ cnt, uint32_t* __restrict__ gsum, float* __restrict__ amax) {
  using C = typename RowChunk<In>::T;
  __shared__ uint32_t wsum[kRowWaves];
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);  // wave-uniform
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t R = int64_t(kRowWaves) * rpw;
  const int64_t r0 = bid * R;
  const int64_t r1 = (r0 + R < M) ? r0 + R : M;
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
  const uint32_t bias = count_bias<In>(tkey);
  uint32_t total = 0;
  for (int64_t r = r0 + w; r < r1; r += kRowWaves) {
    const typename In::T* row = A + r * lda;
    uint32_t c = 0, mk = 0;
    for_row_slabs(K, [&](auto ch, auto full, int64_t c0) __attribute__((always_inline)) {
      constexpr int CH = decltype(ch)::value;
      C v[CH];
      load_row_slab<In, kFast, decltype(full)::value, CH, kStream>(row, c0, K, v);
#pragma unroll
      for (int j = 0; j < CH; ++j) count_fold<kAmax>(v[j], bias, c, mk);
    });
    c = wave_sum_u32(c);
    total += c;
    if (lane == 0) cnt[r] = c;
    if constexpr (kAmax) {
      const uint32_t k = row_key_max<In>(mk);
      if (lane == 0) amax[r] = In::key_to_float(k < tkey ? k : tkey);
    }
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

template <class In, bool kFast, bool kPick, bool kStream>
__global__ __launch_bounds__(kRowWaves * kWave) void count_rows_kernel(
    const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda, int64_t rpw,
    SelState* st, const uint32_t* __restrict__ fine, float* __restrict__ tau,
    uint32_t* __restrict__ cnt, uint32_t* __restrict__ gsum) {
  count_rows_body<In, kFast, kPick, false, kStream>(blockIdx.x, A, M, K, lda, rpw, st, fine, tau, cnt,
                                           gsum, nullptr);
}

// What the compaction also does with the slabs it holds.
constexpr int kQuantNone = 0;   // nothing (the select alone)
constexpr int kQuantToken = 1;  // token-wise codes; sX[r] holds the row's clamped amax on entry
                                // and its scale on exit
constexpr int kQuantMx = 2;     // micro-scaled codes and block scales (Xs, step-major)

// Row-major COO and row_ptr. The workgroup's first position is the sum of the
// totals of the workgroups before it; within a batch of kRowWaves rows a wave
// adds the counts of the lower rows of the batch, so waves need no barrier
// after the first. With kQuant, the codes of the row's padded length ldq * 2
// (zero past K) go to Xq + r * ldq.
template <class In, bool kFast, int kQuant, bool kStream>
__device__ __attribute__((always_inline)) inline void compact_rows_body(
    int64_t bid, const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda,
    int64_t rpw, const SelState* __restrict__ st, const float* __restrict__ tau_p,
    const uint32_t* __restrict__ cnt, const uint32_t* __restrict__ gsum, int64_t capacity,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ out_row, int32_t* __restrict__ out_col,
    float* __restrict__ out_val, uint8_t* __restrict__ Xq, int64_t ldq, float* __restrict__ sX,
    uint8_t* __restrict__ Xs) {
  using C = typename RowChunk<In>::T;
  __shared__ uint32_t wsum[kRowWaves];
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);  // wave-uniform
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t R = int64_t(kRowWaves) * rpw;
  const int64_t r0 = bid * R;
  const int64_t r1 = (r0 + R < M) ? r0 + R : M;
  const uint32_t tkey = st->tau_key;
  const uint32_t bias = count_bias<In>(tkey);
  const float tau = *tau_p;
  const uint32_t cap = uint32_t(capacity < INT32_MAX ? capacity : INT32_MAX);
  const int64_t Kp = ldq * 2;
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
      const typename In::T* row = A + r * lda;
      uint8_t* qrow = Xq + r * ldq;
      float inv = 0.0f, inv4 = 0.0f, cap4 = 0.0f;
      if constexpr (kQuant == kQuantToken) {
        float s;
        vector_scale(sX[r], s, inv);
        inv4 = __fmul_rn(inv, 4.0f);
        cap4 = code_cap4(tau, inv4);
        if (lane == 0) sX[r] = s;
      }
      const bool quick = inv4 < __builtin_huge_valf();
      uint32_t pos = base + before;
      for_row_slabs(K, [&](auto ch, auto full, int64_t c0) __attribute__((always_inline)) {
        constexpr int CH = decltype(ch)::value;
        constexpr bool kFull = decltype(full)::value;
        C v[CH];
        load_row_slab<In, kFast, kFull, CH, kStream>(row, c0, K, v);
        compact_slab<C, CH>(v, c0, r, tkey, bias, tau, pos, cap, out_row, out_col, out_val);
        if constexpr (kQuant != kQuantNone) {
#pragma unroll
          for (int j = 0; j < CH; ++j) {
            // chunks in [K, Kp) are zero and encode to the zero padding
            const int64_t c = c0 + (int64_t(j) * kWave + lane) * 8;
            if constexpr (kQuant == kQuantToken) {
              const uint32_t word = encode_chunk(v[j], tau, inv, inv4, cap4, quick);
              if (kFull || c < Kp) *reinterpret_cast<uint32_t*>(qrow + c / 2) = word;
            } else {
              int e;
              const uint32_t word = encode_chunk_mx(v[j], tau, e);
              if (kFull || c < Kp) {
                *reinterpret_cast<uint32_t*>(qrow + c / 2) = word;
                const int64_t b = c / 32;  // block of this chunk
                if ((lane & 3) == 0) Xs[(b / 4) * 4 * M + 4 * r + (b & 3)] = uint8_t(e + 127);
              }
            }
          }
        }
      });
      if (lane == 0) row_ptr[r + 1] = int32_t(base + before + own);
    }
    base += all;
  }
}

template <class In, bool kFast, bool kStream>
__global__ __launch_bounds__(kRowWaves * kWave) void compact_rows_kernel(
    const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda, int64_t rpw,
    const SelState* __restrict__ st, const float* __restrict__ tau_p,
    const uint32_t* __restrict__ cnt, const uint32_t* __restrict__ gsum, int64_t capacity,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ out_row, int32_t* __restrict__ out_col,
    float* __restrict__ out_val) {
  compact_rows_body<In, kFast, kQuantNone, kStream>(blockIdx.x, A, M, K, lda, rpw, st, tau_p, cnt, gsum,
                                           capacity, row_ptr, out_row, out_col, out_val, nullptr,
                                           0, nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// Whole-layer forward: the quantization of W has no dependence on the select,
// so its passes share launches with the select's row kernels: the column
// maxima (micro-scaled: W's only pass) with the row count, the codes with the
// compaction. The cleared column maxima come from the first histogram pass.
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

// W's side of a pair launch: nb workgroups over a gx-wide grid of tiles.
struct WPass {
  const void* W;
  int64_t K, N, ldw;
  uint32_t* colmax;  // token-wise column maxima (cleared by the first histogram pass)
  uint8_t* Wq;
  int64_t ldq;
  void* sW;  // token-wise: float scales; micro-scaled: step-major E8M0 bytes
  int64_t gx, nb;
};

template <class In, bool kFast, bool kWAligned, bool kMx, bool kStream>
__global__ __launch_bounds__(kRowWaves * kWave) void count_wpass_kernel(
    const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda, int64_t rpw,
    SelState* st, const uint32_t* __restrict__ fine, float* __restrict__ tau,
    uint32_t* __restrict__ cnt, uint32_t* __restrict__ gsum, float* __restrict__ amax, int64_t na,
    WPass wp) {
  using T = typename In::T;
  int64_t i;
  if (pair_first(blockIdx.x, na, wp.nb, i))
    count_rows_body<In, kFast, In::kBytes == 2, !kMx, kStream>(i, A, M, K, lda, rpw, st, fine, tau, cnt,
                                                      gsum, amax);
  else if constexpr (kMx)
    quantize_cols_mx_body<In, kWAligned>(i % wp.gx, i / wp.gx, static_cast<const T*>(wp.W), wp.K,
                                         wp.N, wp.ldw, wp.Wq, wp.ldq,
                                         static_cast<uint8_t*>(wp.sW));
  else
    colmax_body<In, kWAligned>(i % wp.gx, i / wp.gx, static_cast<const T*>(wp.W), wp.K, wp.N,
                               wp.ldw, wp.colmax);
}

template <class In, bool kFast, bool kWAligned, bool kMx, bool kStream>
__global__ __launch_bounds__(kRowWaves * kWave) void compact_wpass_kernel(
    const typename In::T* __restrict__ A, int64_t M, int64_t K, int64_t lda, int64_t rpw,
    const SelState* __restrict__ st, const float* __restrict__ tau_p,
    const uint32_t* __restrict__ cnt, const uint32_t* __restrict__ gsum, int64_t capacity,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ out_row, int32_t* __restrict__ out_col,
    float* __restrict__ out_val, uint8_t* __restrict__ Xq, int64_t ldq, float* __restrict__ sX,
    uint8_t* __restrict__ Xs, int64_t na, WPass wp) {
  using T = typename In::T;
  int64_t i;
  if (pair_first(blockIdx.x, na, wp.nb, i))
    compact_rows_body<In, kFast, kMx ? kQuantMx : kQuantToken, kStream>(
        i, A, M, K, lda, rpw, st, tau_p, cnt, gsum, capacity, row_ptr, out_row, out_col, out_val,
        Xq, ldq, sX, Xs);
  else if constexpr (!kMx)
    quantize_cols_body<In, kWAligned>(i % wp.gx, i / wp.gx, static_cast<const T*>(wp.W), wp.K,
                                      wp.N, wp.ldw, wp.colmax, wp.Wq, wp.ldq,
                                      static_cast<float*>(wp.sW));
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

// float32 set-up: clears the histograms (and nclear words at clear) and sets
// the state to rank k of all keys.
__global__ void select_init_kernel(SelState* st, uint32_t* hist, int64_t nwords, int64_t k,
                                   uint32_t* clear, int64_t nclear) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < nwords;
       i += int64_t(gridDim.x) * blockDim.x)
    hist[i] = 0u;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < nclear;
       i += int64_t(gridDim.x) * blockDim.x)
    clear[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    st->prefix = 0u;
    st->tau_key = 0u;
    st->krem = k;
  }
}

// The select's workspace: state, then the histogram words (hist_words), the
// row-group totals and the row counts.
template <class In>
struct SelWork {
  SelState* st;
  uint32_t *hist, *gsum, *cnt;
  explicit SelWork(void* ws) {
    st = static_cast<SelState*>(ws);
    hist = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + 256);
    gsum = hist + hist_words<In>();
    cnt = gsum + kMaxRowGroups;
  }
};

// The bfloat16 histogram words: the coarse partial rows, the fine histogram,
// the saved windows.
struct H16Work {
  SelState* st;
  uint32_t *part, *fine, *win, *fwin;
  explicit H16Work(const SelWork<BF16In>& s) {
    st = s.st;
    part = s.hist;
    fine = part + size_t(kMaxH16Groups) * kCoarseBins;
    win = fine + kFineBins;
    fwin = win + kMaxH16Groups;
  }
};

// The two bfloat16 histogram passes (the coarse one also clears nclear words
// at clear).
template <bool kFast, bool kStream>
hipError_t launch_hist16(const uint16_t* A, int64_t M, int64_t K, int64_t lda, int64_t k,
                         const H16Work& w, uint32_t* clear, int64_t nclear, hipStream_t stream) {
  // one workgroup per CU (MI355X: 256), at least one row per wave
  int64_t wgs = (M + kH16Waves - 1) / kH16Waves;
  wgs = wgs < kMaxH16Groups ? wgs : kMaxH16Groups;
  const int64_t per = (M + wgs - 1) / wgs;
  const dim3 g(static_cast<unsigned>(wgs));
  // k < M*K < 2^32
  const uint32_t k32 = uint32_t(k);
  // two slabs are held in registers at once: at most 8 chunks per lane (4
  // with element loads)
  auto run = [&](auto ch) {
    constexpr int CH = decltype(ch)::value;
    select_hist16_kernel<kFast, false, CH, kStream><<<g, kH16Threads, 0, stream>>>(
        A, M, K, lda, per, w.part, 0, k32, w.st, w.fine, w.win, w.fwin, clear, nclear);
    select_hist16_kernel<kFast, true, CH, kStream><<<g, kH16Threads, 0, stream>>>(
        A, M, K, lda, per, w.part, int(wgs), k32, w.st, w.fine, w.win, w.fwin, nullptr, 0);
    return hipSuccess;
  };
  switch (chunks_per_lane(K, kFast ? 8 : 4)) {
    case 1:
      return run(std::integral_constant<int, 1>{});
    case 2:
      return run(std::integral_constant<int, 2>{});
    case 4:
      return run(std::integral_constant<int, 4>{});
    default:
      if constexpr (kFast) return run(std::integral_constant<int, 8>{});
      return hipErrorInvalidValue;
  }
}

// The three float32 digit passes (the set-up also clears nclear words at
// clear); the last pick writes tau and its key.
template <bool kFast>
void launch_hist32(const float* A, int64_t M, int64_t K, int64_t lda, int64_t k,
                   const SelWork<F32In>& w, float* tau, uint32_t* clear, int64_t nclear,
                   hipStream_t stream) {
  select_init_kernel<<<1, 256, 0, stream>>>(w.st, w.hist, int64_t(hist_words<F32In>()), k, clear,
                                            nclear);
  // Enough workgroups to fill the chip, each with several slabs so that the
  // per-group histogram merge stays small.
  const int64_t slab = int64_t(kHistThreads) * kHistCh * 8;
  const int64_t slabs = M * ((K + slab - 1) / slab);
  const int64_t g = slabs < 1024 ? slabs : 1024;
  for (int p = 0; p < F32Digits::kPasses; ++p) {
    const int shift = F32Digits::shift(p);
    const int width = F32Digits::width(p);
    const int hi = shift + width;
    select_hist_kernel<F32In, kFast><<<dim3(unsigned(g)), kHistThreads, 0, stream>>>(
        A, M, K, lda, w.st, shift, width, hi >= F32Digits::kKeyBits ? 32 : hi,
        w.hist + size_t(p) * kHistBins);
    select_pick_kernel<<<1, 256, 0, stream>>>(w.st, w.hist + size_t(p) * kHistBins, width,
                                               p == F32Digits::kPasses - 1 ? 1 : 0, 0, tau);
  }
}

template <class In, bool kFast, bool kStream>
hipError_t run_select(const void* Ap, int64_t M, int64_t K, int64_t lda, int64_t k, float* tau,
                      int64_t capacity, int32_t* row, int32_t* col, float* val,
                      int32_t* row_ptr, void* ws, hipStream_t stream) {
  using T = typename In::T;
  const T* A = static_cast<const T*>(Ap);
  const SelWork<In> w(ws);
  const uint32_t* fine = nullptr;
  if constexpr (In::kBytes == 2) {
    const H16Work h(w);
    const hipError_t e = launch_hist16<kFast, kStream>(A, M, K, lda, k, h, nullptr, 0, stream);
    if (e != hipSuccess) return e;
    fine = h.fine;
  } else {
    launch_hist32<kFast>(A, M, K, lda, k, w, tau, nullptr, 0, stream);
  }
  const int64_t rpw = rows_per_wave(M);
  const dim3 g(static_cast<unsigned>(row_groups(M)));
  count_rows_kernel<In, kFast, In::kBytes == 2, kStream><<<g, kRowWaves * kWave, 0, stream>>>(
      A, M, K, lda, rpw, w.st, fine, tau, w.cnt, w.gsum);
  compact_rows_kernel<In, kFast, kStream><<<g, kRowWaves * kWave, 0, stream>>>(
      A, M, K, lda, rpw, w.st, tau, w.cnt, w.gsum, capacity, row_ptr, row, col, val);
  return hipGetLastError();
}

bool rows_fast(const void* A, int esz, int64_t K, int64_t lda) {
  return (reinterpret_cast<uintptr_t>(A) % 16 == 0) && ((lda * esz) % 16 == 0) && (K % 8 == 0);
}

// Histograms, then the row count with W's first pass, then the compaction
// (with the quantization of A) with W's codes.
template <class In, bool kFast, bool kWAligned, bool kMx, bool kStream>
hipError_t forward_front(const FrontArgs& f, hipStream_t stream) {
  using T = typename In::T;
  const T* A = static_cast<const T*>(f.A);
  const SelWork<In> w(f.ws);
  uint32_t* clear = kMx ? nullptr : f.colmax;
  const int64_t nclear = kMx ? 0 : f.N;
  const uint32_t* fine = nullptr;
  if constexpr (In::kBytes == 2) {
    const H16Work h(w);
    const hipError_t e =
        launch_hist16<kFast, kStream>(A, f.M, f.K, f.lda, f.k, h, clear, nclear, stream);
    if (e != hipSuccess) return e;
    fine = h.fine;
  } else {
    launch_hist32<kFast>(A, f.M, f.K, f.lda, f.k, w, f.tau, clear, nclear, stream);
  }
  const int64_t rpw = rows_per_wave(f.M);
  const int64_t na = row_groups(f.M);
  const int64_t Kp = f.ldq * 2;
  WPass wp{f.W, f.K, f.N, f.ldw, f.colmax, f.Wq, f.ldq, f.sW, 0, 0};
  // pass 1: column maxima on 512-column strips x 64-row splits, or the
  // micro-scaled codes on 128 x 128 tiles
  if constexpr (kMx) {
    wp.gx = (f.N + kMxTN - 1) / kMxTN;
    wp.nb = wp.gx * (Kp / kMxTK);
  } else {
    wp.gx = (f.N + kColStrip - 1) / kColStrip;
    wp.nb = wp.gx * ((f.K + kColRows - 1) / kColRows);
  }
  count_wpass_kernel<In, kFast, kWAligned, kMx, kStream>
      <<<dim3(unsigned(na + wp.nb)), kRowWaves * kWave, 0, stream>>>(
          A, f.M, f.K, f.lda, rpw, w.st, fine, f.tau, w.cnt, w.gsum, static_cast<float*>(f.sA),
          na, wp);
  // pass 2: the token-wise codes on 128 x 128 tiles (micro-scaled: none)
  if constexpr (kMx) {
    wp.gx = 0;
    wp.nb = 0;
  } else {
    wp.gx = (f.N + kTN - 1) / kTN;
    wp.nb = wp.gx * (Kp / kTK);
  }
  compact_wpass_kernel<In, kFast, kWAligned, kMx, kStream>
      <<<dim3(unsigned(na + wp.nb)), kRowWaves * kWave, 0, stream>>>(
          A, f.M, f.K, f.lda, rpw, w.st, f.tau, w.cnt, w.gsum, f.capacity, f.row_ptr, f.row,
          f.col, f.val, f.Aq, f.ldq, kMx ? nullptr : static_cast<float*>(f.sA),
          kMx ? static_cast<uint8_t*>(f.sA) : nullptr, na, wp);
  return hipGetLastError();
}

// The row kernels and the bfloat16 histogram passes read A with the
// non-temporal hint when the operands of the passes (A, and W in the forward)
// exceed kStreamBytes: the last-level cache then cannot keep them from one
// pass to the next, and streaming A through without allocating keeps more of
// W (read twice, then gathered by the compensation) resident. Below it, A
// stays cached for the passes after the first.

template <class In, bool kMx>
hipError_t forward_front_dispatch(const FrontArgs& f, hipStream_t stream) {
  const bool fast = rows_fast(f.A, In::kBytes, f.K, f.lda);
  const bool w_aligned = (reinterpret_cast<uintptr_t>(f.W) % 16 == 0) &&
                         ((f.ldw * In::kBytes) % 16 == 0);
  const bool streamed = (f.M * f.K + f.K * f.N) * In::kBytes > kStreamBytes;
  auto run = [&](auto fast_c, auto waligned_c) {
    constexpr bool kF = decltype(fast_c)::value, kW = decltype(waligned_c)::value;
    return streamed ? forward_front<In, kF, kW, kMx, true>(f, stream)
                    : forward_front<In, kF, kW, kMx, false>(f, stream);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (fast) return w_aligned ? run(T_{}, T_{}) : run(T_{}, F_{});
  return w_aligned ? run(F_{}, T_{}) : run(F_{}, F_{});
}

template <class In>
hipError_t select_dispatch(const void* A, int64_t M, int64_t K, int64_t lda, int64_t k,
                           float* tau, int64_t capacity, int32_t* row, int32_t* col, float* val,
                           int32_t* row_ptr, void* ws, hipStream_t stream) {
  const bool fast = rows_fast(A, In::kBytes, K, lda);
  const bool streamed = M * K * In::kBytes > kStreamBytes;
  if (fast)
    return streamed ? run_select<In, true, true>(A, M, K, lda, k, tau, capacity, row, col, val,
                                                 row_ptr, ws, stream)
                    : run_select<In, true, false>(A, M, K, lda, k, tau, capacity, row, col, val,
                                                  row_ptr, ws, stream);
  return streamed ? run_select<In, false, true>(A, M, K, lda, k, tau, capacity, row, col, val,
                                                row_ptr, ws, stream)
                  : run_select<In, false, false>(A, M, K, lda, k, tau, capacity, row, col, val,
                                                 row_ptr, ws, stream);
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
                                 hipStream_t stream) {
  return bf16 ? select_dispatch<BF16In>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr,
                                        ws, stream)
              : select_dispatch<F32In>(A, M, K, lda, k, tau, capacity, row, col, val, row_ptr, ws,
                                       stream);
}

hipError_t launch_forward_front(const FrontArgs& f, hipStream_t stream) {
  if (f.bf16)
    return f.mx ? forward_front_dispatch<BF16In, true>(f, stream)
                : forward_front_dispatch<BF16In, false>(f, stream);
  return f.mx ? forward_front_dispatch<F32In, true>(f, stream)
              : forward_front_dispatch<F32In, false>(f, stream);
}

}  // namespace fp4lin
