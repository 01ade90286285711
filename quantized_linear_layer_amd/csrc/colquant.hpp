// Channel-wise (per column) quantization of a K x N row-major matrix into
// E2M1 codes packed N-major, as device bodies of 256-thread workgroups that
// take their workgroup coordinates as arguments: the column-max pass and the
// encode pass of the token-wise format, and the one pass of the micro-scaled
// format (blocks of 32 codes along K). The quantize_weight kernels launch
// them directly; the forward pairs them with the select's row kernels in
// shared launches.
#pragma once

#include "device_common.hpp"

namespace fp4lin {

constexpr int kColStrip = 512;    // columns per workgroup (8 per lane)
constexpr int kColRows = 64;      // rows per workgroup split
constexpr int kColUnroll = 8;     // loads in flight per thread

// Pass 1, workgroup (bx, by): columns bx*512 .. +511, rows by*64 .. +63.
template <class In, bool kAligned>
__device__ __attribute__((always_inline)) inline void colmax_body(int64_t bx, int64_t by, const typename In::T* __restrict__ W,
                                   int64_t K, int64_t N, int64_t ldw,
                                   uint32_t* __restrict__ colmax) {
  __shared__ uint32_t red[4][kColStrip];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t c = bx * kColStrip + lane * 8;
  const int64_t k0 = by * kColRows;
  const int64_t k1 = (k0 + kColRows < K) ? k0 + kColRows : K;
  const int64_t valid = N - c;
  float m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = 0.0f;
  if (valid > 0) {
    // kColUnroll rows in flight per thread; rows past k1 read as zero
    for (int64_t kb = k0 + wave; kb < k1; kb += 4 * kColUnroll) {
      Vec8<In> v[kColUnroll];
#pragma unroll
      for (int u = 0; u < kColUnroll; ++u) {
        const int64_t k = kb + 4 * u;
        if (k < k1) {
          load8<In, kAligned>(W + k * ldw + c, valid, v[u]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[u].v[i] = typename In::T(0);
        }
      }
#pragma unroll
      for (int u = 0; u < kColUnroll; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(In::widen(v[u].v[i])));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = __float_as_uint(m[i]);
  __syncthreads();
  for (int j = threadIdx.x; j < kColStrip; j += 256) {
    uint32_t x = red[0][j];
    x = x > red[1][j] ? x : red[1][j];
    x = x > red[2][j] ? x : red[2][j];
    x = x > red[3][j] ? x : red[3][j];
    const int64_t col = bx * kColStrip + j;
    if (col < N) atomicMax(&colmax[col], x);
  }
}

// Pass 2 tile: 128 codes along K x 128 columns. Thread (kg, g) = (t % 16,
// t / 16) owns rows k0 + 8kg .. +7 and columns n0 + 8g .. +7, so for each of its
// columns the 8 codes along K form one 32-bit word of that column's packed row
// (low nibble first), stored directly: a wave's store covers 64 contiguous
// bytes of each of 4 packed rows, and its loads 64 contiguous bytes of each of
// 16 rows of W.
constexpr int kTK = 128;
constexpr int kTN = 128;

template <class In, bool kAligned>
__device__ __attribute__((always_inline)) inline void quantize_cols_body(int64_t bx, int64_t by,
                                          const typename In::T* __restrict__ W, int64_t K,
                                          int64_t N, int64_t ldw,
                                          const uint32_t* __restrict__ colmax,
                                          uint8_t* __restrict__ Wq, int64_t ldq,
                                          float* __restrict__ sW) {
  __shared__ float inv_s[kTN];
  const int t = threadIdx.x;
  const int64_t n0 = bx * kTN;
  const int64_t k0 = by * kTK;
  if (t < kTN) {
    const int64_t n = n0 + t;
    float s = 0.0f, inv = 0.0f;
    if (n < N) {
      vector_scale(__uint_as_float(colmax[n]), s, inv);
      if (by == 0) sW[n] = s;
    }
    inv_s[t] = inv;
  }
  const int kg = t & 15, g = t >> 4;
  const int64_t c = n0 + g * 8;
  const int64_t valid = N - c;
  const int64_t kr = k0 + kg * 8;
  Vec8<In> v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (kr + u < K && valid > 0) {
      load8<In, kAligned>(W + (kr + u) * ldw + c, valid, v[u]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[u].v[j] = typename In::T(0);
    }
  }
  __syncthreads();
  if (valid <= 0) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= valid) break;
    const float inv = inv_s[g * 8 + j];
    uint32_t word = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // rows past K were loaded as zero and encode to the zero padding
      const uint32_t code =
          e2m1_magnitude(fabsf(In::widen(v[u].v[j])), inv) | (In::sign_bit(v[u].v[j]) << 3);
      word |= code << (4 * u);
    }
    *reinterpret_cast<uint32_t*>(Wq + (c + j) * ldq + kr / 2) = word;
  }
}

// Micro-scaled tile (bx, by): columns bx*128 .. +127, rows by*128 .. +127
// (rows past K read as zero and give the zero padding). Thread (kg, g) =
// (t % 16, t / 16) owns rows k0 + 8kg .. +7 of columns n0 + 8g .. +7: the 8
// codes of one column are one 32-bit word of its packed row, and lanes
// 4q .. 4q+3 share block q. Block scales go to the step-major array Ws (the
// byte of block b of column n at (b / 4) * 4N + 4n + b % 4).
constexpr int kMxTK = 128;  // codes along K per column tile
constexpr int kMxTN = 128;  // columns per tile

template <class In, bool kAligned>
__device__ __attribute__((always_inline)) inline void quantize_cols_mx_body(
    int64_t bx, int64_t by, const typename In::T* __restrict__ W, int64_t K, int64_t N,
    int64_t ldw, uint8_t* __restrict__ Wq, int64_t ldq, uint8_t* __restrict__ Ws) {
  const int t = threadIdx.x;
  const int kg = t & 15, g = t >> 4;
  const int64_t n0 = bx * kMxTN;
  const int64_t k0 = by * kMxTK;
  const int64_t c = n0 + g * 8;
  const int64_t valid = N - c;
  const int64_t kr = k0 + kg * 8;
  Vec8<In> v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (kr + u < K && valid > 0) {
      load8<In, kAligned>(W + (kr + u) * ldw + c, valid, v[u]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[u].v[j] = typename In::T(0);
    }
  }
  int e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float m = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) m = fmaxf(m, fabsf(In::widen(v[u].v[j])));
    e[j] = mx_exponent(quad_max(m));
  }
  if (valid <= 0) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= valid) break;
    uint32_t word = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      word |= (mx_magnitude(fabsf(In::widen(v[u].v[j])), e[j]) | (In::sign_bit(v[u].v[j]) << 3))
              << (4 * u);
    *reinterpret_cast<uint32_t*>(Wq + (c + j) * ldq + kr / 2) = word;
    // rows kr .. kr+7: block kr / 32 of K step kr / 128 (the tile's step by)
    if ((kg & 3) == 0) Ws[(kr / 128) * 4 * N + 4 * (c + j) + ((kr / 32) & 3)] = uint8_t(e[j] + 127);
  }
}

}  // namespace fp4lin
