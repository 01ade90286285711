// Vector-wise ScaleShift quantization to E2M1 (FP4 training write-up
// "微软首创FP4训练框架": the granularity paragraph — activations per row
// (token-wise), weights per column (channel-wise) — and the rounding and
// ScaleShift paragraphs — scale each vector into the FP4 range, then round to
// the nearest FP4 value).
//
// Rows:    one wave per row; pass 1 finds the (clamped) row amax, pass 2
//          re-reads the row (from cache) and writes 8 codes per lane as one
//          32-bit store; the zero padding up to roundup(K,128) is written too.
// Columns: pass 1 takes per-column maxima of the K x N row-major weight with
//          loads coalesced along N (8 columns per lane) and merges them with
//          integer atomicMax on the float bits (non-negative floats order like
//          their bits); pass 2 quantizes a 128 x 64 tile and transposes it
//          through LDS so that each output row (one column of W) is written as
//          contiguous 16-byte stores.
#include "device_common.hpp"
#include "internal.hpp"

namespace fp4lin {

namespace {

template <class In>
__device__ inline uint32_t encode8(const Vec8<In>& v, int64_t valid, float tau, float inv) {
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float ax = fminf(fabsf(In::widen(v.v[i])), tau);
    uint32_t code = e2m1_magnitude(ax, inv) | (In::sign_bit(v.v[i]) << 3);
    code = (i < valid) ? code : 0u;
    word |= code << (4 * i);
  }
  return word;
}

template <class In, bool kAligned>
__global__ __launch_bounds__(256) void quantize_rows_kernel(
    const typename In::T* __restrict__ X, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ tau_p, uint8_t* __restrict__ Xq, int64_t ldq,
    float* __restrict__ sX) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (r >= M) return;
  const float tau = tau_p ? *tau_p : __builtin_huge_valf();
  const typename In::T* row = X + r * ldx;
  float m = 0.0f;
  for (int64_t c = int64_t(lane) * 8; c < K; c += kWave * 8) {
    Vec8<In> v;
    const int64_t valid = K - c;
    load8<In, kAligned>(row + c, valid, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(In::widen(v.v[i])));
  }
  m = wave_max(m);
  const float amax = fminf(m, tau);
  float s, inv;
  vector_scale(amax, s, inv);
  if (lane == 0) sX[r] = s;
  uint8_t* qrow = Xq + r * ldq;
  const int64_t Kp = ldq * 2;
  for (int64_t c = int64_t(lane) * 8; c < Kp; c += kWave * 8) {
    const int64_t valid = K - c;
    uint32_t word = 0;
    if (valid > 0) {
      Vec8<In> v;
      load8<In, kAligned>(row + c, valid, v);
      word = encode8<In>(v, valid, tau, inv);
    }
    *reinterpret_cast<uint32_t*>(qrow + c / 2) = word;
  }
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

constexpr int kColStrip = 512;    // columns per workgroup (8 per lane)
constexpr int kColRows = 64;      // rows per workgroup split

template <class In, bool kAligned>
__global__ __launch_bounds__(256) void colmax_kernel(const typename In::T* __restrict__ W,
                                                     int64_t K, int64_t N, int64_t ldw,
                                                     uint32_t* __restrict__ colmax) {
  __shared__ uint32_t red[4][kColStrip];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t c = int64_t(blockIdx.x) * kColStrip + lane * 8;
  const int64_t k0 = int64_t(blockIdx.y) * kColRows;
  const int64_t k1 = (k0 + kColRows < K) ? k0 + kColRows : K;
  const int64_t valid = N - c;
  float m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = 0.0f;
  if (valid > 0) {
    for (int64_t k = k0 + wave; k < k1; k += 4) {
      Vec8<In> v;
      load8<In, kAligned>(W + k * ldw + c, valid, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(In::widen(v.v[i])));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = __float_as_uint(m[i]);
  __syncthreads();
  for (int j = threadIdx.x; j < kColStrip; j += blockDim.x) {
    uint32_t x = red[0][j];
    x = x > red[1][j] ? x : red[1][j];
    x = x > red[2][j] ? x : red[2][j];
    x = x > red[3][j] ? x : red[3][j];
    const int64_t col = int64_t(blockIdx.x) * kColStrip + j;
    if (col < N) atomicMax(&colmax[col], x);
  }
}

constexpr int kTK = 128;  // codes along K per tile (64 packed bytes)
constexpr int kTN = 64;   // columns per tile

template <class In, bool kAligned>
__global__ __launch_bounds__(256) void quantize_cols_kernel(
    const typename In::T* __restrict__ W, int64_t K, int64_t N, int64_t ldw,
    const uint32_t* __restrict__ colmax, uint8_t* __restrict__ Wq, int64_t ldq,
    float* __restrict__ sW) {
  __shared__ uint8_t codes[kTN][kTK + 4];
  __shared__ float inv_s[kTN];
  const int t = threadIdx.x;
  const int64_t n0 = int64_t(blockIdx.x) * kTN;
  const int64_t k0 = int64_t(blockIdx.y) * kTK;
  if (t < kTN) {
    const int64_t n = n0 + t;
    float s = 0.0f, inv = 0.0f;
    if (n < N) {
      vector_scale(__uint_as_float(colmax[n]), s, inv);
      if (blockIdx.y == 0) sW[n] = s;
    }
    inv_s[t] = inv;
  }
  __syncthreads();
  // load + encode: thread owns 8 columns x 4 rows
  const int g = t & 7;
  const int r0 = t >> 3;
  const int64_t c = n0 + g * 8;
  const int64_t valid = N - c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kl = r0 + 32 * i;
    const int64_t k = k0 + kl;
    Vec8<In> v;
    if (k < K && valid > 0) {
      load8<In, kAligned>(W + k * ldw + c, valid, v);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v.v[j] = typename In::T(0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float inv = inv_s[g * 8 + j];
      const uint32_t code = e2m1_magnitude(fabsf(In::widen(v.v[j])), inv) | (In::sign_bit(v.v[j]) << 3);
      codes[g * 8 + j][kl] = uint8_t((k < K && j < valid) ? code : 0u);
    }
  }
  __syncthreads();
  // transpose out: thread writes 16 bytes (32 codes) of one output row
  const int nl = t >> 2;
  const int part = t & 3;
  const int64_t n = n0 + nl;
  if (n < N) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) word |= uint32_t(codes[nl][part * 32 + q * 8 + j]) << (4 * j);
      w[q] = word;
    }
    uint4 out = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(Wq + n * ldq + k0 / 2 + part * 16) = out;
  }
}

template <class In, bool kAligned>
hipError_t run_quantize_weight(const void* Wp, int64_t K, int64_t N, int64_t ldw, uint8_t* Wq,
                               int64_t ldq, float* sW, void* ws, hipStream_t stream) {
  using T = typename In::T;
  const T* W = static_cast<const T*>(Wp);
  uint32_t* colmax = static_cast<uint32_t*>(ws);
  fill_u32_kernel<<<dim3(unsigned((N + 255) / 256 < 1024 ? (N + 255) / 256 : 1024)), 256, 0,
                    stream>>>(colmax, N, 0u);
  dim3 g1(unsigned((N + kColStrip - 1) / kColStrip), unsigned((K + kColRows - 1) / kColRows));
  colmax_kernel<In, kAligned><<<g1, 256, 0, stream>>>(W, K, N, ldw, colmax);
  dim3 g2(unsigned((N + kTN - 1) / kTN), unsigned((ldq * 2) / kTK));
  quantize_cols_kernel<In, kAligned><<<g2, 256, 0, stream>>>(W, K, N, ldw, colmax, Wq, ldq, sW);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows(const void* X, bool bf16, int64_t M, int64_t K, int64_t ldx,
                                const float* tau, uint8_t* Xq, int64_t ldq, float* sX,
                                hipStream_t stream) {
  const int esz = bf16 ? 2 : 4;
  const bool aligned = (reinterpret_cast<uintptr_t>(X) % 16 == 0) && ((ldx * esz) % 16 == 0);
  const unsigned blocks = unsigned((M + 3) / 4);
  if (bf16) {
    const uint16_t* x = static_cast<const uint16_t*>(X);
    if (aligned)
      quantize_rows_kernel<BF16In, true><<<blocks, 256, 0, stream>>>(x, M, K, ldx, tau, Xq, ldq, sX);
    else
      quantize_rows_kernel<BF16In, false><<<blocks, 256, 0, stream>>>(x, M, K, ldx, tau, Xq, ldq, sX);
  } else {
    const float* x = static_cast<const float*>(X);
    if (aligned)
      quantize_rows_kernel<F32In, true><<<blocks, 256, 0, stream>>>(x, M, K, ldx, tau, Xq, ldq, sX);
    else
      quantize_rows_kernel<F32In, false><<<blocks, 256, 0, stream>>>(x, M, K, ldx, tau, Xq, ldq, sX);
  }
  return hipGetLastError();
}

size_t weight_workspace_bytes(int64_t N) { return size_t(N) * 4; }

hipError_t launch_quantize_weight(const void* W, bool bf16, int64_t K, int64_t N, int64_t ldw,
                                  uint8_t* Wq, int64_t ldq, float* sW, void* ws,
                                  hipStream_t stream) {
  const int esz = bf16 ? 2 : 4;
  const bool aligned = (reinterpret_cast<uintptr_t>(W) % 16 == 0) && ((ldw * esz) % 16 == 0);
  if (bf16)
    return aligned ? run_quantize_weight<BF16In, true>(W, K, N, ldw, Wq, ldq, sW, ws, stream)
                   : run_quantize_weight<BF16In, false>(W, K, N, ldw, Wq, ldq, sW, ws, stream);
  return aligned ? run_quantize_weight<F32In, true>(W, K, N, ldw, Wq, ldq, sW, ws, stream)
                 : run_quantize_weight<F32In, false>(W, K, N, ldw, Wq, ldq, sW, ws, stream);
}

}  // namespace fp4lin
