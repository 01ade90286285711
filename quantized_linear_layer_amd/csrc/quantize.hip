// Vector-wise ScaleShift quantization to E2M1 (FP4 training write-up
// "微软首创FP4训练框架": the granularity paragraph — activations per row
// (token-wise), weights per column (channel-wise) — and the rounding and
// ScaleShift paragraphs — scale each vector into the FP4 range, then round to
// the nearest FP4 value).
//
// Rows:    one wave per row; the row (all of it, for K up to 8192 bfloat16,
//          16384 when the rows are 16-byte aligned, or 4096 float32) is loaded
//          into registers with every 16-byte load
//          issued before the first is used, reduced to the (clamped) row amax
//          with wave shuffles, and encoded from the registers, 8 codes per
//          32-bit store; the zero padding up to roundup(K,128) is written too.
// Columns: pass 1 takes per-column maxima of the K x N row-major weight with
//          loads coalesced along N (8 columns per lane, 8 rows in flight) and
//          merges them with integer atomicMax on the float bits (non-negative
//          floats order like their bits); pass 2 gives each thread 8 columns x
//          8 consecutive rows, so the 8 codes of one column along K are one
//          32-bit word of the column's packed (N-major) row, stored directly.
#include "colquant.hpp"
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

// One wave per row (workgroups of 4 waves striding over rows). The row is
// read in slabs of CH chunks per lane. When one slab covers the padded row
// (K up to 512 * CH) it stays in registers between the amax reduction and the
// encode, so A is read once; longer rows are read a second time for the
// encode.
template <class In, int CH>
__device__ inline void encode_slab(const Vec8<In> (&v)[CH], int64_t c0, int64_t K, int64_t Kp,
                                   float tau, float inv, uint8_t* __restrict__ qrow) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int64_t c = c0 + (int64_t(j) * kWave + lane) * 8;
    // chunks in [K, Kp) are zero and encode to the zero padding
    if (c < Kp) *reinterpret_cast<uint32_t*>(qrow + c / 2) = encode8<In>(v[j], K - c, tau, inv);
  }
}

template <class In, int CH>
__device__ inline float slab_absmax(const Vec8<In> (&v)[CH], float m) {
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(In::widen(v[j].v[i])));
  return m;
}

template <class In, bool kFast, int CH>
__global__ __launch_bounds__(kRowWaves * kWave) void quantize_rows_kernel(
    const typename In::T* __restrict__ X, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ tau_p, uint8_t* __restrict__ Xq, int64_t ldq,
    float* __restrict__ sX) {
  const float tau = tau_p ? *tau_p : __builtin_huge_valf();
  const int64_t slab = int64_t(kWave) * CH * 8;
  const int64_t Kp = ldq * 2;
  const int64_t stride = int64_t(gridDim.x) * kRowWaves;
  for (int64_t r = int64_t(blockIdx.x) * kRowWaves + threadIdx.x / kWave; r < M; r += stride) {
    const typename In::T* row = X + r * ldx;
    uint8_t* qrow = Xq + r * ldq;
    Vec8<In> v[CH];
    float m = 0.0f;
    for (int64_t c0 = 0; c0 < K; c0 += slab) {
      load_wave_slab<In, kFast, CH>(row, c0, K, v);
      m = slab_absmax<In, CH>(v, m);
    }
    const float amax = fminf(wave_max(m), tau);
    float s, inv;
    vector_scale(amax, s, inv);
    if ((threadIdx.x & (kWave - 1)) == 0) sX[r] = s;
    if (Kp <= slab) {
      encode_slab<In, CH>(v, 0, K, Kp, tau, inv, qrow);
    } else {
      for (int64_t c0 = 0; c0 < Kp; c0 += slab) {
        load_wave_slab<In, kFast, CH>(row, c0, K, v);
        encode_slab<In, CH>(v, c0, K, Kp, tau, inv, qrow);
      }
    }
  }
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

// One-dimensional grids over gx column tiles x row tiles (workgroup b takes
// tile (b % gx, b / gx)), so the number of row tiles along K is not held to
// the 65535 of a grid's second dimension.
template <class In, bool kAligned>
__global__ __launch_bounds__(256) void colmax_kernel(const typename In::T* __restrict__ W,
                                                     int64_t K, int64_t N, int64_t ldw,
                                                     uint32_t* __restrict__ colmax, int64_t gx) {
  colmax_body<In, kAligned>(blockIdx.x % gx, blockIdx.x / gx, W, K, N, ldw, colmax);
}

template <class In, bool kAligned>
__global__ __launch_bounds__(256) void quantize_cols_kernel(
    const typename In::T* __restrict__ W, int64_t K, int64_t N, int64_t ldw,
    const uint32_t* __restrict__ colmax, uint8_t* __restrict__ Wq, int64_t ldq,
    float* __restrict__ sW, int64_t gx) {
  quantize_cols_body<In, kAligned>(blockIdx.x % gx, blockIdx.x / gx, W, K, N, ldw, colmax, Wq,
                                   ldq, sW);
}

// the column maxima (into colmax, which starts at zero) and the codes
template <class In, bool kAligned>
void launch_col_passes(const typename In::T* W, int64_t K, int64_t N, int64_t ldw, uint8_t* Wq,
                       int64_t ldq, float* sW, uint32_t* colmax, hipStream_t stream) {
  const int64_t gx1 = (N + kColStrip - 1) / kColStrip;
  const int64_t g1 = gx1 * ((K + kColRows - 1) / kColRows);
  colmax_kernel<In, kAligned><<<dim3(unsigned(g1)), 256, 0, stream>>>(W, K, N, ldw, colmax, gx1);
  const int64_t gx2 = (N + kTN - 1) / kTN;
  const int64_t g2 = gx2 * ((ldq * 2) / kTK);
  quantize_cols_kernel<In, kAligned><<<dim3(unsigned(g2)), 256, 0, stream>>>(W, K, N, ldw, colmax,
                                                                             Wq, ldq, sW, gx2);
}

template <class In, bool kAligned>
hipError_t run_quantize_weight(const void* Wp, int64_t K, int64_t N, int64_t ldw, uint8_t* Wq,
                               int64_t ldq, float* sW, void* ws, hipStream_t stream) {
  using T = typename In::T;
  const T* W = static_cast<const T*>(Wp);
  uint32_t* colmax = static_cast<uint32_t*>(ws);
  fill_u32_kernel<<<dim3(unsigned((N + 255) / 256 < 1024 ? (N + 255) / 256 : 1024)), 256, 0,
                    stream>>>(colmax, N, 0u);
  launch_col_passes<In, kAligned>(W, K, N, ldw, Wq, ldq, sW, colmax, stream);
  return hipGetLastError();
}

// bfloat16 rows that are 16-byte aligned with K % 8 == 0 and fit one slab
// (K <= 512 * CH, CH up to 32): the raw 16-byte words are kept as loaded and
// quantized by quantize_bf16_row.
template <int CH>
__global__ __launch_bounds__(kRowWaves * kWave) void quantize_rows_bf16_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ tau_p, uint8_t* __restrict__ Xq, int64_t ldq,
    float* __restrict__ sX) {
  const float tau = tau_p ? *tau_p : __builtin_huge_valf();
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t stride = int64_t(gridDim.x) * kRowWaves;
  for (int64_t r = int64_t(blockIdx.x) * kRowWaves + threadIdx.x / kWave; r < M; r += stride) {
    const uint16_t* row = X + r * ldx;
    uint4 w[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int64_t c = (int64_t(j) * kWave + lane) * 8;
      w[j] = *reinterpret_cast<const uint4*>(row + (c < K ? c : K - 8));
      if (c >= K) w[j] = make_uint4(0, 0, 0, 0);
    }
    quantize_bf16_row<CH>(w, ldq * 2, tau, Xq + r * ldq, sX + r);
  }
}

template <class In, bool kFast>
hipError_t run_quantize_rows(const void* Xp, int64_t M, int64_t K, int64_t ldx, const float* tau,
                             uint8_t* Xq, int64_t ldq, float* sX, hipStream_t stream) {
  const typename In::T* X = static_cast<const typename In::T*>(Xp);
  const unsigned blocks = row_blocks(M);
  // rows up to 512 * CH padded columns kept in registers (bfloat16: 8192, or
  // 16384 for aligned rows; float32: 4096)
  constexpr int kMaxCh = In::kBytes == 2 ? 16 : 8;
  const int ch = chunks_per_lane(ldq * 2, kMaxCh);
  if constexpr (In::kBytes == 2 && kFast) {
    // rows of 8193 .. 16384 padded columns stay in registers too (32 chunks
    // per lane, two waves per SIMD) rather than being read twice
    if (ldq * 2 > int64_t(kWave) * 16 * 8 && ldq * 2 <= int64_t(kWave) * 32 * 8) {
      quantize_rows_bf16_kernel<32><<<blocks, kRowWaves * kWave, 0, stream>>>(X, M, K, ldx, tau, Xq, ldq, sX);
      return hipGetLastError();
    }
    if (int64_t(ch) * kWave * 8 >= ldq * 2) {
      switch (ch) {
        case 1: quantize_rows_bf16_kernel<1><<<blocks, kRowWaves * kWave, 0, stream>>>(X, M, K, ldx, tau, Xq, ldq, sX); break;
        case 2: quantize_rows_bf16_kernel<2><<<blocks, kRowWaves * kWave, 0, stream>>>(X, M, K, ldx, tau, Xq, ldq, sX); break;
        case 4: quantize_rows_bf16_kernel<4><<<blocks, kRowWaves * kWave, 0, stream>>>(X, M, K, ldx, tau, Xq, ldq, sX); break;
        case 8: quantize_rows_bf16_kernel<8><<<blocks, kRowWaves * kWave, 0, stream>>>(X, M, K, ldx, tau, Xq, ldq, sX); break;
        case 16: quantize_rows_bf16_kernel<16><<<blocks, kRowWaves * kWave, 0, stream>>>(X, M, K, ldx, tau, Xq, ldq, sX); break;
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    }
  }
  switch (ch) {
#define FP4LIN_QROWS(CH)                                                                      \
  case CH:                                                                                    \
    quantize_rows_kernel<In, kFast, CH><<<blocks, kRowWaves * kWave, 0, stream>>>(            \
        X, M, K, ldx, tau, Xq, ldq, sX);                                                      \
    break;
    FP4LIN_QROWS(1)
    FP4LIN_QROWS(2)
    FP4LIN_QROWS(4)
    FP4LIN_QROWS(8)
#undef FP4LIN_QROWS
    case 16:
      if constexpr (kMaxCh >= 16) {
        quantize_rows_kernel<In, kFast, 16><<<blocks, kRowWaves * kWave, 0, stream>>>(
            X, M, K, ldx, tau, Xq, ldq, sX);
        break;
      }
      return hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows(const void* X, bool bf16, int64_t M, int64_t K, int64_t ldx,
                                const float* tau, uint8_t* Xq, int64_t ldq, float* sX,
                                hipStream_t stream) {
  const int esz = bf16 ? 2 : 4;
  const bool fast = (reinterpret_cast<uintptr_t>(X) % 16 == 0) && ((ldx * esz) % 16 == 0) &&
                    (K % 8 == 0);
  if (bf16)
    return fast ? run_quantize_rows<BF16In, true>(X, M, K, ldx, tau, Xq, ldq, sX, stream)
                : run_quantize_rows<BF16In, false>(X, M, K, ldx, tau, Xq, ldq, sX, stream);
  return fast ? run_quantize_rows<F32In, true>(X, M, K, ldx, tau, Xq, ldq, sX, stream)
              : run_quantize_rows<F32In, false>(X, M, K, ldx, tau, Xq, ldq, sX, stream);
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
