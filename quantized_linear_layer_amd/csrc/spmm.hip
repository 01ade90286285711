// Sparse compensation term of the FP4 linear layer: Y += dA . W.
//
// The outlier paragraph of the FP4 training write-up ("微软首创FP4训练框架") keeps
// the clipped residue dA = A - A_clamped as a sparse matrix that is non-zero
// only where A was clamped; its product with the unquantized weight is added
// to the FP4 product so that the outliers are not lost.
//
// One wave owns one (row i, 512-column strip) unit: it reads Y[i, strip] (the
// scaled FP4 product the GEMM kernel just wrote), adds
//   sum over the row's non-zeros (k ascending) of val * W[k, strip]
// with fp32 fused multiply-add, and writes it back. Each lane owns 8
// consecutive columns, so a non-zero costs one 16-byte W load per lane. The
// row's non-zeros are fetched 64 at a time (one per lane) and walked with
// eight W row segments in flight. Units are ordered strip by strip, and each
// XCD takes a contiguous run of that order, so the waves running together on
// an XCD read the same W strip through its L2. Rows without non-zeros are
// left untouched.
#include "device_common.hpp"
#include "internal.hpp"

namespace fp4lin {

namespace {

constexpr int kStrip = 512;  // columns per unit (8 per lane)
constexpr int kCPL = 8;

template <bool kBf16>
__device__ inline void load_w8(const void* __restrict__ W, int64_t off, int valid, bool vec,
                               float w[kCPL]) {
  if constexpr (kBf16) {
    const uint16_t* p = static_cast<const uint16_t*>(W) + off;
    if (vec && valid >= kCPL) {
      const uint4 u = *reinterpret_cast<const uint4*>(p);
      const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[2 * q] = __uint_as_float(d[q] << 16);
        w[2 * q + 1] = __uint_as_float(d[q] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int c = 0; c < kCPL; ++c) w[c] = (c < valid) ? __uint_as_float(uint32_t(p[c]) << 16) : 0.0f;
    }
  } else {
    const float* p = static_cast<const float*>(W) + off;
    if (vec && valid >= kCPL) {
      const float4 u0 = *reinterpret_cast<const float4*>(p);
      const float4 u1 = *reinterpret_cast<const float4*>(p + 4);
      w[0] = u0.x; w[1] = u0.y; w[2] = u0.z; w[3] = u0.w;
      w[4] = u1.x; w[5] = u1.y; w[6] = u1.z; w[7] = u1.w;
    } else {
#pragma unroll
      for (int c = 0; c < kCPL; ++c) w[c] = (c < valid) ? p[c] : 0.0f;
    }
  }
}

__device__ inline float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

template <bool kBf16>
__global__ __launch_bounds__(256) void sparse_add_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
    const float* __restrict__ val, const void* __restrict__ W, int64_t ldw, int w_vec,
    float* __restrict__ Y, int64_t ldy, int y_vec, int M, int N, int64_t units) {
  const int lane = threadIdx.x & 63;
  // XCD-contiguous unit order (workgroups go round-robin over the 8 XCDs)
  const int64_t nb = gridDim.x;
  const int64_t xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const int64_t base_b = nb >> 3, rem = nb & 7;
  const int64_t blk = xcd * base_b + (xcd < rem ? xcd : rem) + idx;
  const int64_t unit = blk * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (unit >= units) return;
  const int strip = int(unit / M);
  const int row = int(unit - int64_t(strip) * M);
  const int e0 = row_ptr[row], e1 = row_ptr[row + 1];
  if (e0 >= e1) return;

  const int64_t col0 = int64_t(strip) * kStrip + lane * kCPL;
  const int valid = int(N - col0);
  float y[kCPL];
  float* yrow = Y + int64_t(row) * ldy + col0;
  if (valid > 0) {
    if (y_vec && valid >= kCPL) {
      const float4 u0 = *reinterpret_cast<const float4*>(yrow);
      const float4 u1 = *reinterpret_cast<const float4*>(yrow + 4);
      y[0] = u0.x; y[1] = u0.y; y[2] = u0.z; y[3] = u0.w;
      y[4] = u1.x; y[5] = u1.y; y[6] = u1.z; y[7] = u1.w;
    } else {
#pragma unroll
      for (int c = 0; c < kCPL; ++c) y[c] = (c < valid) ? yrow[c] : 0.0f;
    }
  } else {
#pragma unroll
    for (int c = 0; c < kCPL; ++c) y[c] = 0.0f;
  }

  const bool vec = w_vec != 0;
  for (int base = e0; base < e1; base += 64) {
    const int n = (e1 - base) < 64 ? (e1 - base) : 64;
    int mk = 0;
    float mv = 0.0f;
    if (lane < n) {
      mk = col[base + lane];
      mv = val[base + lane];
    }
    int j = 0;
    for (; j + 8 <= n; j += 8) {
      float w[8][kCPL];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t k = __builtin_amdgcn_readlane(mk, j + u);
        if (valid > 0) load_w8<kBf16>(W, k * ldw + col0, valid, vec, w[u]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float v = readlane_f(mv, j + u);
#pragma unroll
        for (int c = 0; c < kCPL; ++c) y[c] = fmaf(v, w[u][c], y[c]);
      }
    }
    for (; j < n; ++j) {
      const int64_t k = __builtin_amdgcn_readlane(mk, j);
      float w[kCPL];
      if (valid > 0) load_w8<kBf16>(W, k * ldw + col0, valid, vec, w);
      const float v = readlane_f(mv, j);
#pragma unroll
      for (int c = 0; c < kCPL; ++c) y[c] = fmaf(v, w[c], y[c]);
    }
  }

  if (valid > 0) {
    if (y_vec && valid >= kCPL) {
      *reinterpret_cast<float4*>(yrow) = make_float4(y[0], y[1], y[2], y[3]);
      *reinterpret_cast<float4*>(yrow + 4) = make_float4(y[4], y[5], y[6], y[7]);
    } else {
#pragma unroll
      for (int c = 0; c < kCPL; ++c)
        if (c < valid) yrow[c] = y[c];
    }
  }
}

}  // namespace

hipError_t launch_sparse_add(const SparseArgs& sp, int64_t M, int64_t N, float* Y, int64_t ldy,
                             hipStream_t stream) {
  const int64_t strips = (N + kStrip - 1) / kStrip;
  const int64_t units = strips * M;
  const int64_t blocks = (units + 3) / 4;
  const int64_t esz = sp.w_bf16 ? 2 : 4;
  // 16-byte vector access needs every row start of W and Y 16-byte aligned
  // (column offsets are multiples of 8 elements).
  const bool w_vec = (reinterpret_cast<uintptr_t>(sp.W) % 16 == 0) && ((sp.ldw * esz) % 16 == 0);
  const bool y_vec = (reinterpret_cast<uintptr_t>(Y) % 16 == 0) && ((ldy * 4) % 16 == 0);
  if (sp.w_bf16)
    sparse_add_kernel<true><<<dim3(unsigned(blocks)), 256, 0, stream>>>(
        sp.row_ptr, sp.col, sp.val, sp.W, sp.ldw, w_vec ? 1 : 0, Y, ldy, y_vec ? 1 : 0, int(M),
        int(N), units);
  else
    sparse_add_kernel<false><<<dim3(unsigned(blocks)), 256, 0, stream>>>(
        sp.row_ptr, sp.col, sp.val, sp.W, sp.ldw, w_vec ? 1 : 0, Y, ldy, y_vec ? 1 : 0, int(M),
        int(N), units);
  return hipGetLastError();
}

}  // namespace fp4lin
