// Sparse compensation term of the FP4 linear layer: Y += dA . W.
//
// The outlier paragraph of the FP4 training write-up ("微软首创FP4训练框架") keeps
// the clipped residue dA = A - A_clamped as a sparse matrix that is non-zero
// only where A was clamped; its product with the unquantized weight is added
// to the FP4 product so that the outliers are not lost.
//
// One single-wave workgroup owns one (row i, 512-column strip) unit: it forms
//   s = sum over the row's non-zeros (k ascending) of val * W[k, strip]
// from 0 with fp32 fused multiply-add, then adds s once to Y[i, strip] (the
// scaled FP4 product the GEMM kernel wrote; its load is issued first, so that
// it arrives while the gathers run). Each lane owns 8 consecutive columns, so
// a non-zero costs one 16-byte (bf16) W load per lane, addressed with the row
// offset in the scalar operand of a buffer load; the row's entries are read
// with scalar loads. The gathers go out in groups of four, software-pipelined:
// the entries of group g+2 are requested while the W rows of group g+1 are in
// flight and group g is multiplied. Y is stored with non-temporal stores, so
// the stream of Y lines does not evict the W strip from L2.
// Units are ordered strip by strip and each XCD takes a contiguous run of that
// order, so the waves running together on an XCD read the same W strip
// through its L2. Single-wave workgroups free their slot as soon as their own
// row is done. Rows without non-zeros are left untouched.
#include <type_traits>

#include "device_common.hpp"
#include "internal.hpp"

namespace fp4lin {

namespace {

constexpr int kCPL = 8;                // columns per lane
constexpr int kStrip = 64 * kCPL;      // columns per unit
// W row segments per load group (two groups in flight). Small groups keep the
// register count low enough for 8 waves per SIMD: each wave's work is a short
// chain (row bounds, entries, gathers, Y), so many independent waves hide the
// latency better than deep per-wave pipelines do.
constexpr int kGroup = 4;
constexpr int kBufferFlags = 0x00020000;  // raw buffer resource word 3 (gfx9 family)

// W words of one non-zero for this lane's 8 columns: bf16 -> one 16-byte
// word, fp32 -> two. Converted to fp32 when consumed.
template <bool kBf16>
struct WRaw {
  uint4 u[kBf16 ? 1 : 2];
};

template <bool kBf16>
__device__ inline void fma_raw(float v, const WRaw<kBf16>& r, float y[kCPL]) {
  if constexpr (kBf16) {
    const uint32_t d[4] = {r.u[0].x, r.u[0].y, r.u[0].z, r.u[0].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      y[2 * q] = fmaf(v, __uint_as_float(d[q] << 16), y[2 * q]);
      y[2 * q + 1] = fmaf(v, __uint_as_float(d[q] & 0xffff0000u), y[2 * q + 1]);
    }
  } else {
    const uint32_t d[8] = {r.u[0].x, r.u[0].y, r.u[0].z, r.u[0].w,
                           r.u[1].x, r.u[1].y, r.u[1].z, r.u[1].w};
#pragma unroll
    for (int c = 0; c < kCPL; ++c) y[c] = fmaf(v, __uint_as_float(d[c]), y[c]);
  }
}

// Full-width load of W[k, col0 .. col0+7] through the buffer resource: the row
// offset k*ldw is wave-uniform and goes in the scalar offset, the column
// offset is the lane's constant vector offset.
template <bool kBf16>
__device__ inline WRaw<kBf16> load_full(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  WRaw<kBf16> r;
  r.u[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
  if constexpr (!kBf16)
    r.u[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, soff, 0));
  return r;
}

// Element loads for a lane whose 8 columns run past N (last strip only).
template <bool kBf16>
__device__ inline WRaw<kBf16> load_part(const void* __restrict__ W, int64_t off, int valid) {
  WRaw<kBf16> r;
  if constexpr (kBf16) {
    const uint16_t* p = static_cast<const uint16_t*>(W) + off;
    uint32_t h[kCPL];
#pragma unroll
    for (int c = 0; c < kCPL; ++c) h[c] = (c < valid) ? uint32_t(p[c]) : 0u;
    r.u[0] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                        h[6] | (h[7] << 16));
  } else {
    const float* p = static_cast<const float*>(W) + off;
    uint32_t h[kCPL];
#pragma unroll
    for (int c = 0; c < kCPL; ++c) h[c] = (c < valid) ? __float_as_uint(p[c]) : 0u;
    r.u[0] = make_uint4(h[0], h[1], h[2], h[3]);
    r.u[1] = make_uint4(h[4], h[5], h[6], h[7]);
  }
  return r;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Y is streamed once per unit. The result is stored non-temporally, so the
// stream of Y lines does not evict the W strip that the gathers reuse from L2.
// When Y and W together exceed what the last-level cache holds (kStreamY) the
// Y read is non-temporal too, which keeps W resident there for the gathers;
// below that a plain load measured faster (Y then stays cached itself).
template <bool kStreamY>
__device__ inline f32x4 load_y4(const float* p) {
  if constexpr (kStreamY)
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  else
    return *reinterpret_cast<const f32x4*>(p);
}
__device__ inline void store_y4(f32x4 v, float* p) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

template <bool kBf16, bool kStreamY>
__global__ __launch_bounds__(64) void sparse_add_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
    const float* __restrict__ val, const void* __restrict__ W, int64_t ldw, int w_bytes,
    int w_vec, float* __restrict__ Y, int64_t ldy, int y_vec, int M, int N, int64_t unit_base,
    int64_t units) {
  constexpr int esz = kBf16 ? 2 : 4;
  const int lane = threadIdx.x & 63;
  // XCD-contiguous unit order (workgroups go round-robin over the 8 XCDs)
  const int64_t nb = gridDim.x;
  const int64_t xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const int64_t base_b = nb >> 3, rem = nb & 7;
  const int64_t unit = unit_base + xcd * base_b + (xcd < rem ? xcd : rem) + idx;
  if (unit >= units) return;
  const int strip = int(unit / M);
  const int row = int(unit - int64_t(strip) * M);
  const int e0 = row_ptr[row], e1 = row_ptr[row + 1];
  if (e0 >= e1) return;

  const int col0 = strip * kStrip + lane * kCPL;
  const int valid = N - col0;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(W), 0, w_bytes, kBufferFlags);
  // Column byte offset of the lane's 8 columns inside a W row. The buffer's
  // range check does not cover the row offset in the scalar operand, so in the
  // vector path (N a multiple of 8, or a strip wholly below N) a lane past N
  // reads the row's last 8 columns instead of memory past the row; it stores
  // nothing.
  const int voff = (col0 + kCPL <= N ? col0 : N - kCPL) * esz;
  const int row_bytes = int(ldw) * esz;
  const bool y_full = y_vec && valid >= kCPL;

  float* yrow = Y + int64_t(row) * ldy + col0;
  // Y segment requested before the gathers so that its latency is hidden
  float yo[kCPL];
  if (valid > 0) {
    if (y_full) {
      const f32x4 u0 = load_y4<kStreamY>(yrow), u1 = load_y4<kStreamY>(yrow + 4);
      yo[0] = u0[0]; yo[1] = u0[1]; yo[2] = u0[2]; yo[3] = u0[3];
      yo[4] = u1[0]; yo[5] = u1[1]; yo[6] = u1[2]; yo[7] = u1[3];
    } else {
#pragma unroll
      for (int c = 0; c < kCPL; ++c) yo[c] = (c < valid) ? yrow[c] : 0.0f;
    }
  }

  float y[kCPL];  // the compensation sum, from 0; added to Y at the end
#pragma unroll
  for (int c = 0; c < kCPL; ++c) y[c] = 0.0f;

  const int n = e1 - e0;
  const int ng = (n + kGroup - 1) / kGroup;
  const int32_t* __restrict__ cp = col + e0;
  const float* __restrict__ vp = val + e0;
  // Entries of group g (wave-uniform, scalar loads). In the row's last group
  // the indexes are clamped to its last entry and the extra slots get weight
  // 0 (an integer mask, so the selection stays scalar), so every group is
  // full and every read stays inside the row.
  auto entries = [&](int g, int (&kk)[kGroup], float (&vv)[kGroup]) {
    const int j0 = g * kGroup;
    if (j0 + kGroup <= n) {
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        kk[u] = cp[j0 + u];
        vv[u] = vp[j0 + u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        const int j = min(j0 + u, n - 1);
        kk[u] = cp[j];
        const uint32_t keep = (j0 + u < n) ? 0xffffffffu : 0u;
        vv[u] = __uint_as_float(__float_as_uint(vp[j]) & keep);
      }
    }
  };
  auto gather = [&](const int (&kk)[kGroup], WRaw<kBf16> (&w)[kGroup]) {
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      w[u] = load_full<kBf16>(rs, voff, kk[u] * row_bytes);
    }
  };
  auto multiply = [&](const float (&vv)[kGroup], const WRaw<kBf16> (&w)[kGroup]) {
#pragma unroll
    for (int u = 0; u < kGroup; ++u) fma_raw<kBf16>(vv[u], w[u], y);
  };

  // Every lane holds 8 columns or none (no lane straddles N), and W rows are
  // 16-byte aligned: one 16-byte buffer load per entry and lane. Lanes past N
  // load the row's last 8 columns and store nothing.
  const bool vec_path = w_vec != 0 && ((N % kCPL) == 0 || (strip + 1) * kStrip <= N);
  if (vec_path) {
    // Software pipeline over groups, two W buffers used in turn: the entries
    // of group g+2 are requested while the W rows of group g+1 are in flight
    // and group g is multiplied.
    int kA[kGroup], kB[kGroup];
    float vA[kGroup], vB[kGroup];
    WRaw<kBf16> wA[kGroup], wB[kGroup];
    entries(0, kA, vA);
    gather(kA, wA);
    if (ng > 1) entries(1, kB, vB);
    for (int g = 0; g < ng; g += 2) {
      int k2[kGroup];
      float v2[kGroup];
      if (g + 1 < ng) gather(kB, wB);
      if (g + 2 < ng) entries(g + 2, k2, v2);
      multiply(vA, wA);
      if (g + 1 >= ng) break;
      if (g + 2 < ng) gather(k2, wA);
      if (g + 3 < ng) entries(g + 3, kA, vA);  // kA/vA are free: group g is done
      multiply(vB, wB);
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        kB[u] = kA[u];  // group g+3 entries
        vB[u] = vA[u];
        vA[u] = v2[u];  // group g+2 values (its W rows are in wA)
      }
    }
  } else {
    // Unaligned W or a ragged last strip: per-lane element loads where a lane
    // straddles N, one group of entries at a time.
    const bool full = w_vec != 0 && valid >= kCPL;
    for (int g = 0; g < ng; ++g) {
      int kk[kGroup];
      float vv[kGroup];
      entries(g, kk, vv);
      WRaw<kBf16> w[kGroup];
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        if (full)
          w[u] = load_full<kBf16>(rs, voff, kk[u] * row_bytes);
        else if (valid > 0)
          w[u] = load_part<kBf16>(W, int64_t(kk[u]) * ldw + col0, valid);
        else
          w[u] = WRaw<kBf16>{};
      }
#pragma unroll
      for (int u = 0; u < kGroup; ++u) fma_raw<kBf16>(vv[u], w[u], y);
    }
  }

  if (valid > 0) {
    if (y_full) {
      store_y4(f32x4{__fadd_rn(yo[0], y[0]), __fadd_rn(yo[1], y[1]), __fadd_rn(yo[2], y[2]),
                     __fadd_rn(yo[3], y[3])}, yrow);
      store_y4(f32x4{__fadd_rn(yo[4], y[4]), __fadd_rn(yo[5], y[5]), __fadd_rn(yo[6], y[6]),
                     __fadd_rn(yo[7], y[7])}, yrow + 4);
    } else {
#pragma unroll
      for (int c = 0; c < kCPL; ++c)
        if (c < valid) yrow[c] = __fadd_rn(yo[c], y[c]);
    }
  }
}

}  // namespace

hipError_t launch_sparse_add(const SparseArgs& sp, int64_t M, int64_t N, float* Y, int64_t ldy,
                             hipStream_t stream) {
  const int64_t strips = (N + kStrip - 1) / kStrip;
  const int64_t units = strips * M;
  const int64_t esz = sp.w_bf16 ? 2 : 4;
  // Vector access of a lane's 8 columns needs every row start of W 16-byte
  // aligned and of Y 16-byte aligned (column offsets are multiples of 8).
  const bool w_vec = (reinterpret_cast<uintptr_t>(sp.W) % 16 == 0) && ((sp.ldw * esz) % 16 == 0);
  const bool y_vec = (reinterpret_cast<uintptr_t>(Y) % 16 == 0) && (ldy % 4 == 0);
  const int w_bytes = int(sp.w_rows * sp.ldw * esz);
  // One single-wave workgroup per unit, launched in chunks that keep the
  // thread count of one launch below 2^32.
  constexpr int64_t kChunk = int64_t(1) << 24;
  const bool stream_y = M * N * 4 + sp.w_rows * N * esz > kStreamBytes;
  auto run = [&](auto bf16_c, auto stream_c, int64_t base, int64_t blocks) {
    sparse_add_kernel<decltype(bf16_c)::value, decltype(stream_c)::value>
        <<<dim3(unsigned(blocks)), 64, 0, stream>>>(sp.row_ptr, sp.col, sp.val, sp.W, sp.ldw,
                                                    w_bytes, w_vec ? 1 : 0, Y, ldy,
                                                    y_vec ? 1 : 0, int(M), int(N), base,
                                                    base + blocks);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  for (int64_t base = 0; base < units; base += kChunk) {
    const int64_t blocks = units - base < kChunk ? units - base : kChunk;
    if (sp.w_bf16)
      stream_y ? run(T_{}, T_{}, base, blocks) : run(T_{}, F_{}, base, blocks);
    else
      stream_y ? run(F_{}, T_{}, base, blocks) : run(F_{}, F_{}, base, blocks);
  }
  return hipGetLastError();
}

}  // namespace fp4lin
