// FP4 x FP4 GEMM on the gfx950 matrix cores with a fused epilogue.
//
// Role (FP4 training write-up "微软首创FP4训练框架", the GeMM-kernel paragraph): a
// dedicated FP4 matrix-multiply kernel stages packed FP4 tiles of A and B in
// shared memory, multiplies them block by block and reduces the partial
// results. That kernel simulated FP4 on FP8 tensor cores; here the product runs
// on CDNA4's native FP4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4 with both
// operands in E2M1 and unit E8M0 block scales, 127 = 2^0), accumulating in fp32.
// Every FP4 product is a multiple of 1/4 of magnitude <= 36 and |acc| <= 36*K,
// so the fp32 accumulation is exact for K < 2^24/144 whatever the order.
//
// Epilogue, per output element (the granularity paragraph: row scales of A and
// column scales of W factor out of the K reduction, so they are applied once,
// after it), then the sparse compensation of the outlier paragraph:
//   Y[i,j] = RN32(RN32(acc*sA[i])*sB[j]) + sum_{(i,k) in dA} val * W[k,j]
//
// Layout: A is M x ldq bytes and B is N x ldq bytes, both K-contiguous packed
// rows (two codes per byte, even index in the low nibble). A workgroup owns a
// BM x BN output tile and walks K in 256-code (128-byte) steps through a
// double-buffered LDS stage; each 16-byte chunk of a staged row is stored at
// chunk ^ (row & 7) so that the 32 lanes reading one chunk column of 32
// consecutive rows spread over all banks. For the 32x32x64 MFMA a lane supplies
// 32 consecutive codes (16 bytes) of one row of A (lane % 32) and of one
// column of B (lane % 32); lanes 32..63 supply the next 32 codes. A and B use
// the same code-to-lane assignment, so the k order inside the instruction does
// not matter for the (exact) sum.
//
// The output tile is staged through LDS 32 rows per wave row at a time; each
// wave then owns whole rows: it applies the scales, walks that row's non-zeros
// of dA (wave-uniform loop: one W row segment per non-zero, coalesced along N)
// and writes the row with contiguous stores.
#include "device_common.hpp"
#include "internal.hpp"

namespace fp4lin {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBKBytes = 128;  // 256 FP4 codes per K step

template <int BM, int BN, int WM, int WN>
struct GemmCfg {
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int kWaves = WM * WN;
  static constexpr int FM = BM / WM / 32;
  static constexpr int FN = BN / WN / 32;
  static constexpr int kAChunks = BM * 8 / kThreads;
  static constexpr int kBChunks = BN * 8 / kThreads;
  static constexpr int kStageBytes = (BM + BN) * kBKBytes;
  static constexpr int kEpiRows = WM * 32;
  static constexpr int kEpiLd = BN + 4;  // floats
  static constexpr int kEpiBytes = kEpiRows * kEpiLd * 4;
  static constexpr int kLdsBytes = (2 * kStageBytes > kEpiBytes) ? 2 * kStageBytes : kEpiBytes;
  static constexpr int kCPL = BN / 64;  // output columns per lane in the row phase
  static_assert(FM >= 1 && FN >= 1, "tile too small for the wave grid");
  static_assert(kAChunks >= 1 && kBChunks >= 1, "tile too small for the thread count");
  static_assert(kCPL == 4, "row phase assumes 4 columns per lane");
};

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2):
// give each XCD a contiguous run of tiles, and order tiles in groups of 8 tile
// rows sweeping across N so that neighbours share A rows and B columns.
__device__ inline void tile_coords(int bid, int nblocks, int tiles_m, int tiles_n, int& tm,
                                   int& tn) {
  const int xcd = bid & 7;
  const int idx = bid >> 3;
  const int base = nblocks >> 3, rem = nblocks & 7;
  const int t = xcd * base + (xcd < rem ? xcd : rem) + idx;
  constexpr int G = 8;
  const int per_group = G * tiles_n;
  const int grp = t / per_group;
  const int first_m = grp * G;
  const int gsize = (tiles_m - first_m) < G ? (tiles_m - first_m) : G;
  const int within = t - grp * per_group;
  tm = first_m + within % gsize;
  tn = within / gsize;
}

__device__ inline void load_w4(const void* __restrict__ W, int w_bf16, int64_t off, int valid,
                               bool vec, float w[4]) {
  if (w_bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(W) + off;
    if (vec && valid >= 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      w[0] = __uint_as_float(u.x << 16);
      w[1] = __uint_as_float(u.x & 0xffff0000u);
      w[2] = __uint_as_float(u.y << 16);
      w[3] = __uint_as_float(u.y & 0xffff0000u);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = (c < valid) ? __uint_as_float(uint32_t(p[c]) << 16) : 0.0f;
    }
  } else {
    const float* p = static_cast<const float*>(W) + off;
    if (vec && valid >= 4) {
      const float4 u = *reinterpret_cast<const float4*>(p);
      w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = (c < valid) ? p[c] : 0.0f;
    }
  }
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64, 1) void fp4_gemm_kernel(
    const uint8_t* __restrict__ Aq, const float* __restrict__ sA,
    const uint8_t* __restrict__ Bq, const float* __restrict__ sB, int M, int N, int ldq,
    int tiles_m, int tiles_n, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col, const float* __restrict__ val, const void* __restrict__ W,
    int w_bf16, int64_t ldw, int w_vec, float* __restrict__ Y, int64_t ldy, int y_vec) {
  using C = GemmCfg<BM, BN, WM, WN>;
  constexpr int FM = C::FM, FN = C::FN, NT = C::kThreads;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::kLdsBytes];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nkt = (ldq + kBKBytes - 1) / kBKBytes;

  uint4 ra[C::kAChunks], rb[C::kBChunks];
  auto gload = [&](int kt) {
    const int kb = kt * kBKBytes;
#pragma unroll
    for (int i = 0; i < C::kAChunks; ++i) {
      const int id = t + i * NT;
      const int row = id >> 3, c = id & 7;
      const int grow = (m0 + row < M) ? m0 + row : M - 1;
      const int off = kb + c * 16;
      ra[i] = (off < ldq) ? *reinterpret_cast<const uint4*>(Aq + int64_t(grow) * ldq + off)
                          : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < C::kBChunks; ++i) {
      const int id = t + i * NT;
      const int row = id >> 3, c = id & 7;
      const int gcol = (n0 + row < N) ? n0 + row : N - 1;
      const int off = kb + c * 16;
      rb[i] = (off < ldq) ? *reinterpret_cast<const uint4*>(Bq + int64_t(gcol) * ldq + off)
                          : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* As = lds + buf * C::kStageBytes;
    uint8_t* Bs = As + BM * kBKBytes;
#pragma unroll
    for (int i = 0; i < C::kAChunks; ++i) {
      const int id = t + i * NT;
      const int row = id >> 3, c = id & 7;
      *reinterpret_cast<uint4*>(As + row * kBKBytes + ((c ^ (row & 7)) << 4)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::kBChunks; ++i) {
      const int id = t + i * NT;
      const int row = id >> 3, c = id & 7;
      *reinterpret_cast<uint4*>(Bs + row * kBKBytes + ((c ^ (row & 7)) << 4)) = rb[i];
    }
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
    const uint8_t* As = lds + cur * C::kStageBytes;
    const uint8_t* Bs = As + BM * kBKBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      v8i a[FM], b[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int row = wm * (FM * 32) + fm * 32 + (lane & 31);
        const uint4 u = *reinterpret_cast<const uint4*>(As + row * kBKBytes + ((c ^ (row & 7)) << 4));
        a[fm] = v8i{int(u.x), int(u.y), int(u.z), int(u.w), 0, 0, 0, 0};
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int row = wn * (FN * 32) + fn * 32 + (lane & 31);
        const uint4 u = *reinterpret_cast<const uint4*>(Bs + row * kBKBytes + ((c ^ (row & 7)) << 4));
        b[fn] = v8i{int(u.x), int(u.y), int(u.z), int(u.w), 0, 0, 0, 0};
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              a[fm], b[fn], acc[fm][fn], 4, 4, 0, 127, 0, 127);
    }
    if (kt + 1 < nkt) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
  float* Ys = reinterpret_cast<float*>(lds);
  constexpr int CPL = C::kCPL;
  const int jl = lane * CPL;
  const int valid_n = N - (n0 + jl);
  float sb[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) sb[c] = (c < valid_n) ? sB[n0 + jl + c] : 0.0f;

#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int lcol = wn * (FN * 32) + fn * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lrow = wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        Ys[lrow * C::kEpiLd + lcol] = acc[fm][fn][r];
      }
    }
    __syncthreads();
    for (int lr = wave; lr < C::kEpiRows; lr += C::kWaves) {
      const int grow = m0 + (lr >> 5) * (FM * 32) + fm * 32 + (lr & 31);
      if (grow >= M) continue;
      const float sa = sA[grow];
      float y[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) y[c] = __fmul_rn(__fmul_rn(Ys[lr * C::kEpiLd + jl + c], sa), sb[c]);
      if (row_ptr != nullptr) {
        const int e0 = row_ptr[grow], e1 = row_ptr[grow + 1];
        for (int e = e0; e < e1; ++e) {
          const int64_t k = col[e];
          const float v = val[e];
          float w[CPL];
          load_w4(W, w_bf16, k * ldw + n0 + jl, valid_n, w_vec != 0, w);
#pragma unroll
          for (int c = 0; c < CPL; ++c) y[c] = fmaf(v, w[c], y[c]);
        }
      }
      float* yrow = Y + int64_t(grow) * ldy + n0 + jl;
      if (y_vec && valid_n >= 4) {
        *reinterpret_cast<float4*>(yrow) = make_float4(y[0], y[1], y[2], y[3]);
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          if (c < valid_n) yrow[c] = y[c];
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_fp4_gemm(const uint8_t* Aq, const float* sA, const uint8_t* Bq, const float* sB,
                           int64_t M, int64_t N, int64_t ldq, const SparseArgs& sp, float* Y,
                           int64_t ldy, hipStream_t stream) {
  constexpr int BM = 256, BN = 256, WM = 2, WN = 2;
  const int tiles_m = int((M + BM - 1) / BM);
  const int tiles_n = int((N + BN - 1) / BN);
  const int nblocks = tiles_m * tiles_n;
  const int esz = sp.w_bf16 ? 2 : 4;
  const bool w_vec = sp.W != nullptr && (reinterpret_cast<uintptr_t>(sp.W) % 16 == 0) &&
                     ((sp.ldw * esz) % 16 == 0);
  const bool y_vec = (reinterpret_cast<uintptr_t>(Y) % 16 == 0) && (ldy % 4 == 0);
  fp4_gemm_kernel<BM, BN, WM, WN><<<dim3(unsigned(nblocks)), WM * WN * 64, 0, stream>>>(
      Aq, sA, Bq, sB, int(M), int(N), int(ldq), tiles_m, tiles_n, sp.row_ptr, sp.col, sp.val,
      sp.W, sp.w_bf16 ? 1 : 0, sp.ldw, w_vec ? 1 : 0, Y, ldy, y_vec ? 1 : 0);
  return hipGetLastError();
}

}  // namespace fp4lin
