// FP4 x FP4 GEMM on the gfx950 matrix cores with the scale epilogue.
//
// Role (FP4 training write-up "微软首创FP4训练框架", the GeMM-kernel paragraph): a
// dedicated FP4 matrix-multiply kernel stages packed FP4 tiles of A and B in
// shared memory, multiplies them block by block and reduces the partial
// results. That kernel simulated FP4 on FP8 tensor cores; here the product runs
// on CDNA4's native FP4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4 with both
// operands in E2M1 and unit E8M0 block scales, 127 = 2^0), accumulating in fp32.
// Every FP4 product is a multiple of 1/4 of magnitude <= 36 and |acc| <= 36*K,
// so the fp32 accumulation is exact for K < 2^24/144 whatever the order.
// (The 32x32x64 shape is used because on gfx950 it runs FP4 at twice the FP8
// rate; the 16x16x128 shape runs FP4 at the FP8 rate.)
//
// Epilogue (the granularity paragraph: row scales of A and column scales of W
// factor out of the K reduction, so they are applied once, after it):
//   Y[i,j] = RN32(RN32(acc[i,j] * sA[i]) * sB[j])
// The sparse compensation term is added afterwards by spmm.hip.
//
// Layout and schedule:
//  * A is M x ldq bytes and B is N x ldq bytes, K-contiguous packed rows.
//  * A workgroup of 4 waves (2 x 2 grid, each wave 64 x 128 outputs) owns a
//    128 x 256 output tile and walks K in 128-code (64-byte) steps through a
//    double-buffered LDS stage (48 KiB). Operand loads are buffer loads held in
//    registers and issued two K steps before they are stored to LDS. Two
//    workgroups share a CU, so one's stores overlap the other's MFMA loop.
//  * Each 16-byte chunk of a staged row is stored at a chunk index XOR-ed with
//    row bits, so that the lanes reading one chunk column of consecutive rows
//    hit distinct banks.
//  * For the 32x32x64 MFMA a lane supplies 32 consecutive codes (16 bytes) of
//    one row of A (lane % 32) and of one column of B (lane % 32); lanes 32..63
//    supply the next 32 codes. A and B use the same code-to-lane assignment,
//    so the k order inside the instruction does not matter for the exact sum.
//  * Tiles are visited in groups of 4 tile rows sweeping across N, and each of
//    the 8 XCDs (own L2 each; workgroups are dispatched round-robin over them)
//    takes a contiguous run of that order, so concurrent tiles on an XCD share
//    A rows and B columns in its L2.
//  * The scaled tile leaves through LDS: each wave writes two 32 x 32
//    fragments at a time into its own block of the (then idle) stage buffers
//    and stores them back as rows, 16 bytes per lane, so Y is written with
//    full-width stores of whole 256-byte row segments (4x fewer store
//    instructions than storing from the MFMA layout). The stores are
//    non-temporal: the output stream is not kept in L2 at the expense of the
//    operand tiles that concurrent workgroups re-read.
#include "device_common.hpp"
#include "internal.hpp"

namespace fp4lin {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format,
// no swizzle); with stride 0 the bounds check is offset < num_records.
constexpr int kBufferFlags = 0x00020000;

template <int BM_, int BN_, int WM_, int WN_, int BKB_, int MINB_, int STAGES_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BKB = BKB_;
  static constexpr int kMinBlocks = MINB_;  // workgroups per CU the register budget targets
  static constexpr int kStages = STAGES_;   // K steps of operand loads in flight (registers)
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int FM = BM / WM / 32;
  static constexpr int FN = BN / WN / 32;
  static constexpr int CPR = BKB / 16;            // 16-byte chunks per staged row
  static constexpr int kSub = BKB / 32;            // 64-code MFMA steps per K step
  static constexpr int kAChunks = BM * CPR / kThreads;
  static constexpr int kBChunks = BN * CPR / kThreads;
  static constexpr int kStageBytes = (BM + BN) * BKB;
  static_assert(FM >= 1 && FN >= 1, "tile too small for the wave grid");
  static_assert(kAChunks >= 1 && kBChunks >= 1, "tile too small for the thread count");
  static_assert(BM * CPR % kThreads == 0 && BN * CPR % kThreads == 0, "uneven tile load");
  static_assert(CPR == 4 || CPR == 8, "swizzle assumes 64- or 128-byte staged rows");
};

// Physical 16-byte chunk of logical chunk c in staged row r. A 128-bit LDS
// read of 32 consecutive rows at one logical chunk must not put two lanes of
// the same bank group on one bank; the mapping below spreads every aligned
// group of 16 consecutive rows over 256 distinct bytes (64 banks) and every
// aligned group of 8 rows over 128 distinct bytes (32 banks):
//   64-byte rows:  chunk ^ (((r >> 1) ^ (r >> 3)) & 3)
//   128-byte rows: chunk ^ ((r ^ (r >> 3)) & 7)
template <int CPR>
__device__ inline int swz(int r, int c) {
  if constexpr (CPR == 4) return c ^ (((r >> 1) ^ (r >> 3)) & 3);
  return c ^ ((r ^ (r >> 3)) & 7);
}

// Tile order: groups of G tile rows sweeping across N; each XCD takes a
// contiguous run of that order (a bijection from workgroup id to tile).
__device__ inline void tile_coords(int bid, int nblocks, int tiles_m, int& tm, int& tn) {
  const int xcd = bid & 7;
  const int idx = bid >> 3;
  const int base = nblocks >> 3, rem = nblocks & 7;
  const int t = xcd * base + (xcd < rem ? xcd : rem) + idx;
  const int tiles_n = nblocks / tiles_m;
  constexpr int G = 4;
  const int per_group = G * tiles_n;
  const int grp = t / per_group;
  const int first_m = grp * G;
  const int gsize = (tiles_m - first_m) < G ? (tiles_m - first_m) : G;
  const int within = t - grp * per_group;
  tm = first_m + within % gsize;
  tn = within / gsize;
}

template <class C>
__global__ __launch_bounds__(C::kThreads, C::kMinBlocks) void fp4_gemm_kernel(
    const uint8_t* __restrict__ Aq, const float* __restrict__ sA,
    const uint8_t* __restrict__ Bq, const float* __restrict__ sB, int M, int N, int ldq,
    int tiles_m, float* __restrict__ Y, int64_t ldy) {
  constexpr int BM = C::BM, BN = C::BN, WN = C::WN, BKB = C::BKB, CPR = C::CPR;
  constexpr int FM = C::FM, FN = C::FN, NT = C::kThreads;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::kStageBytes];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nkt = (ldq + BKB - 1) / BKB;

  // Operand tiles are fetched with buffer loads: the resource descriptor holds
  // the base and the byte size of the packed matrix, and the hardware returns
  // zeros for any offset past the end, so rows past M (or N) read as zero
  // codes. Each thread keeps one 32-bit offset per 16-byte chunk (the K step is
  // added to it, inside the checked offset). Chunk c of a thread is fixed (the
  // thread count is a multiple of the chunks per row). The host keeps
  // (rows + 1) * ldq below 2^31.
  const int tc = t % CPR;
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(Aq), 0, int(int64_t(M) * ldq), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsB =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(Bq), 0, int(int64_t(N) * ldq), kBufferFlags);
  int a_off[C::kAChunks], b_off[C::kBChunks];
#pragma unroll
  for (int i = 0; i < C::kAChunks; ++i) {
    const int row = (t + i * NT) / CPR;
    a_off[i] = (m0 + row < M) ? (m0 + row) * ldq + tc * 16 : int(int64_t(M) * ldq);
  }
#pragma unroll
  for (int i = 0; i < C::kBChunks; ++i) {
    const int row = (t + i * NT) / CPR;
    b_off[i] = (n0 + row < N) ? (n0 + row) * ldq + tc * 16 : int(int64_t(N) * ldq);
  }

  constexpr int S = C::kStages;
  uint4 ra[S][C::kAChunks], rb[S][C::kBChunks];
  // K tail: a chunk past the packed row length would read the next row, so it
  // is replaced by zero codes (the load itself stays in bounds).
  auto gload = [&](int kt, int slot) {
    const int kb = kt * BKB;
    const bool ok = kb + tc * 16 < ldq;
#pragma unroll
    for (int i = 0; i < C::kAChunks; ++i) {
      const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsA, a_off[i] + kb, 0, 0));
      ra[slot][i] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < C::kBChunks; ++i) {
      const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsB, b_off[i] + kb, 0, 0));
      rb[slot][i] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto lstore = [&](int buf, int slot) {
    uint8_t* base = lds + buf * C::kStageBytes;
#pragma unroll
    for (int i = 0; i < C::kAChunks; ++i) {
      const int row = (t + i * NT) / CPR;
      *reinterpret_cast<uint4*>(base + row * BKB + (swz<CPR>(row, tc) << 4)) = ra[slot][i];
    }
#pragma unroll
    for (int i = 0; i < C::kBChunks; ++i) {
      const int row = (t + i * NT) / CPR;
      *reinterpret_cast<uint4*>(base + BM * BKB + row * BKB + (swz<CPR>(row, tc) << 4)) = rb[slot][i];
    }
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

  // fragment source offsets inside a stage (row part; chunk added per step)
  int a_row[FM], b_row[FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) a_row[fm] = wm * (FM * 32) + fm * 32 + (lane & 31);
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) b_row[fn] = wn * (FN * 32) + fn * 32 + (lane & 31);

  // Pipeline: LDS stage kt & 1 holds step kt; register slot (j % S) holds the
  // loads of step j in flight, issued S steps before they are stored to LDS.
  gload(0, 0);
  lstore(0, 0);
#pragma unroll
  for (int j = 1; j <= S; ++j)
    if (j < nkt) gload(j, j % S);
  __syncthreads();
  for (int kt0 = 0; kt0 < nkt; kt0 += S) {
#pragma unroll
  for (int sub = 0; sub < S; ++sub) {
    const int kt = kt0 + sub;
    if (kt >= nkt) break;
    const int cur = kt & 1;
    // slot of step kt+1 (and of step kt+1+S, loaded after it is stored)
    const int nslot = (sub + 1) % S;
    const uint8_t* As = lds + cur * C::kStageBytes;
    const uint8_t* Bs = As + BM * BKB;
    // Fragments of sub-step kk+1 are read from LDS before the MFMAs of sub-step
    // kk are issued (two fragment sets live); the scheduling barriers keep the
    // compiler from hoisting every sub-step's reads to the top of the step.
    v8i a[2][FM], b[2][FN];
    auto read_frags = [&](int kk, v8i* af, v8i* bf) {
      const int c = kk * 2 + (lane >> 5);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int r = a_row[fm];
        const uint4 u = *reinterpret_cast<const uint4*>(As + r * BKB + (swz<CPR>(r, c) << 4));
        af[fm] = v8i{int(u.x), int(u.y), int(u.z), int(u.w), 0, 0, 0, 0};
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int r = b_row[fn];
        const uint4 u = *reinterpret_cast<const uint4*>(Bs + r * BKB + (swz<CPR>(r, c) << 4));
        bf[fn] = v8i{int(u.x), int(u.y), int(u.z), int(u.w), 0, 0, 0, 0};
      }
    };
    read_frags(0, a[0], b[0]);
#pragma unroll
    for (int kk = 0; kk < C::kSub; ++kk) {
      if (kk + 1 < C::kSub) read_frags(kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              a[kk & 1][fm], b[kk & 1][fn], acc[fm][fn], 4, 4, 0, 127, 0, 127);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kt + 1 < nkt) lstore(cur ^ 1, nslot);
    if (kt + 1 + S < nkt) gload(kt + 1 + S, nslot);
    __syncthreads();
  }
  }

  // ---- epilogue -------------------------------------------------------------
  // Scales are applied in the MFMA output layout: for accumulator element r,
  // lanes 0..31 hold 32 consecutive columns of one row and lanes 32..63 the
  // same columns four rows down. All row and column scales of the lane are
  // loaded before any is used.
  const int col_l = lane & 31;
  float sb[FN];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int gc = n0 + wn * (FN * 32) + fn * 32 + col_l;
    sb[fn] = (gc < N) ? sB[gc] : 0.0f;
  }
  float sa[FM][16];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int gr = m0 + wm * (FM * 32) + fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      sa[fm][r] = (gr < M) ? sA[gr] : 0.0f;
    }
  // Output through a wave-private LDS block (the stage buffers are free after
  // the main loop's last barrier): two 32x32 fragments at a time are written
  // in the MFMA layout, read back as rows and stored 16 bytes per lane.
  constexpr int kER = 72;  // padded row of a 32 x 64 chunk (floats)
  static_assert((NT / kWave) * 32 * kER * 4 <= 2 * C::kStageBytes,
                "epilogue chunks fit the stage buffers");
  static_assert(FN % 2 == 0, "fragments are staged in pairs");
  float* eb = reinterpret_cast<float*>(lds) + wave * (32 * kER);
  const bool y_vec = ((reinterpret_cast<uintptr_t>(Y) & 15) == 0) && ((ldy & 3) == 0);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fp = 0; fp < FN; fp += 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          eb[rl * kER + h * 32 + col_l] = __fmul_rn(__fmul_rn(acc[fm][fp + h][r], sa[fm][r]), sb[fp + h]);
        }
      const int row_base = m0 + wm * (FM * 32) + fm * 32;
      const int col_base = n0 + wn * (FN * 32) + fp * 32;
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int rl = it * 4 + (lane >> 4);
        const int cl = (lane & 15) * 4;
        const float4 v = *reinterpret_cast<const float4*>(eb + rl * kER + cl);
        const int gr = row_base + rl, gc = col_base + cl;
        if (gr < M) {
          float* dst = Y + int64_t(gr) * ldy + gc;
          if (y_vec && gc + 4 <= N) {
            __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(dst));
          } else {
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (gc + c < N) dst[c] = vv[c];
          }
        }
      }
    }
}

using GemmTile = GemmCfg<128, 256, 2, 2, 64, 2, 2>;

}  // namespace

hipError_t launch_fp4_gemm(const uint8_t* Aq, const float* sA, const uint8_t* Bq, const float* sB,
                           int64_t M, int64_t N, int64_t ldq, const SparseArgs& sp, float* Y,
                           int64_t ldy, hipStream_t stream) {
  using C = GemmTile;
  const int tiles_m = int((M + C::BM - 1) / C::BM);
  const int tiles_n = int((N + C::BN - 1) / C::BN);
  fp4_gemm_kernel<C><<<dim3(unsigned(tiles_m * tiles_n)), C::kThreads, 0, stream>>>(
      Aq, sA, Bq, sB, int(M), int(N), int(ldq), tiles_m, Y, ldy);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp.row_ptr == nullptr) return e;
  return launch_sparse_add(sp, M, N, Y, ldy, stream);
}

}  // namespace fp4lin
