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
// With the sparse compensation matrix dA (the outlier and compensation
// paragraphs: dA = A - A_clamped, non-zero only where A was clamped, its
// product with the unquantized weight added back), the same epilogue adds
//   s[i,j] = sum over row i's non-zeros, k ascending, of val * W[k,j]
// (fp32 fused multiply-add from 0) to each element of a row that has
// non-zeros, before Y's only store: Y = Y0 + s. The result is bit-identical to
// the scaled product followed by the separate compensation kernel (spmm.hip),
// without reading Y back.
//
// Micro-scaled variant (kMx; the micro-scaling lecture "FP4量化训练的硬件挑战：
// NVIDIA Blackwell架构上的微缩放格式（Micro-scaling）实现", section 3, with the E8M0
// block scales of the format survey "训练大型语言模型的挑战"): A and B carry one
// E8M0 byte per 32 codes along K (mx.hip), which the instruction takes as its
// per-lane block-scale operands in place of the unit scales, and the epilogue
// writes the accumulator as it is: Y[i,j] = sum over blocks of
// 2^(eA + eB) * (block's FP4 dot product), accumulated in fp32.
//
// Layout and schedule:
//  * A is M x ldq bytes and B is N x ldq bytes, K-contiguous packed rows.
//  * A workgroup of 8 waves (4 x 2 grid, each wave 64 x 128 outputs) owns a
//    256 x 256 output tile and walks K in 128-code (64-byte) steps through
//    three LDS stages of 32 KiB. Operand tiles go from global memory straight
//    into LDS (buffer loads with an LDS destination, no register staging),
//    issued three steps ahead into the stage the previous step finished.
//    Each step issues its first 64-code sub-step of MFMAs, then waits for its
//    own loads of the next stage and meets the other waves at the barrier
//    while the matrix core works through the queued MFMAs, then issues the
//    next loads, the second sub-step of MFMAs and the next step's first
//    fragment reads. One workgroup per CU, two waves per SIMD. (Against
//    128 x 256 tiles with two 4-wave workgroups per CU, each wave moves 4
//    instead of 6 KiB of operands per step for the same 16 MFMAs: 3-13%
//    faster on the LLaMA shapes.)
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
//  * With the compensation, the tile leaves in four chunks of 64 rows x all
//    256 columns (each wave row's 16 x 256 block in half a stage buffer).
//    After a barrier each wave finishes 8 whole rows of a chunk, one after the
//    other: a lane owns 4 consecutive columns, so a non-zero costs one 8-byte
//    (bf16 W) or 16-byte (fp32 W) gather per lane, addressed with the W row
//    offset in the scalar operand of a buffer load. A row's first 8 entries
//    (column, value) come in with one vector load by lanes 0..7 and reach the
//    wave through readlane; entries are loaded two rows ahead and gathered
//    one row ahead of the row being multiplied. Each row is stored once,
//    1 KiB per wave instruction.
#include <type_traits>

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

template <int BM_, int BN_, int WM_, int WN_, int BKB_, int MINB_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BKB = BKB_;
  static constexpr int kMinBlocks = MINB_;  // workgroups per CU the register budget targets
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int FM = BM / WM / 32;
  static constexpr int FN = BN / WN / 32;
  static constexpr int CPR = BKB / 16;            // 16-byte chunks per staged row
  static constexpr int kSub = BKB / 32;            // 64-code MFMA steps per K step
  static constexpr int kStageBytes = (BM + BN) * BKB;
  static_assert(FM >= 1 && FN >= 1, "tile too small for the wave grid");
  static_assert(CPR == 4 || CPR == 8, "swizzle assumes 64- or 128-byte staged rows");
};

// s_waitcnt immediate of gfx9-family parts: vmcnt in bits 3:0 (and 15:14),
// expcnt in 6:4 (7: do not wait), lgkmcnt in 11:8.
constexpr int waitcnt_vm_lgkm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

// Physical 16-byte chunk of logical chunk c in staged row r. A fragment read
// is a 128-bit LDS read of 32 consecutive rows at one logical chunk (lanes
// 32..63 at the next chunk). On gfx950 such a read takes 4 LDS cycles when
// every 16 consecutive lanes cover 64 distinct 4-byte banks, the rate of a
// contiguous 1 KiB read; measured on the device, the mapping below reaches
// it for 64-byte rows, while an unswizzled layout takes 16 cycles:
//   64-byte rows:  chunk ^ ((r >> 2) & 3)
//   128-byte rows: chunk ^ ((r ^ (r >> 3)) & 7)
template <int CPR>
__device__ inline int swz(int r, int c) {
  if constexpr (CPR == 4) return c ^ ((r >> 2) & 3);
  return c ^ ((r ^ (r >> 3)) & 7);
}

// Tiles of one launch: positions base .. base + nblocks / split - 1 of the
// order of a tiles_m x tiles_n grid, each cut into split tiles along M (split
// 2: the two 128-row halves of a 256-row tile).
struct TileMap {
  int base, tiles_m, tiles_n, split;
};

// Tile order: groups of G tile rows sweeping across N; each XCD takes a
// contiguous run of that order (a bijection from workgroup id to tile).
// kColumns: the tile columns one after another instead, each swept down M, so
// that the tiles an XCD runs together share one 256-column strip of the
// operands and of W (the compensation's gathers then stay in that XCD's L2).
template <bool kColumns = false>
__device__ inline void tile_coords(int bid, int nblocks, const TileMap& tmap, int& tm, int& tn) {
  const int xcd = bid & 7;
  const int idx = bid >> 3;
  const int base = nblocks >> 3, rem = nblocks & 7;
  const int t = xcd * base + (xcd < rem ? xcd : rem) + idx;
  if constexpr (kColumns) {
    tn = t / tmap.tiles_m;
    tm = t - tn * tmap.tiles_m;
    return;
  }
  const int u = tmap.base + t / tmap.split;  // position in the order
  const int half = t % tmap.split;
  const int tiles_m = tmap.tiles_m;
  constexpr int G = 4;
  const int per_group = G * tmap.tiles_n;
  const int grp = u / per_group;
  const int first_m = grp * G;
  const int gsize = (tiles_m - first_m) < G ? (tiles_m - first_m) : G;
  const int within = u - grp * per_group;
  tm = (first_m + within % gsize) * tmap.split + half;
  tn = within / gsize;
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// dst + 16 * l (dst wave-uniform).
__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t rs, uint8_t* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, voff,
                                           0, 0, 0);
}

// Workgroup barrier that the compiler may not move memory accesses across;
// the caller waits for the counters it needs first.
__device__ inline void raw_barrier() { asm volatile("s_barrier" ::: "memory"); }


// The weight operand of the fused epilogue's compensation. The COO arrays
// are separate __restrict__ kernel arguments, which lets the compiler read a
// wave's entries with scalar loads (Y's stores cannot alias them).
struct CompArgs {
  const void* W;           // K x N weight, bf16 or fp32, row stride ldw elements
  int ldw;
  int w_bytes;             // K * ldw * element size (< 2^31)
  int w_vec;               // W rows allow 4-column vector loads
};

// One compensation gather: this lane's 4 columns of W row k (bf16: 8 bytes,
// fp32: 16 bytes), the row offset k * ldw in the scalar operand and the
// column offsets in vo (byte offsets of the lane's columns, each clamped into
// [0, N) so that every address lies inside row k whatever the lane: the
// buffer range check does not cover the scalar offset). With vector access
// (W and its row stride aligned to 4 elements and N a multiple of 4, so a
// lane's 4 columns are all below N or all past it, and lanes past N read the
// row's last 4) one load moves the 4 columns, vo[0] being their start;
// otherwise the 4 elements are loaded one by one.
template <bool kBf16W>
struct WSeg {
  uint32_t d[kBf16W ? 2 : 4];
};

template <bool kBf16W, bool kVec>
__device__ inline WSeg<kBf16W> load_wseg(__amdgpu_buffer_rsrc_t rs, const int (&vo)[4], int soff) {
  WSeg<kBf16W> w;
  if constexpr (kBf16W) {
    if constexpr (kVec) {
      const auto u = __builtin_amdgcn_raw_buffer_load_b64(rs, vo[0], soff, 0);
      w.d[0] = u[0];
      w.d[1] = u[1];
    } else {
      const uint32_t h0 = __builtin_amdgcn_raw_buffer_load_b16(rs, vo[0], soff, 0);
      const uint32_t h1 = __builtin_amdgcn_raw_buffer_load_b16(rs, vo[1], soff, 0);
      const uint32_t h2 = __builtin_amdgcn_raw_buffer_load_b16(rs, vo[2], soff, 0);
      const uint32_t h3 = __builtin_amdgcn_raw_buffer_load_b16(rs, vo[3], soff, 0);
      w.d[0] = h0 | (h1 << 16);
      w.d[1] = h2 | (h3 << 16);
    }
  } else {
    if constexpr (kVec) {
      const auto u = __builtin_amdgcn_raw_buffer_load_b128(rs, vo[0], soff, 0);
      w.d[0] = u[0];
      w.d[1] = u[1];
      w.d[2] = u[2];
      w.d[3] = u[3];
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) w.d[c] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo[c], soff, 0);
    }
  }
  return w;
}

// s[c] = fma(v, W[k, col + c], s[c]) for the lane's 4 columns.
template <bool kBf16W>
__device__ inline void fma_wseg(float v, const WSeg<kBf16W>& w, float (&s)[4]) {
  if constexpr (kBf16W) {
    s[0] = fmaf(v, __uint_as_float(w.d[0] << 16), s[0]);
    s[1] = fmaf(v, __uint_as_float(w.d[0] & 0xffff0000u), s[1]);
    s[2] = fmaf(v, __uint_as_float(w.d[1] << 16), s[2]);
    s[3] = fmaf(v, __uint_as_float(w.d[1] & 0xffff0000u), s[3]);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) s[c] = fmaf(v, __uint_as_float(w.d[c]), s[c]);
  }
}

// Epilogue with the sparse compensation (see the header). The tile (BM x BN =
// 256 x 256, eight waves of 64 x 128 in a 4 x 2 grid) leaves in four chunks;
// chunk c holds the rows wm * 64 + (c >> 1) * 32 + (c & 1) * 16 + [0, 16) of
// all four wave rows wm, all 256 columns: wave row wm's 16 x 256 block is
// half (wm & 1) of stage wm >> 1 (with 128-row tiles of two wave rows, the
// whole of stage wm). Wave w then finishes the 8 rows
// (w & 1) * 8 + [0, 8) of wave row w >> 1's block. A block row is 256 floats
// (two blocks fill a stage); the 32-float halves of its 128-byte groups swap
// in rows with bit 2 set (lds_col), so that the lanes 32..63 of a staging
// write, four rows below lanes 0..31, hit the other 32 banks, while a row
// still reads back as 64 16-byte pieces.
template <class C, bool kMx, bool kBf16W, bool kWVec>
__device__ __attribute__((always_inline)) inline void fused_epilogue(
    v16f (&acc)[C::FM][C::FN], const float (&sa)[C::FM][16], const float (&sb)[C::FN],
    uint8_t* st0, uint8_t* st1, int wave, int wm, int wn, int lane, int m0, int n0, int M, int N,
    float* __restrict__ Y, int64_t ldy, const CompArgs& cp, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col, const float* __restrict__ val) {
  constexpr int FM = C::FM, FN = C::FN, BN = C::BN;
  static_assert(C::BM == 64 * C::WM && (C::WM == 2 || C::WM == 4) && BN == 256 && C::WN == 2 &&
                    FM == 2 && FN == 4,
                "chunk layout of the fused epilogue");
  constexpr int kPitch = BN;  // floats
  constexpr int kPerStage = C::WM / 2;  // 16-row blocks per stage buffer (wave rows / 2 stages)
  static_assert(kPerStage * 16 * kPitch * 4 <= C::kStageBytes, "the blocks fit two stages");
  // LDS column of column c in block row r
  auto lds_col = [](int r, int c) { return c ^ (((r >> 2) & 1) << 5); };
  // non-zeros per gather group (one group per row is in flight ahead)
  constexpr int G = 8;

  // scales applied once, in place (the accumulators are then the output)
  if constexpr (!kMx) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[fm][fn][r] = __fmul_rn(__fmul_rn(acc[fm][fn][r], sa[fm][r]), sb[fn]);
  }
  float* const wblk =
      reinterpret_cast<float*>(wm < kPerStage ? st0 : st1) + (wm % kPerStage) * 16 * kPitch;
  const int pr = wave >> 1, ph = wave & 1;
  const float* const rblk = reinterpret_cast<const float*>(pr < kPerStage ? st0 : st1) +
                            (pr % kPerStage) * 16 * kPitch + ph * 8 * kPitch;
  const int c4 = 4 * lane;
  const int gc = n0 + c4;
  constexpr int esz = kBf16W ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rsW =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(cp.W), 0, cp.w_bytes, kBufferFlags);
  const int row_bytes = cp.ldw * esz;
  // byte offsets of this lane's 4 columns inside a W row, clamped below N
  // (vector access: the 4-column group itself, the last one for lanes past N)
  int voffW[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int cc = kWVec ? (gc + 4 <= N ? gc : N - 4) + c : (gc + c < N ? gc + c : N - 1);
    voffW[c] = cc * esz;
  }
  // the whole tile width lies below N and Y takes 16-byte stores (uniform)
  const bool y_full = ((reinterpret_cast<uintptr_t>(Y) & 15) == 0) && ((ldy & 3) == 0) &&
                      n0 + BN <= N;
  // Row boundaries come through the constant address space as scalar loads
  // (the COO is read-only while the kernel runs). The entries themselves
  // (column, value) are read as buffers that return zero at or past nnz, a
  // group of G by lanes 0 .. G-1 of one vector load, and reach the wave as
  // scalars through readlane: the scalar unit, which a CU shares among its
  // waves, is left almost nothing to do per non-zero (with scalar entry
  // loads, bounds clamps, per-slot weight masks and a search of the row
  // boundaries it ran about 30 scalar instructions per non-zero and set the
  // pace of the whole epilogue).
  typedef const __attribute__((address_space(4))) int32_t cint32;
  cint32* const rp_c = (cint32*)row_ptr;
  // nnz <= capacity <= 10 M (this schedule's limit) and M < 2^25 (packed rows
  // of at least 64 bytes addressed with 32-bit offsets), so byte offsets of
  // entries fit 32 bits
  const int nnz = rp_c[M];
  const __amdgpu_buffer_rsrc_t rsCol =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(col), 0, nnz * 4, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsVal =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(val), 0, nnz * 4, kBufferFlags);
  // entries e0 .. e0+G-1: lane u < G gets entry e0 + u (zero past nnz)
  auto load_entries = [&](int e0, int& cv, float& vv) {
    const int voff = lane < G ? (e0 + lane) * 4 : nnz * 4;
    cv = __builtin_amdgcn_raw_buffer_load_b32(rsCol, voff, 0, 0);
    vv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsVal, voff, 0, 0));
  };
  // the G gathers of a group whose first n entries are the row's (n may
  // exceed G): slots past n take weight 0 (0 * w adds nothing, so the fp32
  // sum keeps its value) and read the W row of whatever entry they hold
  auto gather = [&](int cv, float vv, int n, WSeg<kBf16W> (&w)[G], float (&wt)[G]) {
    const int offv = cv * row_bytes;  // < K * ldw * element size < 2^31
    const float vm = lane < n ? vv : 0.0f;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int so = __builtin_amdgcn_readlane(offv, u);
      wt[u] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(vm), u));
      w[u] = load_wseg<kBf16W, kWVec>(rsW, voffW, so);
    }
  };

  // Rows g0 .. g0+7 of the chunk just staged (their LDS rows at rblk, which
  // only this wave touches until the next barrier), one row after the other
  // in compile-time order. A row's first G non-zeros are one group; its
  // entries are loaded two rows ahead and its gathers one row ahead, so the
  // gathers of row j+1 are in flight while row j is multiplied. The rare
  // longer rows take their further groups one at a time after the first.
  // Every row, empty or not, issues the same loads, so the counter waits the
  // compiler places stay exact; then Y0 + s goes into the row's LDS row. No
  // store is issued in the loop: the 8 rows leave for Y after it.
  auto finish_rows = [&](int g0) {
    float* const rows = const_cast<float*>(rblk);
    // the 9 row boundaries (rows past M have no entries)
    int rp[9];
#pragma unroll
    for (int j = 0; j < 9; ++j) rp[j] = rp_c[g0 + j < M ? g0 + j : M];
    if (rp[0] < rp[8]) {
      int ce[2];
      float ve[2];
      WSeg<kBf16W> wq[2][G];
      float wt[2][G];
      load_entries(rp[0], ce[0], ve[0]);
      load_entries(rp[1], ce[1], ve[1]);
      gather(ce[0], ve[0], rp[1] - rp[0], wq[0], wt[0]);
      auto row = [&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        if constexpr (j + 2 <= 7) load_entries(rp[j + 2], ce[j & 1], ve[j & 1]);
        if constexpr (j + 1 <= 7)
          gather(ce[(j + 1) & 1], ve[(j + 1) & 1], rp[j + 2] - rp[j + 1], wq[(j + 1) & 1],
                 wt[(j + 1) & 1]);
        float acc4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < G; ++u) fma_wseg<kBf16W>(wt[j & 1][u], wq[j & 1][u], acc4);
        // further groups of a row of more than G non-zeros
        for (int e0 = rp[j] + G; e0 < rp[j + 1]; e0 += G) {
          int cv;
          float vv;
          load_entries(e0, cv, vv);
          WSeg<kBf16W> w[G];
          float t[G];
          gather(cv, vv, rp[j + 1] - e0, w, t);
#pragma unroll
          for (int u = 0; u < G; ++u) fma_wseg<kBf16W>(t[u], w[u], acc4);
        }
        if (rp[j + 1] > rp[j]) {
          float* const p = rows + j * kPitch + lds_col(j, c4);
          f32x4 y = *reinterpret_cast<const f32x4*>(p);
          y[0] = __fadd_rn(y[0], acc4[0]);
          y[1] = __fadd_rn(y[1], acc4[1]);
          y[2] = __fadd_rn(y[2], acc4[2]);
          y[3] = __fadd_rn(y[3], acc4[3]);
          *reinterpret_cast<f32x4*>(p) = y;
        }
      };
      row(std::integral_constant<int, 0>{});
      row(std::integral_constant<int, 1>{});
      row(std::integral_constant<int, 2>{});
      row(std::integral_constant<int, 3>{});
      row(std::integral_constant<int, 4>{});
      row(std::integral_constant<int, 5>{});
      row(std::integral_constant<int, 6>{});
      row(std::integral_constant<int, 7>{});
    }
    // the 8 rows, Y0 + s (rows without non-zeros: Y0 as it is), to Y
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int gr = g0 + i;
      const f32x4 y = *reinterpret_cast<const f32x4*>(rows + i * kPitch + lds_col(i, c4));
      if (gr < M) {
        float* dst = Y + int64_t(gr) * ldy + gc;
        if (y_full) {
          __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(dst));
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (gc + c < N) dst[c] = y[c];
        }
      }
    }
  };

  // acc element r of fragment row fm holds row 8 * (r >> 2) + 4 * (lane >> 5)
  // + (r & 3) of the fragment: elements h * 8 .. h * 8 + 7 are its rows
  // h * 16 + [0, 16)
  auto stage_chunk = [&](auto fm_c, auto h_c) {
    constexpr int fm = decltype(fm_c)::value, h = decltype(h_c)::value;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int rl = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
        wblk[rl * kPitch + lds_col(rl, wn * (FN * 32) + fn * 32 + (lane & 31))] =
            acc[fm][fn][h * 8 + rr];
      }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
#pragma nounroll
  for (int c = 0; c < 4; ++c) {
    switch (c) {
      case 0: stage_chunk(I0{}, I0{}); break;
      case 1: stage_chunk(I0{}, I1{}); break;
      case 2: stage_chunk(I1{}, I0{}); break;
      default: stage_chunk(I1{}, I1{}); break;
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(63, 0));
    raw_barrier();
    finish_rows(m0 + pr * 64 + (c >> 1) * 32 + (c & 1) * 16 + ph * 8);
    // every wave's LDS reads of this chunk are done before the next is staged
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(63, 0));
    raw_barrier();
  }
}

// Tile order of the kernels with the fused compensation (see tile_coords).
constexpr bool kFusedColumns = true;

// Largest COO capacity per row of A for which the compensation runs in the
// GEMM's epilogue (see run_gemm).
constexpr int64_t kFusedMaxPerRow = 10;

// kComp: 0 no compensation; with it, 1 + (W is float32) + 2 * (W rows allow
// 4-column vector gathers): 1 / 3 bfloat16 W, 2 / 4 float32 W.
template <class C, bool kMx, int kComp>
__global__ __launch_bounds__(C::kThreads, C::kMinBlocks) void fp4_gemm_kernel(
    const uint8_t* __restrict__ Aq, const float* __restrict__ sA,
    const uint8_t* __restrict__ Bq, const float* __restrict__ sB, int M, int N, int ldq,
    TileMap tmap, float* __restrict__ Y, int64_t ldy, const uint8_t* __restrict__ As,
    const uint8_t* __restrict__ Bs, CompArgs cp, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col, const float* __restrict__ val) {
  constexpr int BM = C::BM, BN = C::BN, WN = C::WN, BKB = C::BKB, CPR = C::CPR;
  constexpr int FM = C::FM, FN = C::FN, NT = C::kThreads;
  constexpr int SB = C::kStageBytes;
  // Three LDS stages, separate objects so that the compiler can tell the
  // direct-to-LDS loads into one stage from the fragment reads of another.
  __shared__ __attribute__((aligned(16))) uint8_t st0[SB];
  __shared__ __attribute__((aligned(16))) uint8_t st1[SB];
  __shared__ __attribute__((aligned(16))) uint8_t st2[SB];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  int tm, tn;
  tile_coords<(kComp != 0) && kFusedColumns>(blockIdx.x, gridDim.x, tmap, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nkt = (ldq + BKB - 1) / BKB;

  // Operand tiles go straight from global memory to LDS (buffer loads with
  // the LDS destination): one instruction moves 1 KiB, lane l landing at byte
  // 16*l of the block, so the XOR swizzle is applied to the source address.
  // The resource holds the packed matrix size, so rows past M (or N) read as
  // zero codes. A stage is (BM + BN) rows of BKB bytes in 1 KiB blocks (A rows
  // first); wave w moves blocks w, w + W, w + 2W, ...
  static_assert(BKB == 64, "one 1 KiB block is 16 rows of 64 bytes");
  constexpr int kBlocks = SB / 1024;
  constexpr int kWaves = NT / kWave;
  constexpr int kPer = kBlocks / kWaves;
  static_assert(kBlocks % kWaves == 0 && BM % 16 == 0, "even block split");
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(Aq), 0, int(int64_t(M) * ldq), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsB =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(Bq), 0, int(int64_t(N) * ldq), kBufferFlags);
  int src_off[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int b = wave + j * kWaves;
    const bool is_a = b < BM / 16;
    const int r = (is_a ? b * 16 : (b - BM / 16) * 16) + (lane >> 2);
    const int c = (lane & 3) ^ (swz<CPR>(r, 0));  // logical chunk stored at physical lane & 3
    if (is_a)
      src_off[j] = (m0 + r < M) ? (m0 + r) * ldq + c * 16 : int(int64_t(M) * ldq);
    else
      src_off[j] = (n0 + r < N) ? (n0 + r) * ldq + c * 16 : int(int64_t(N) * ldq);
  }
  auto dma = [&](int kt, uint8_t* stage) {
    const int kb = kt * BKB;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int b = wave + j * kWaves;
      load_lds16(b < BM / 16 ? rsA : rsB, stage + b * 1024, src_off[j] + kb);
    }
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

  int a_row[FM], b_row[FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) a_row[fm] = wm * (FM * 32) + fm * 32 + (lane & 31);
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) b_row[fn] = wn * (FN * 32) + fn * 32 + (lane & 31);

  static_assert(C::kSub == 2, "two 64-code MFMA sub-steps per K step");
  // fragments of one sub-step (kk) of a stage
  auto read_frags = [&](const uint8_t* As, int kk, v8i* af, v8i* bf) {
    const uint8_t* Bs = As + BM * BKB;
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
  // Block scales (kMx), stored step-major: for K step kt (128 codes, blocks
  // 4kt .. 4kt+3) each row has one 32-bit word at 4 * (kt * rows + row), so
  // the 32 rows of a fragment read 128 contiguous bytes. Lane half h supplies
  // codes 32h .. 32h+31 of each 64-code sub-step, i.e. block 4kt + 2kk + h in
  // sub-step kk: the word shifted right by 8h, byte kk*2 of it picked by the
  // instruction's op_sel. Rows past M (N) take the scales of the last row:
  // their codes are zero, so any finite scale gives zero. One load serves two
  // fragments (A's two, then B's in pairs): lanes 0..31 read the rows of the
  // first, lanes 32..63 those of the second (64 consecutive rows, 256
  // contiguous bytes), and a lane-half swap (v_permlane32_swap) then gives
  // every lane its row's word of both. The raw words of step kt go into slot
  // kt mod 3 of a register ring, loaded three steps ahead.
  constexpr int NS = kMx ? FM + FN : 0;  // scale words per step (one per fragment)
  constexpr int NL = NS / 2;             // scale loads per step
  static_assert(!kMx || (FM % 2 == 0 && FN % 2 == 0), "fragments pair up");
  const int nblk = ldq / 16;
  const __amdgpu_buffer_rsrc_t rsSA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(As), 0, kMx ? M * nblk : 0, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsSB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Bs), 0, kMx ? N * nblk : 0, kBufferFlags);
  int sc_off[NL > 0 ? NL : 1];
  if constexpr (kMx) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int f = 2 * j + (lane >> 5);  // this lane's fragment of load j
      const int row = f < FM ? m0 + a_row[f] : n0 + b_row[f - FM];
      const int lim = f < FM ? M : N;
      sc_off[j] = 4 * (row < lim ? row : lim - 1);
    }
  }
  const int hshift = (lane >> 5) * 8;
  uint32_t sc0[NL > 0 ? NL : 1], sc1[NL > 0 ? NL : 1], sc2[NL > 0 ? NL : 1];
  // The manual vmcnt waits below count the stage loads and these in issue
  // order; scheduling barriers keep every group where it is written.
  auto load_scales = [&](int kt, uint32_t* dst) {
    if constexpr (kMx) {
#pragma unroll
      for (int j = 0; j < NL; ++j)
        dst[j] = __builtin_amdgcn_raw_buffer_load_b32(2 * j < FM ? rsSA : rsSB,
                                                      sc_off[j] + kt * 4 * (2 * j < FM ? M : N), 0, 0);
    }
  };
  // one scale word per fragment from the raw words of a step, shifted to the
  // lane half's block
  auto expand = [&](const uint32_t* raw, uint32_t* w) {
    if constexpr (kMx) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const auto sw = __builtin_amdgcn_permlane32_swap(raw[j], raw[j], false, false);
        w[2 * j] = uint32_t(sw[0]) >> hshift;
        w[2 * j + 1] = uint32_t(sw[1]) >> hshift;
      }
    }
  };
  // kk_c: the sub-step (0 or 1) as a type, so that op_sel is a constant
  auto mfmas = [&](auto kk_c, const v8i* af, const v8i* bf, const uint32_t* sc) {
    constexpr int KK = decltype(kk_c)::value;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        if constexpr (kMx)
          acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[fm], bf[fn], acc[fm][fn], 4, 4, 2 * KK, int(sc[fm]), 2 * KK, int(sc[FM + fn]));
        else
          acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[fm], bf[fn], acc[fm][fn],
                                                                        4, 4, 0, 127, 0, 127);
      }
  };
  using Sub0 = std::integral_constant<int, 0>;
  using Sub1 = std::integral_constant<int, 1>;

  // Pipeline over K steps (stage of step s: s mod 3). On entry to step kt the
  // first sub-step's fragments of stage kt are in registers. The step reads
  // its second sub-step's fragments, issues the first sub-step's MFMAs, then
  // waits for its own loads of stage kt+1 (those of kt+2 stay in flight) and
  // for its fragment reads, and meets the other waves at a barrier while the
  // matrix core works through the queued MFMAs. After the barrier stage kt+1
  // is complete and nobody reads stage kt any more, so the loads of step kt+3
  // go there; then the second sub-step's MFMAs and the next step's first
  // fragment reads. Every wave issues kPer loads per step on every path
  // (past the last step they repeat it into a stage that is not read).
  // With block scales, each step also issues the NL scale loads of step kt+3
  // after its second sub-step; a step's wait then leaves that step's and the
  // previous step's scale loads in flight besides the stage of kt+2.
  constexpr int kWaitCnt = waitcnt_vm_lgkm(kPer + 2 * NL, 0);
  static_assert(2 * kPer + 2 * NL < 64, "vmcnt immediate");
  v8i a0[FM], b0[FN], a1[FM], b1[FN];
  // a full step inside the main loop (steps kt, kt+1 and kt+2 all exist);
  // sc holds the raw scale words of step kt and is refilled for step kt+3
  uint32_t scw[NS > 0 ? NS : 1];
  auto step = [&](int kt, const uint8_t* cur, const uint8_t* nxt, uint8_t* ldst, uint32_t* sc) {
    read_frags(cur, 1, a1, b1);
    expand(sc, scw);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(Sub0{}, a0, b0, scw);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitCnt);
    raw_barrier();
    __builtin_amdgcn_sched_barrier(0);
    dma(kt + 3 < nkt ? kt + 3 : nkt - 1, ldst);
    mfmas(Sub1{}, a1, b1, scw);
    __builtin_amdgcn_sched_barrier(0);
    load_scales(kt + 3 < nkt ? kt + 3 : nkt - 1, sc);
    read_frags(nxt, 0, a0, b0);
  };
  // one of the last (up to two) steps: no more loads are issued
  auto tail_step = [&](const uint8_t* cur, const uint8_t* nxt, bool has_next, const uint32_t* sc) {
    read_frags(cur, 1, a1, b1);
    expand(sc, scw);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(Sub0{}, a0, b0, scw);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(0, 0));
    raw_barrier();
    __builtin_amdgcn_sched_barrier(0);
    mfmas(Sub1{}, a1, b1, scw);
    __builtin_amdgcn_sched_barrier(0);
    if (has_next) read_frags(nxt, 0, a0, b0);
  };
  dma(0, st0);
  load_scales(0, sc0);
  __builtin_amdgcn_sched_barrier(0);
  dma(nkt > 1 ? 1 : nkt - 1, st1);
  load_scales(nkt > 1 ? 1 : nkt - 1, sc1);
  __builtin_amdgcn_sched_barrier(0);
  dma(nkt > 2 ? 2 : nkt - 1, st2);
  load_scales(nkt > 2 ? 2 : nkt - 1, sc2);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(2 * kPer + 2 * NL, 0));  // step 0 landed
  raw_barrier();
  read_frags(st0, 0, a0, b0);
  int kt0 = 0;
  for (; kt0 + 3 <= nkt; kt0 += 3) {
    step(kt0, st0, st1, st0, sc0);
    step(kt0 + 1, st1, st2, st1, sc1);
    step(kt0 + 2, st2, st0, st2, sc2);
  }
  if (kt0 < nkt) tail_step(st0, st1, kt0 + 1 < nkt, sc0);
  if (kt0 + 1 < nkt) tail_step(st1, st2, false, sc1);
  // every load has landed and every wave is done with the stages before they
  // are reused for the output
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(0, 0));
  raw_barrier();

  // ---- epilogue -------------------------------------------------------------
  // Scales are applied in the MFMA output layout: for accumulator element r,
  // lanes 0..31 hold 32 consecutive columns of one row and lanes 32..63 the
  // same columns four rows down. All row and column scales of the lane are
  // loaded before any is used.
  // (With block scales the accumulator is the output and no scale is loaded.)
  const int col_l = lane & 31;
  float sb[FN];
  float sa[FM][16];
  if constexpr (!kMx) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int gc = n0 + wn * (FN * 32) + fn * 32 + col_l;
      sb[fn] = (gc < N) ? sB[gc] : 0.0f;
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gr = m0 + wm * (FM * 32) + fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        sa[fm][r] = (gr < M) ? sA[gr] : 0.0f;
      }
  }
  if constexpr (kComp != 0) {
    fused_epilogue<C, kMx, (kComp & 1) != 0, kComp >= 3>(acc, sa, sb, st0, st1, wave, wm, wn,
                                                          lane, m0, n0, M, N, Y, ldy, cp,
                                                          row_ptr, col, val);
    return;
  }
  // Output through a wave-private LDS block (the stage buffers are free after
  // the main loop's last barrier): two 32x32 fragments at a time are written
  // in the MFMA layout, read back as rows and stored 16 bytes per lane.
  constexpr int kER = 72;  // padded row of a 32 x 64 chunk (floats)
  // each stage buffer holds the blocks of kEpiPer waves
  constexpr int kEpiPer = C::kStageBytes / (32 * kER * 4);
  static_assert(kEpiPer >= 1 && 3 * kEpiPer >= NT / kWave, "epilogue blocks fit the stages");
  static_assert(FN % 2 == 0, "fragments are staged in pairs");
  uint8_t* const ebs = wave < kEpiPer ? st0 : (wave < 2 * kEpiPer ? st1 : st2);
  float* eb = reinterpret_cast<float*>(ebs) + (wave % kEpiPer) * (32 * kER);
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
          eb[rl * kER + h * 32 + col_l] =
              kMx ? acc[fm][fp + h][r] : __fmul_rn(__fmul_rn(acc[fm][fp + h][r], sa[fm][r]), sb[fp + h]);
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

// Tiles of the GEMM without compensation: 256 x 256 (eight waves, one
// workgroup per CU) once the grid fills the 256 CUs twice, 128 x 256 (four
// waves, two workgroups per CU) below that, where finer tiles balance better
// (LLaMA 1.3B up, 352 large tiles: 45.6 against 41.6 us).
using GemmTile = GemmCfg<256, 256, 4, 2, 64, 1>;
using GemmSmallTile = GemmCfg<128, 256, 2, 2, 64, 2>;
constexpr int kLargeTilesMin = 512;
constexpr int kCUs = 256;  // MI355X
// Tile of the GEMM with the compensation in its epilogue: the two workgroups
// on a CU keep the matrix core busy in turn while either one gathers (13B up:
// 509 against 521 us with 256 x 256 tiles).
using GemmFusedTile = GemmCfg<128, 256, 2, 2, 64, 2>;

// The GEMM without compensation over positions base .. base + count - 1 of
// the order of a tiles_m x tiles_n grid of 256 x 256 tiles (C: those tiles,
// or with 128-row C their two halves).
template <class C, bool kMx>
hipError_t launch_plain(const uint8_t* Aq, const float* sA, const uint8_t* Bq, const float* sB,
                        const uint8_t* As, const uint8_t* Bs, int64_t M, int64_t N, int64_t ldq,
                        float* Y, int64_t ldy, const TileMap& tmap, int count,
                        hipStream_t stream) {
  fp4_gemm_kernel<C, kMx, 0><<<dim3(unsigned(count * tmap.split)), C::kThreads, 0, stream>>>(
      Aq, sA, Bq, sB, int(M), int(N), int(ldq), tmap, Y, ldy, As, Bs, CompArgs{nullptr, 0, 0, 0},
      nullptr, nullptr, nullptr);
  return hipGetLastError();
}

template <bool kMx>
hipError_t run_gemm(const uint8_t* Aq, const float* sA, const uint8_t* Bq, const float* sB,
                    const uint8_t* As, const uint8_t* Bs, int64_t M, int64_t N, int64_t ldq,
                    const SparseArgs& sp, float* Y, int64_t ldy, hipStream_t stream) {
  // K steps are whole 64-byte chunks of the packed rows (the packed row length
  // is a multiple of 64 bytes), so no step reads past a row.
  static_assert(GemmTile::BKB == 64 && GemmSmallTile::BKB == 64 && GemmFusedTile::BKB == 64,
                "one K step per 64 bytes");
  if (ldq % 64 != 0) return hipErrorInvalidValue;
  // The two schedules of the compensation give the same bits. The fused
  // epilogue saves the read-modify-write of Y (8 bytes per output), but its
  // gathers run in the GEMM's waves (two per SIMD), which hide memory latency
  // worse than the separate kernel's eight, and it needs the 128 x 256 tile.
  // Measured on the LLaMA-shaped workloads (GEMM with compensation, us,
  // fused against the large-tile GEMM + separate kernel): 13B up 5.1/row
  // 437-459 against 295 + 215; 13B down 13.8/row 384 against 364; 1.3B up
  // 20/row 144 against 112; 7B up 41/row 948 against 656. The COO's capacity
  // bounds the non-zeros (for the select's own COO it is M*K*(1-q)).
  const bool fused = sp.row_ptr != nullptr && sp.capacity <= kFusedMaxPerRow * M;
  if (!fused) {
    static_assert(GemmTile::BM == 2 * GemmSmallTile::BM && GemmTile::BN == GemmSmallTile::BN,
                  "a large tile is two small ones");
    const int tiles_m = int((M + GemmTile::BM - 1) / GemmTile::BM);
    const int tiles_n = int((N + GemmTile::BN - 1) / GemmTile::BN);
    const int large = tiles_m * tiles_n;
    hipError_t e;
    if (large >= kLargeTilesMin) {
      // whole rounds of large tiles (one per CU), then, when at most half a
      // round is left, the rest of the order as 128-row halves, two
      // workgroups per CU: a last round of large tiles would leave most CUs
      // idle (7B, 96 left: 231 against 222 us; 13B down, 128 left: 279
      // against 264), while a fuller one runs better as large tiles (13B up,
      // 192 left: 293 against 300)
      const int rest = large % kCUs;
      const int whole = rest <= kCUs / 2 ? large - rest : large;
      e = launch_plain<GemmTile, kMx>(Aq, sA, Bq, sB, As, Bs, M, N, ldq, Y, ldy,
                                      TileMap{0, tiles_m, tiles_n, 1}, whole, stream);
      if (e == hipSuccess && whole < large)
        e = launch_plain<GemmSmallTile, kMx>(Aq, sA, Bq, sB, As, Bs, M, N, ldq, Y, ldy,
                                             TileMap{whole, tiles_m, tiles_n, 2}, large - whole,
                                             stream);
    } else {
      e = launch_plain<GemmSmallTile, kMx>(Aq, sA, Bq, sB, As, Bs, M, N, ldq, Y, ldy,
                                           TileMap{0, tiles_m, tiles_n, 2}, large, stream);
    }
    if (e != hipSuccess || sp.row_ptr == nullptr) return e;
    return launch_sparse_add(sp, M, N, Y, ldy, stream);
  }
  CompArgs cp{nullptr, 0, 0, 0};
  using CF = GemmFusedTile;
  const int tiles_mf = int((M + CF::BM - 1) / CF::BM);
  const int tiles_nf = int((N + CF::BN - 1) / CF::BN);
  const int64_t esz = sp.w_bf16 ? 2 : 4;
  // 4-column vector gathers need every W row start aligned to 4 elements
  // (8 bytes for bf16, 16 for fp32) and N a multiple of 4 (no lane straddles N)
  const bool w_vec = (reinterpret_cast<uintptr_t>(sp.W) % (4 * esz) == 0) && (sp.ldw % 4 == 0) &&
                     (N % 4 == 0);
  cp = CompArgs{sp.W, int(sp.ldw), int(sp.w_rows * sp.ldw * esz), w_vec ? 1 : 0};
  const int mode = (sp.w_bf16 ? 1 : 2) + (w_vec ? 2 : 0);
#define FP4LIN_GEMM_COMP(MODE)                                                                  \
  case MODE:                                                                                    \
    fp4_gemm_kernel<CF, kMx, MODE><<<dim3(unsigned(tiles_mf * tiles_nf)), CF::kThreads, 0,      \
                                     stream>>>(                                                 \
        Aq, sA, Bq, sB, int(M), int(N), int(ldq), TileMap{0, tiles_mf, tiles_nf, 1}, Y, ldy, As, \
        Bs, cp, sp.row_ptr,                                                                     \
        sp.col, sp.val);                                                                        \
    break;
  switch (mode) {
    FP4LIN_GEMM_COMP(1)
    FP4LIN_GEMM_COMP(2)
    FP4LIN_GEMM_COMP(3)
    FP4LIN_GEMM_COMP(4)
    default: return hipErrorInvalidValue;
  }
#undef FP4LIN_GEMM_COMP
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp4_gemm(const uint8_t* Aq, const float* sA, const uint8_t* Bq, const float* sB,
                           int64_t M, int64_t N, int64_t ldq, const SparseArgs& sp, float* Y,
                           int64_t ldy, hipStream_t stream) {
  return run_gemm<false>(Aq, sA, Bq, sB, nullptr, nullptr, M, N, ldq, sp, Y, ldy, stream);
}

hipError_t launch_fp4_gemm_mx(const uint8_t* Aq, const uint8_t* As, const uint8_t* Bq,
                              const uint8_t* Bs, int64_t M, int64_t N, int64_t ldq,
                              const SparseArgs& sp, float* Y, int64_t ldy, hipStream_t stream) {
  return run_gemm<true>(Aq, nullptr, Bq, nullptr, As, Bs, M, N, ldq, sp, Y, ldy, stream);
}

}  // namespace fp4lin
