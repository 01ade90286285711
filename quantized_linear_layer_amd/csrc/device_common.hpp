// Device helpers shared by the fp4lin kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4lin {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element access. Inputs are float32 or bfloat16 (raw uint16 bits).
// ---------------------------------------------------------------------------
struct F32In {
  using T = float;
  static constexpr int kBytes = 4;
  __device__ static inline uint32_t bits(T v) { return __float_as_uint(v); }
  __device__ static inline float widen(T v) { return v; }
  // |a| as an order-preserving integer key (finite inputs).
  __device__ static inline uint32_t key(T v) { return __float_as_uint(v) & 0x7fffffffu; }
  __device__ static inline float key_to_float(uint32_t k) { return __uint_as_float(k); }
  __device__ static inline uint32_t sign_bit(T v) { return __float_as_uint(v) >> 31; }
};

struct BF16In {
  using T = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static inline uint32_t bits(T v) { return v; }
  __device__ static inline float widen(T v) { return __uint_as_float(uint32_t(v) << 16); }
  __device__ static inline uint32_t key(T v) { return uint32_t(v) & 0x7fffu; }
  __device__ static inline float key_to_float(uint32_t k) { return __uint_as_float(k << 16); }
  __device__ static inline uint32_t sign_bit(T v) { return uint32_t(v) >> 15; }
};

// Operand bytes above which a kernel streams its single-use data with the
// non-temporal hint: most of the 256 MB last-level cache (MI355X), so that
// below it everything a layer reads stays cached from one kernel to the next.
constexpr int64_t kStreamBytes = int64_t(192) << 20;

// One 16-byte load. kStream sets the non-temporal hint: a stream that is
// read once per pass and is too large to stay in the last-level cache between
// passes then does not evict the data that does stay there.
template <bool kStream>
__device__ inline uint4 load16(const void* p) {
  if constexpr (kStream) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
  } else {
    return *static_cast<const uint4*>(p);
  }
}

// Eight consecutive elements, loaded with one 16-byte (fp32: two 16-byte)
// access when the caller has established alignment, else one by one.
template <class In>
struct Vec8 {
  typename In::T v[8];
};

template <class In, bool kAligned, bool kStream = false>
__device__ inline void load8(const typename In::T* __restrict__ p, int64_t valid,
                             Vec8<In>& out) {
  if (kAligned && valid >= 8) {
    if constexpr (In::kBytes == 2) {
      uint4 u = load16<kStream>(p);
      out.v[0] = uint16_t(u.x); out.v[1] = uint16_t(u.x >> 16);
      out.v[2] = uint16_t(u.y); out.v[3] = uint16_t(u.y >> 16);
      out.v[4] = uint16_t(u.z); out.v[5] = uint16_t(u.z >> 16);
      out.v[6] = uint16_t(u.w); out.v[7] = uint16_t(u.w >> 16);
    } else {
      const uint4 a = load16<kStream>(p), b = load16<kStream>(p + 4);
      out.v[0] = __uint_as_float(a.x); out.v[1] = __uint_as_float(a.y);
      out.v[2] = __uint_as_float(a.z); out.v[3] = __uint_as_float(a.w);
      out.v[4] = __uint_as_float(b.x); out.v[5] = __uint_as_float(b.y);
      out.v[6] = __uint_as_float(b.z); out.v[7] = __uint_as_float(b.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) out.v[i] = (i < valid) ? p[i] : typename In::T(0);
  }
}

// Chunk c (elements c .. c+7) of a row of K elements, zero where it lies past
// K. kFast: the row is 16-byte aligned and K % 8 == 0, so a chunk is either
// wholly inside the row or wholly outside; the load address is clamped into
// the row so that the vector load is unconditional and several of them can be
// in flight before the first is used. Otherwise elements are loaded one by one.
template <class In, bool kFast, bool kStream = false>
__device__ inline void load_chunk(const typename In::T* __restrict__ row, int64_t c, int64_t K,
                                  Vec8<In>& v) {
  if constexpr (kFast) {
    load8<In, true, kStream>(row + (c < K ? c : K - 8), 8, v);
    if (c >= K) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v.v[i] = typename In::T(0);
    }
  } else {
    load8<In, false>(row + c, K - c, v);
  }
}

// Row streaming, one wave per row: a row is read in slabs of CH chunks per
// lane, chunk j of lane l starting at column c0 + (j * 64 + l) * 8, so each j
// is one coalesced 64-lane sweep and all CH loads of a slab are issued before
// the first is used. Reductions over the row stay inside the wave.
template <class In, bool kFast, int CH, bool kStream = false>
__device__ inline void load_wave_slab(const typename In::T* __restrict__ row, int64_t c0,
                                      int64_t K, Vec8<In> (&v)[CH]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int j = 0; j < CH; ++j)
    load_chunk<In, kFast, kStream>(row, c0 + (int64_t(j) * kWave + lane) * 8, K, v[j]);
}

// Chunks per lane that cover `cols` columns in one slab, capped at kMax.
__host__ inline int chunks_per_lane(int64_t cols, int kMax) {
  int ch = 1;
  while (ch < kMax && int64_t(ch) * kWave * 8 < cols) ch *= 2;
  return ch;
}

// Workgroups of the one-wave-per-row kernels: 4 waves each, striding over
// rows. A wave takes about kRowsPerWave rows, so that the waves sharing a SIMD
// drift apart and one wave's loads overlap another's arithmetic (with one row
// per wave every wave loads, then every wave computes).
constexpr int kRowWaves = 4;
constexpr int kRowsPerWave = 1;
__host__ inline unsigned row_blocks(int64_t M) {
  const int64_t b = (M + kRowWaves * kRowsPerWave - 1) / (kRowWaves * kRowsPerWave);
  return unsigned(b < (int64_t(1) << 20) ? b : (int64_t(1) << 20));
}

// ---------------------------------------------------------------------------
// E2M1 encoding (round to nearest, ties away from zero, saturating at 6).
//
// The magnitude index of y >= 0 is the number of midpoints
// {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5} that y reaches. Multiplying by 4 (exact)
// turns the midpoints into the integers {1, 3, 5, 7, 10, 14, 20}, so
// "y >= t" is "floor(4y) >= 4t" and the index is a table lookup on
// n = min(floor(4y), 20). The 21 three-bit entries live in one 64-bit constant.
// v_cvt_u32_f32 truncates, saturates large values and +Inf to 0xffffffff and
// turns NaN (0 * Inf when a vector's amax is 0) into 0, which the lookup maps
// to magnitude 0, exactly as the threshold count does.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr uint64_t e2m1_lut() {
  uint64_t lut = 0;
  for (int n = 0; n <= 20; ++n) {
    int idx = (n >= 1) + (n >= 3) + (n >= 5) + (n >= 7) + (n >= 10) + (n >= 14) + (n >= 20);
    lut |= uint64_t(idx) << (3 * n);
  }
  return lut;
}

__device__ inline uint32_t cvt_u32_sat(float x) {
  uint32_t r;
  asm("v_cvt_u32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// Magnitude index of y = RN32(ax * inv).
__device__ inline uint32_t e2m1_magnitude(float ax, float inv) {
  float y = __fmul_rn(ax, inv);
  float y4 = __fmul_rn(y, 4.0f);
  uint32_t n = cvt_u32_sat(y4);
  n = n < 20u ? n : 20u;
  return uint32_t(e2m1_lut() >> (3u * n)) & 7u;
}

// Per-vector scale and encode multiplier from the vector's amax:
// s = RN32(amax/6), inv = RN32(6/amax). The quotients are formed in double and
// rounded once to float; double has more than 2*24+2 bits, so the result is
// the correctly rounded float quotient.
__device__ inline void vector_scale(float amax, float& s, float& inv) {
  double a = double(amax);
  s = float(a / 6.0);
  inv = float(6.0 / a);
}

// ---------------------------------------------------------------------------
// Wave reductions.
// ---------------------------------------------------------------------------
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ inline uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Exclusive prefix sum across the wave.
__device__ inline uint32_t wave_exclusive_scan(uint32_t v, uint32_t& total) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  total = __shfl(x, kWave - 1, kWave);
  return x - v;
}

// ---------------------------------------------------------------------------
// Token-wise quantization of one bfloat16 row held in registers as raw 16-byte
// words (16-byte aligned rows with K % 8 == 0 that fit one slab). The row amax
// is a packed 16-bit integer max of the magnitude bits (finite bfloat16 magnitudes
// order like their bits), and two codes are encoded per 32-bit word. When
// 4 * inv is finite, y4 = RN32(|x| * 4inv) equals 4 * RN32(|x| * inv) wherever
// the code can depend on it (scaling by 4 commutes with rounding in the normal
// range, and |x| * inv <= 6 cannot overflow), so the code is the table lookup
// at n = (uint)min(y4, 20) with no NaN to guard against; otherwise (a zero or
// subnormal row amax) the encoder of the generic path is used.
// The clamp to tau costs no operation of its own: rounding is monotone, so
// RN32(min(|x|, tau) * 4inv) = min(RN32(|x| * 4inv), RN32(tau * 4inv)), and with
// the cap at 20 both minima fold into one against cap4 = min(RN32(tau * 4inv), 20).
__device__ inline float code_cap4(float tau, float inv4) {
  return fminf(__fmul_rn(tau, inv4), 20.0f);
}

// Magnitude codes of the two elements of a bfloat16 pair word (bits 0-2: the
// low half, bits 4-6: the high half).
__device__ inline uint32_t bf16_pair_mag(uint32_t w, float inv4, float cap4) {
  const uint32_t nlo = uint32_t(fminf(__fmul_rn(fabsf(__uint_as_float(w << 16)), inv4), cap4));
  const uint32_t nhi =
      uint32_t(fminf(__fmul_rn(fabsf(__uint_as_float(w & 0xffff0000u)), inv4), cap4));
  constexpr uint64_t kLut = e2m1_lut();
  const uint32_t mlo = uint32_t(kLut >> (3u * nlo)) & 7u;
  const uint32_t mhi = uint32_t(kLut >> (3u * nhi)) & 7u;
  return mlo | (mhi << 4);
}

// Sign bits of the 8 codes of a bfloat16 chunk (bit 3 of each nibble): byte k
// of the code word holds elements 2k (low half of word k) and 2k+1 (high
// half), whose signs are bit 7 of bytes 1 and 3 of word k. Four byte permutes
// gather those bytes, one per word, into place.
__device__ inline uint32_t bf16_chunk_signs(const uint4& w) {
  const uint32_t hs = __builtin_amdgcn_perm(w.y, w.x, 0x0c0c0703u) |
                      __builtin_amdgcn_perm(w.w, w.z, 0x07030c0cu);
  const uint32_t ls = __builtin_amdgcn_perm(w.y, w.x, 0x0c0c0501u) |
                      __builtin_amdgcn_perm(w.w, w.z, 0x05010c0cu);
  return (hs & 0x80808080u) | ((ls >> 4) & 0x08080808u);
}

// The 8 codes of a bfloat16 chunk (4 * inv finite), low nibble first.
__device__ inline uint32_t bf16_chunk_code(const uint4& w, float inv4, float cap4) {
  return bf16_pair_mag(w.x, inv4, cap4) | (bf16_pair_mag(w.y, inv4, cap4) << 8) |
         (bf16_pair_mag(w.z, inv4, cap4) << 16) | (bf16_pair_mag(w.w, inv4, cap4) << 24) |
         bf16_chunk_signs(w);
}

__device__ inline uint32_t bf16_pair_code_slow(uint32_t w, float tau, float inv) {
  const float lo = fminf(fabsf(__uint_as_float(w << 16)), tau);
  const float hi = fminf(fabsf(__uint_as_float(w & 0xffff0000u)), tau);
  return e2m1_magnitude(lo, inv) | (e2m1_magnitude(hi, inv) << 4) | ((w >> 12) & 0x8u) |
         ((w >> 24) & 0x80u);
}

__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off, kWave);
    v = v > o ? v : o;
  }
  return v;
}


// Row amax (clamped to tau), scale and codes of a bfloat16 row whose words
// w[j] (chunk j of lane l: columns (64j + l) * 8 .. +7, zero past K) the wave
// holds: the codes of the columns below Kp (zero padding included) go to
// qrow, 8 per 32-bit store, and lane 0 writes the scale to *s_out.
template <int CH>
__device__ inline void quantize_bf16_row(const uint4 (&w)[CH], int64_t Kp, float tau,
                                         uint8_t* __restrict__ qrow, float* __restrict__ s_out) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & (kWave - 1);
  u16x2 m2 = {0, 0};
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const uint32_t q[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, q[i] & 0x7fff7fffu));
  }
  const uint32_t mk = wave_max_u32(uint32_t(m2.x > m2.y ? m2.x : m2.y));
  const float amax = fminf(__uint_as_float(mk << 16), tau);
  float s, inv;
  vector_scale(amax, s, inv);
  if (lane == 0) *s_out = s;
  const float inv4 = __fmul_rn(inv, 4.0f);
  if (inv4 < __builtin_huge_valf()) {
    const float cap4 = code_cap4(tau, inv4);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int64_t c = (int64_t(j) * kWave + lane) * 8;
      if (c < Kp) *reinterpret_cast<uint32_t*>(qrow + c / 2) = bf16_chunk_code(w[j], inv4, cap4);
    }
  } else {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int64_t c = (int64_t(j) * kWave + lane) * 8;
      if (c < Kp)
        *reinterpret_cast<uint32_t*>(qrow + c / 2) =
            bf16_pair_code_slow(w[j].x, tau, inv) | (bf16_pair_code_slow(w[j].y, tau, inv) << 8) |
            (bf16_pair_code_slow(w[j].z, tau, inv) << 16) |
            (bf16_pair_code_slow(w[j].w, tau, inv) << 24);
    }
  }
}

// ---------------------------------------------------------------------------
// Micro-scaled (MXFP4) blocks: 32 consecutive codes along K, one E8M0 scale.
// ---------------------------------------------------------------------------
// Least e >= -127 with 6 * 2^e >= amax (amax >= 0, finite). With
// amax = m * 2^E, 1 <= m < 2: 1.5 * 2^E = 6 * 2^(E-2) covers amax exactly when
// m <= 1.5, else 3 * 2^E = 6 * 2^(E-1) does. Zero and subnormal amax (and
// every normal one below 6 * 2^-127) give -127.
__device__ inline int mx_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int biased = int(b >> 23);
  int e = ((b & 0x7fffffu) <= 0x400000u) ? biased - 129 : biased - 128;
  if (biased == 0) e = -127;
  return e < -127 ? -127 : e;
}

// Magnitude index of y = ax / 2^e: 4y = ax * 2^(2-e) is exact (ldexp never
// rounds a result that reaches a midpoint; 4y <= 24), and the index is the
// table lookup of the token-wise encoder at n = min(floor(4y), 20).
__device__ inline uint32_t mx_magnitude(float ax, int e) {
  uint32_t n = cvt_u32_sat(ldexpf(ax, 2 - e));
  n = n < 20u ? n : 20u;
  return uint32_t(e2m1_lut() >> (3u * n)) & 7u;
}

__device__ inline float quad_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1, kWave));
  return fmaxf(v, __shfl_xor(v, 2, kWave));
}

}  // namespace fp4lin
