// qgemv_impl.h -- gfx950 GEMV kernel templates shared by libqgemv.so's
// translation units: the block formats, the fused row dot, the GEMV kernel and
// its launch-shape picker.  Each fused-transform variant of the GEMV kernel is
// instantiated in a translation unit of its own (gemv_op*.hip, and the
// several-token kernels in gemv_batch.hip), so the library builds in
// parallel; qgemv.hip holds the chain kernel and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <stdint.h>

#include <type_traits>
#include <utility>

#include "qgemv.h"

namespace qgemv_detail {


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxWindows = QG_MAX_WINDOWS;
constexpr int kMaxC = 2;         // block columns per lane
constexpr int kMaxWT = 12;       // waves per team

// ---------------------------------------------------------------------------
// Formats.  The unit of work of a lane is 32 consecutive weights: a whole
// block of the 32-weight formats, one sub-block (kUnits = 8 per block) of the
// 256-weight K-quant super-blocks.  Q8_0 and MXFP4: decode() turns a block's
// payload into 32 "unit" values u_j and scale() its scale field into a Scale
// with w_j = apply(scale, u_j); the GEMV applies the scale once to a block's
// partial dot product, the dequant kernel to every u_j.  Q4_0 and the
// K-quants (kDot) have a dot() of their own and a dequant() built from the
// same code formation.  The bit-exact decode check therefore covers the code
// formation of every format's GEMV; the one-hot GEMV tests (x a unit vector,
// every position of a block) cover the GEMV's own arithmetic on it.
// ---------------------------------------------------------------------------

template <int FMT> struct Fmt;

// Q8_0: fp16 d, 32 x int8 q; w = d * q (RAMforge README, "Milestone 5").
template <> struct Fmt<QG_Q8_0> {
  static constexpr int kBytes = 34, kScaleBytes = 2, kWords = 8, kUnits = 1;
  static constexpr bool kSums = false, kDot = false;
  struct Scale { float d; };
  __device__ static inline Scale scale(uint32_t bits) {
    return Scale{__half2float(__ushort_as_half((uint16_t)bits))};
  }
  __device__ static inline void decode(const uint32_t *q, float u[32]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k) u[4 * i + k] = (float)(int8_t)(q[i] >> (8 * k));
    }
  }
  __device__ static inline float apply(Scale s, float v) { return s.d * v; }
  __device__ static inline float fma_acc(Scale s, float v, float acc) { return fmaf(s.d, v, acc); }
};

// Q4_0: fp16 d, 16 bytes of nibbles; w = d * (q - 8) (RAMforge README,
// "Milestone 5").  Element j < 16 is the low nibble of byte j, element j + 16
// the high nibble.  Every code is turned into its weight's exact code value
// before it meets x, so a weight of zero adds exactly zero and a row of zero
// weights gives exactly 0.  Two codes at a time: a nibble masked into the
// mantissa of the fp16 1024 (0x6400) gives 1024 + q (a high nibble, masked in
// place, gives 1024 + 16 q), and one packed fp16 subtraction of 1032 (1152)
// leaves q - 8 (16 (q - 8)) exactly; v_fma_mix_f32 takes those fp16 values
// straight into the fp32 FMAs.  That is 1 shift, 4 and-or, 4 packed
// subtractions and 8 FMAs per 8 weights; the high nibbles' factor 16 comes
// out once per block, exactly.  The dequant kernel forms the weights from the
// same codes().
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
template <> struct Fmt<QG_Q4_0> {
  static constexpr int kBytes = 18, kScaleBytes = 2, kWords = 4, kUnits = 1;
  static constexpr bool kSums = false, kDot = true;
  // Word i of the payload (bytes 4i .. 4i+3) gives four fp16 pairs:
  //   lo[2i]     = (q_{4i}      - 8,  q_{4i+2}      - 8)   low nibbles of bytes 0, 2
  //   lo[2i + 1] = (q_{4i+1}    - 8,  q_{4i+3}      - 8)   low nibbles of bytes 1, 3
  //   hi[2i]     = 16 (q_{16+4i}   - 8, q_{16+4i+2} - 8)   high nibbles of bytes 0, 2
  //   hi[2i + 1] = 16 (q_{16+4i+1} - 8, q_{16+4i+3} - 8)   high nibbles of bytes 1, 3
  __device__ static inline void codes(const uint32_t (&q)[4], h16x2 (&lo)[8], h16x2 (&hi)[8]) {
    const h16x2 b_lo = {(_Float16)1032.0f, (_Float16)1032.0f}, b_hi = {(_Float16)1152.0f, (_Float16)1152.0f};
    // The exponent bits in a register the compiler cannot fold, so that each
    // mask-and-insert is one v_and_or_b32 (mask from a scalar register)
    // rather than an and and an or with literals.
    uint32_t e = 0x64006400u;
    asm("" : "+v"(e));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = q[i], v = q[i] >> 8;
      lo[2 * i] = __builtin_bit_cast(h16x2, (w & 0x000F000Fu) | e) - b_lo;
      lo[2 * i + 1] = __builtin_bit_cast(h16x2, (v & 0x000F000Fu) | e) - b_lo;
      hi[2 * i] = __builtin_bit_cast(h16x2, (w & 0x00F000F0u) | e) - b_hi;
      hi[2 * i + 1] = __builtin_bit_cast(h16x2, (v & 0x00F000F0u) | e) - b_hi;
    }
  }
  // res[t] = acc[t] + the block's dot with token t's inputs: the low-nibble
  // elements in chains p0 (elements 4i, 4i + 2) and p1 (4i + 1, 4i + 3), the
  // high ones (times 16) in p2 and p3; then d ((p0 + p1) + (p2 + p3) / 16).
  template <int NT>
  __device__ static inline void dot(const uint8_t *blk, const float (&x)[NT][32], const float (&xs)[NT][2],
                                    const float (&acc)[NT], float (&res)[NT]);
  // The 32 weights, from the same codes as the dot: d (q - 8), exact in fp32.
  __device__ static inline void dequant(const uint8_t *blk, float w[32]);
};

// MXFP4: E8M0 e, 16 bytes of E2M1 nibbles; w = 2^(e-127) * E2M1(nib) (block
// size from neurostream README, "The idea": 4.41 MB per 2,880 x 2,880 expert).
// gfx950's v_cvt_scalef32_pk_f32_fp4 turns both nibbles of a byte into fp32
// (scale 1.0: the E2M1 value itself, exact); the E8M0 scale is applied with an
// exact ldexp, and e = 255 gives NaN.
template <> struct Fmt<QG_MXFP4> {
  static constexpr int kBytes = 17, kScaleBytes = 1, kWords = 4, kUnits = 1;
  static constexpr bool kSums = false, kDot = false;
  struct Scale { int e; };
  __device__ static inline Scale scale(uint32_t bits) { return Scale{(int)(bits & 0xffu)}; }
  // f = (value of the byte's low nibble, value of its high nibble)
  template <typename V2>
  __device__ static inline void unpack(V2 f, float *u) {
    u[0] = f[0];
    u[16] = f[1];
  }
  __device__ static inline void decode(const uint32_t *q, float u[32]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      unpack(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], 1.0f, 0), u + 4 * i + 0);
      unpack(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], 1.0f, 1), u + 4 * i + 1);
      unpack(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], 1.0f, 2), u + 4 * i + 2);
      unpack(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], 1.0f, 3), u + 4 * i + 3);
    }
  }
  __device__ static inline float apply(Scale s, float v) {
    return s.e == 255 ? __builtin_nanf("") : ldexpf(v, s.e - 127);
  }
  __device__ static inline float fma_acc(Scale s, float v, float acc) { return acc + apply(s, v); }
};

__device__ __forceinline__ float half_bits(uint32_t h) { return __half2float(__ushort_as_half((uint16_t)h)); }
// The fp16 in the low / high half of a word, widened (exact, subnormals kept).
__device__ __forceinline__ float h16_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)v); }
__device__ __forceinline__ float h16_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

template <int NT>
__device__ inline void Fmt<QG_Q4_0>::dot(const uint8_t *blk, const float (&x)[NT][32], const float (&)[NT][2],
                                         const float (&acc)[NT], float (&res)[NT]) {
  uint32_t sbits = 0, q[4];
  __builtin_memcpy(&sbits, blk, 2);
  __builtin_memcpy(q, blk + 2, 16);
  const float d = half_bits(sbits);
  h16x2 lo[8], hi[8];
  codes(q, lo, hi);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[0] = fmaf((float)lo[2 * i][0], x[t][4 * i + 0], p[0]);
      p[1] = fmaf((float)lo[2 * i + 1][0], x[t][4 * i + 1], p[1]);
      p[2] = fmaf((float)hi[2 * i][0], x[t][16 + 4 * i + 0], p[2]);
      p[3] = fmaf((float)hi[2 * i + 1][0], x[t][16 + 4 * i + 1], p[3]);
      p[0] = fmaf((float)lo[2 * i][1], x[t][4 * i + 2], p[0]);
      p[1] = fmaf((float)lo[2 * i + 1][1], x[t][4 * i + 3], p[1]);
      p[2] = fmaf((float)hi[2 * i][1], x[t][16 + 4 * i + 2], p[2]);
      p[3] = fmaf((float)hi[2 * i + 1][1], x[t][16 + 4 * i + 3], p[3]);
    }
    res[t] = fmaf(d, fmaf(p[2] + p[3], 0.0625f, p[0] + p[1]), acc[t]);
  }
}

__device__ inline void Fmt<QG_Q4_0>::dequant(const uint8_t *blk, float w[32]) {
  uint32_t sbits = 0, q[4];
  __builtin_memcpy(&sbits, blk, 2);
  __builtin_memcpy(q, blk + 2, 16);
  const float d = half_bits(sbits);
  h16x2 lo[8], hi[8];
  codes(q, lo, hi);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[4 * i + 0] = d * (float)lo[2 * i][0];
    w[4 * i + 1] = d * (float)lo[2 * i + 1][0];
    w[4 * i + 2] = d * (float)lo[2 * i][1];
    w[4 * i + 3] = d * (float)lo[2 * i + 1][1];
    w[16 + 4 * i + 0] = d * ((float)hi[2 * i][0] * 0.0625f);
    w[16 + 4 * i + 1] = d * ((float)hi[2 * i + 1][0] * 0.0625f);
    w[16 + 4 * i + 2] = d * ((float)hi[2 * i][1] * 0.0625f);
    w[16 + 4 * i + 3] = d * ((float)hi[2 * i + 1][1] * 0.0625f);
  }
}

// Q4_K: 144-byte super-block of 256 weights = fp16 d, fp16 dmin, 12 bytes of
// packed 6-bit sub-block scales sc and mins m, 128 bytes of nibbles;
// w = d sc q - dmin m (RAMforge README, "Milestone 5", Q4_K line), in GGUF's
// packing: sub-block s < 4 keeps sc and m in the low six bits of scale bytes
// s and s + 4; s >= 4 keeps their low nibbles in byte s + 4 and their top two
// bits in the top bits of bytes s - 4 (sc) and s (m).  The codes of
// sub-block s are one nibble (low for even s) of bytes 32 (s / 2) .. + 31.
// A unit's dot is d sc (sum q x) - dmin m (sum x), with sum x formed once per
// activation vector.  The GEMV takes two codes per 32-bit word as fp16
// subnormals, q 2^-24 (or 16 q 2^-24 for an odd sub-block's high nibbles,
// masked in place), which v_fma_mix_f32 multiplies into the fp32 sums with
// no separate conversion; the power of two comes back in the scale, so the
// sums are those of the plain codes, bit for bit.
template <> struct Fmt<QG_Q4_K> {
  static constexpr int kBytes = 144, kUnits = 8;
  static constexpr bool kSums = true, kDot = true;
  __device__ static inline void scale_min(const uint8_t *blk, int s, int &sc, int &m) {
    const int a = blk[4 + (s & 3)], b = blk[8 + (s & 3)], c = blk[12 + (s & 3)];
    sc = s < 4 ? (a & 63) : ((c & 15) | ((a >> 6) << 4));
    m = s < 4 ? (b & 63) : ((c >> 4) | ((b >> 6) << 4));
  }
  // The sub-block's codes, scaled by 16 for odd s, and that scale's inverse.
  template <typename P>
  __device__ static inline float codes(const P *blk, int s, uint32_t q[8]) {
    __builtin_memcpy(q, blk + 16 + 32 * (s >> 1), 32);
    const uint32_t mask = (s & 1) ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] &= mask;
    return (s & 1) ? 0.0625f : 1.0f;
  }
  // res[t] = acc[t] + this sub-block's dot with token t's inputs; the codes
  // are read and masked once for all NT tokens.
  template <int NT>
  __device__ static inline void dot(const uint8_t *blk, int s, const float (&x)[NT][32], const float (&xs)[NT][2],
                                    const float (&acc)[NT], float (&res)[NT]) {
    // d, dmin and the 12 scale bytes in one 16-byte read; this sub-block's
    // three scale bytes are byte s & 3 of words 1, 2 and 3
    uint32_t hw[4];
    __builtin_memcpy(hw, blk, 16);
    const uint32_t hd = hw[0];
    const int sh = 8 * (s & 3);
    const int a = (int)((hw[1] >> sh) & 0xffu), b = (int)((hw[2] >> sh) & 0xffu), c = (int)((hw[3] >> sh) & 0xffu);
    const int sc = s < 4 ? (a & 63) : ((c & 15) | ((a >> 6) << 4));
    const int m = s < 4 ? (b & 63) : ((c >> 4) | ((b >> 6) << 4));
    uint32_t q[8];
    __builtin_memcpy(q, blk + 16 + 32 * (s >> 1), 32);
    // codes of bytes 0 and 2 (then 1 and 3) of a word as two fp16 subnormals
    const uint32_t mask = (s & 1) ? 0x00F000F0u : 0x000F000Fu;
    const float f = (s & 1) ? 0x1p20f : 0x1p24f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t a = q[i] & mask, b = (q[i] >> 8) & mask;
        p[0] = fmaf(h16_lo(a), x[t][4 * i + 0], p[0]);
        p[1] = fmaf(h16_lo(b), x[t][4 * i + 1], p[1]);
        p[2] = fmaf(h16_hi(a), x[t][4 * i + 2], p[2]);
        p[3] = fmaf(h16_hi(b), x[t][4 * i + 3], p[3]);
      }
      const float r = fmaf(half_bits(hd) * (float)sc * f, (p[0] + p[1]) + (p[2] + p[3]), acc[t]);
      res[t] = fmaf(-(half_bits(hd >> 16) * (float)m), xs[t][0] + xs[t][1], r);
    }
  }
  // The 32 weights of sub-block s, each rounded once: d sc q and dmin m are
  // exact in fp32 (so is d sc / 16 times 16 q).
  __device__ static inline void dequant(const uint8_t *blk, int s, float w[32]) {
    uint32_t hd;
    __builtin_memcpy(&hd, blk, 4);
    int sc, m;
    scale_min(blk, s, sc, m);
    uint32_t q[8];
    const float f = codes(blk, s, q);
    const float ds = half_bits(hd) * (float)sc * f, mm = half_bits(hd >> 16) * (float)m;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) w[4 * i + k] = ds * (float)((q[i] >> (8 * k)) & 0xffu) - mm;
  }
};

// Q6_K: 210-byte super-block of 256 weights = 128 bytes of low nibbles ql,
// 64 bytes of 2-bit high parts qh, 16 int8 scales (one per 16 weights), fp16
// d; w = d scale (q - 32) (GGUF's layout; the pages name the format only).
// Unit u = 4 h + i (32 weights 128 h + 32 i + l) takes its low nibbles from
// ql[64 h + 32 (i & 1) + l] (high nibble for i >= 2), its top bits from bits
// 2 i, 2 i + 1 of qh[32 h + l], its scales from bytes 2 u, 2 u + 1.  Each
// 6-bit code is formed as the int8 4 (q - 32), exactly: its low four bits
// rotated to bits 2..5 of the byte, the top two to bits 6, 7 with the top one
// flipped (q ^ 32 is q - 32 in 6-bit two's complement), so a weight of zero
// (q = 32) adds exactly zero and the dot takes no sum of x.  The factor 4
// comes out of d exactly.  The dequant kernel forms the weights from the same
// codes().
// N words of LDS starting at byte p (any alignment), read as N + 1 aligned
// dwords and funnel-shifted into place (p must point into LDS; the reads may
// touch up to 3 bytes past the last word, which the staged rows leave room
// for).  gfx950 serves unaligned DS reads, but each one stalls the CU's LDS
// pipe (SQ_LDS_UNALIGNED_STALL): for Q6_K's 210-byte super-blocks, whose
// alignment changes from one to the next, those stalls bounded the kernel
// (the Q4_K_M pass's Q6_K down projection 40.1 -> 27.0 us per launch with
// this), and for MXFP4's 17-byte blocks they cost the MoE grids a little.
// For Q8_0 and Q4_0 the extra shifts cost more than the stalls.
template <int N>
__device__ __forceinline__ void lds_words(const uint8_t *p, uint32_t (&q)[N]) {
  typedef __attribute__((address_space(3))) const uint8_t lds_u8;
  typedef __attribute__((address_space(3))) const uint32_t lds_u32;
  lds_u8 *lp = (lds_u8 *)p;
  const uint32_t mis = (uint32_t)(uintptr_t)lp & 3u;
  lds_u32 *w = (lds_u32 *)(lp - mis);
  uint32_t v[N + 1];
#pragma unroll
  for (int i = 0; i <= N; ++i) v[i] = w[i];
#pragma unroll
  for (int i = 0; i < N; ++i) q[i] = __builtin_amdgcn_alignbit(v[i + 1], v[i], 8 * mis);
}

template <> struct Fmt<QG_Q6_K> {
  static constexpr int kBytes = 210, kUnits = 8;
  static constexpr bool kSums = false, kDot = true;
  // Byte l of word w of q is 4 (q_e - 32) for element e = 4 w + l of unit u.
  template <bool kLds>
  __device__ static inline void codes(const uint8_t *blk, int u, uint32_t q[8]) {
    const int h = u >> 2, i = u & 3;
    uint32_t lo[8], hi[8];
    if constexpr (kLds) {
      lds_words<8>(blk + 64 * h + 32 * (i & 1), lo);
      lds_words<8>(blk + 128 + 32 * h, hi);
    } else {
      __builtin_memcpy(lo, blk + 64 * h + 32 * (i & 1), 32);
      __builtin_memcpy(hi, blk + 128 + 32 * h, 32);
    }
    // rotations right: the nibble at bit 4 (i >= 2) or 0 of each byte to bit
    // 2; bits 2 i, 2 i + 1 to bits 6, 7 (bits that wrap into another byte land
    // outside the kept field)
    const int rlo = (i >> 1) ? 2 : 30, rhi = (2 * i - 6) & 31;
#pragma unroll
    for (int w = 0; w < 8; ++w)
      q[w] = ((__builtin_amdgcn_alignbit(lo[w], lo[w], rlo) & 0x3C3C3C3Cu) |
              (__builtin_amdgcn_alignbit(hi[w], hi[w], rhi) & 0xC0C0C0C0u)) ^ 0x80808080u;
  }
  template <int NT>
  __device__ static inline void dot(const uint8_t *blk, int u, const float (&x)[NT][32], const float (&)[NT][2],
                                    const float (&acc)[NT], float (&res)[NT]) {
    uint32_t q[8];
    codes<true>(blk, u, q);
    const float sa = (float)(int8_t)blk[192 + 2 * u], sb = (float)(int8_t)blk[193 + 2 * u];
    uint32_t hd = 0;
    __builtin_memcpy(&hd, blk + 208, 2);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int w = 0; w < 8; ++w)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          p[2 * (w >> 2) + (k & 1)] =
              fmaf((float)(int8_t)(q[w] >> (8 * k)), x[t][4 * w + k], p[2 * (w >> 2) + (k & 1)]);
      res[t] = fmaf(half_bits(hd) * 0.25f, fmaf(sa, p[0] + p[1], sb * (p[2] + p[3])), acc[t]);
    }
  }
  // The 32 weights of unit u, each rounded once: d scale is exact in fp32.
  __device__ static inline void dequant(const uint8_t *blk, int u, float w[32]) {
    uint32_t q[8];
    codes<false>(blk, u, q);
    uint32_t hd = 0;
    __builtin_memcpy(&hd, blk + 208, 2);
    const float d4 = half_bits(hd) * 0.25f;
    const float da = d4 * (float)(int8_t)blk[192 + 2 * u], db = d4 * (float)(int8_t)blk[193 + 2 * u];
#pragma unroll
    for (int v = 0; v < 8; ++v)
#pragma unroll
      for (int k = 0; k < 4; ++k) w[4 * v + k] = (v < 4 ? da : db) * (float)(int8_t)(q[v] >> (8 * k));
  }
};

// ---------------------------------------------------------------------------
// GEMV kernel
// ---------------------------------------------------------------------------

struct WinDev {
  const uint8_t *base;  // row 0 of the window's matrix (16-byte aligned)
  const uint8_t *base2; // SwiGLU pairs: row 0 of the up matrix (base is the gate's)
  const float *x;
  const float *x2;      // the multiplier of QG_IN_SILU_MUL, else unused
  float *y;             // y[r - row_start] <-> row r
  int64_t row_start, row_end;
};

struct GemvArgs {
  WinDev win[kMaxWindows];
  int32_t tile_prefix[kMaxWindows + 1];  // tiles of windows [0, w)
  int64_t row_bytes;
  int64_t block_rows;  // > 0 (the host replaces 0 by a bound above every window)
  int32_t n_win, nb, tile_rows, n_tiles;
  int32_t tiles_per_block;  // ceil(block_rows / tile_rows)
  int32_t in_op;   // QG_IN_X, QG_IN_RMS or QG_IN_SILU_MUL: applied as x is loaded
  int32_t out_op;  // QG_OUT_Y or QG_OUT_GELU: applied as y is stored
  float eps;       // of QG_IN_RMS
  // Several tokens per launch (NT > 1): token t's x at win.x + t x_stride,
  // its y at win.y + t y_stride.
  int64_t x_stride, y_stride;
};

// Up to 16 tokens on the matrix cores (gemv_mfma.hip): rows [0, n_rows) of a
// matrix whose row r starts at w + r row_bytes; token t < n_tok reads
// x + t x_stride and writes y + t y_stride.
struct MfmaArgs {
  const uint8_t *w;
  const float *x;
  float *y;
  int64_t row_bytes, n_rows, x_stride, y_stride;
  int32_t nb, n_tok;
};
// Enqueues the launch (Q8_0, Q4_0, MXFP4; else QG_E_FMT); the caller checks
// the launch status.
int launch_gemv_mfma(int32_t fmt, const MfmaArgs &a, hipStream_t stream);

// Sum over the 64 lanes of a wave in a fixed order (DPP row shifts, then row
// broadcasts); the total lands in lane 63.
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK,
                                                               BANK_MASK, false));
}

__device__ __forceinline__ float wave_sum63(float v) {
  v += dpp_f<0x111, 0xf, 0xf>(v);  // row_shr:1
  v += dpp_f<0x112, 0xf, 0xf>(v);  // row_shr:2
  v += dpp_f<0x114, 0xf, 0xe>(v);  // row_shr:4
  v += dpp_f<0x118, 0xf, 0xc>(v);  // row_shr:8
  v += dpp_f<0x142, 0xa, 0xf>(v);  // row_bcast:15
  v += dpp_f<0x143, 0xc, 0xf>(v);  // row_bcast:31
  return v;
}

// Exact (erf) GELU, evaluated as 0.5 t erfc(-t / sqrt 2): equal to
// 0.5 t (1 + erf(t / sqrt 2)), without that form's cancellation for t far
// below 0 (which an RMS normalisation of small GELU values would magnify).
__device__ __forceinline__ float gelu_erf(float t) { return 0.5f * t * erfcf(-t * 0.70710678118654752f); }

// silu(g) * u = g u / (1 + exp(-g)), with the hardware exp2 and reciprocal
// (v_exp_f32, v_rcp_f32: about 1 ulp each; rounding -g log2(e) adds about
// |g| 2^-24 relative), so about (|g| + 4) 2^-24 relative in all.  The fused
// x-load evaluates it for every input a team loads, where a libm exp and an
// IEEE division (some thirty instructions) doubled a small MoE down grid.
// qgemv_silu_mul uses this same function, so the two give the same bits.
__device__ __forceinline__ float silu_times(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// One wave's partial sums for one staged row and NT tokens: lane l dots
// blocks l + 64c (c < C) of the wave's slice, staged at byte `ph` of `sb`,
// with each token's registered activations, decoding every block once.
// Fixed order per token: four FMA chains per block combined as
// (p0 + p1) + (p2 + p3), the block scale applied once, blocks in c order --
// the same for any NT, so a token's sum does not depend on its batch.
template <int FMT, int C, int NT>
__device__ __forceinline__ void row_partial(const uint8_t *sb, int ph, int lane, int slice_n,
                                            const float (&xr)[C][NT][32], const float (&xs)[C][NT][2],
                                            float (&s)[NT]) {
  using F = Fmt<FMT>;
#pragma unroll
  for (int t = 0; t < NT; ++t) s[t] = 0.0f;
  if constexpr (F::kUnits > 1) {
    // K-quants: lane l's unit b = l + 64 c is sub-block b % 8 of the slice's
    // super-block b / 8.
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int b = lane + 64 * c;
      float acc[NT];
      F::template dot<NT>(sb + ph + F::kBytes * (b >> 3), b & 7, xr[c], xs[c], s, acc);
#pragma unroll
      for (int t = 0; t < NT; ++t) s[t] = b < slice_n ? acc[t] : s[t];
    }
  } else if constexpr (F::kDot) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int b = lane + 64 * c;
      float acc[NT];
      F::template dot<NT>(sb + ph + F::kBytes * b, xr[c], xs[c], s, acc);
#pragma unroll
      for (int t = 0; t < NT; ++t) s[t] = b < slice_n ? acc[t] : s[t];
    }
  } else {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int b = lane + 64 * c;
      const int bo = ph + F::kBytes * b;  // block's byte offset in the staged row
      // LDS reads at any byte alignment (gfx950 serves unaligned DS accesses;
      // MXFP4 realigns aligned words instead, as above).
      uint32_t sbits = 0, q[F::kWords];
      __builtin_memcpy(&sbits, sb + bo, F::kScaleBytes);
      if constexpr (FMT == QG_MXFP4) {
        lds_words<F::kWords>(sb + bo + F::kScaleBytes, q);
      } else {
        __builtin_memcpy(q, sb + bo + F::kScaleBytes, 4 * F::kWords);
      }
      float u[32];
      F::decode(q, u);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int e = 0; e < 32; ++e) p[e & 3] = fmaf(u[e], xr[c][t][e], p[e & 3]);
        const float blk_acc = F::fma_acc(F::scale(sbits), (p[0] + p[1]) + (p[2] + p[3]), s[t]);
        s[t] = b < slice_n ? blk_acc : s[t];
      }
    }
  }
}

// One token's partial sum (the chain kernel's form).
template <int FMT, int C>
__device__ __forceinline__ float row_partial(const uint8_t *sb, int ph, int lane, int slice_n,
                                             const float (&xr)[C][32], const float (&xs)[C][2]) {
  float s[1];
  row_partial<FMT, C, 1>(sb, ph, lane, slice_n, reinterpret_cast<const float (&)[C][1][32]>(xr),
                         reinterpret_cast<const float (&)[C][1][2]>(xs), s);
  return s[0];
}

// Each column's sums of its first and last 16 inputs, as row_partial takes
// them for the formats that fold an offset (Q4_0) or a min (K-quants) out of
// the dot; added in element order with no contraction of a producer's
// multiply, so every kernel forms the same bits from the same inputs.
template <int C>
__device__ __forceinline__ void unit_sums(const float (&xr)[C][32], float (&xs)[C][2]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int c = 0; c < C; ++c) {
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      lo += xr[c][e];
      hi += xr[c][16 + e];
    }
    xs[c][0] = lo;
    xs[c][1] = hi;
  }
}

// Largest rows per chain tile, per (format, block columns per lane): a chain
// wave holds its tile's fetched rows in registers until staged.
template <int FMT, int C> struct TileCap { static constexpr int value = 1; };
template <> struct TileCap<QG_Q8_0, 1> { static constexpr int value = 6; };
template <> struct TileCap<QG_Q8_0, 2> { static constexpr int value = 2; };
template <> struct TileCap<QG_Q4_0, 1> { static constexpr int value = 8; };
template <> struct TileCap<QG_Q4_0, 2> { static constexpr int value = 4; };
template <> struct TileCap<QG_MXFP4, 1> { static constexpr int value = 8; };
template <> struct TileCap<QG_MXFP4, 2> { static constexpr int value = 4; };

// Weight staging of gemv_kernel: a wave's slice of a row is copied from HBM
// straight into its LDS ring (gfx950 global_load_lds_dwordx4: lane l's 16
// bytes land at M0 + 16 l), V loads per row, each a whole aligned 16-byte
// granule per lane.  Lanes past the slice's last granule re-read that granule
// into their own place beyond the data, so every load is unconditional and
// the number of loads per row is a constant the waits can count.
template <int FMT, int C> struct Geo {
  static constexpr int CH = (15 + 64 * C / Fmt<FMT>::kUnits * Fmt<FMT>::kBytes + 15) / 16;  // granules a slice can touch
  static constexpr int V = (CH + 63) / 64;                               // loads per lane per row
  static constexpr int SLOT = 1024 * V;                                  // ring slot bytes
};

// Concurrency of gemv_kernel, a function of (format, team size): Q8_0 runs
// about six waves per compute unit, each with two rows in flight while it
// computes one more (one row in flight in teams of more than six waves); the
// 4-bit and 6-bit formats, with more decode work per byte, run twelve waves,
// each with two rows in flight.  More requests in flight than that (more
// waves, deeper rings, or two rows in Q8_0's twelve-wave teams) made the same
// walks slower on MI355X: HBM serves a compact, moderate stream better than a
// wide, deep one.
__host__ __device__ constexpr int gemv_waves_per_cu(int fmt) { return fmt == QG_Q8_0 ? 6 : 12; }
__host__ __device__ constexpr int gemv_teams_per_cu(int fmt, int wt) {
  return wt >= gemv_waves_per_cu(fmt) ? 1 : gemv_waves_per_cu(fmt) / wt;
}
__host__ __device__ constexpr int gemv_in_flight(int fmt, int wt) {
  return fmt != QG_Q8_0 || wt * gemv_teams_per_cu(fmt, wt) <= 6 ? 2 : 1;
}
constexpr int kGemvTileRows = 8;  // most rows per tile

// One asynchronous 16-byte HBM -> LDS copy per lane: global_load_lds_dwordx4
// with a scalar base, a 32-bit lane offset and the LDS destination in M0.
// Written as inline assembly because the compiler's own waits for LDS DMA
// drain every outstanding load before any LDS read; here the kernel counts
// its loads and waits with s_waitcnt vmcnt itself.  Weights are read once
// per pass, so the loads carry the non-temporal hint (nt): on MI355X that
// took the 44-layer Q8_0 pass from 4.17 to 4.02 ms per token (the
// k = 24576 GEMV from 31.1 to 29.1 us).
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
template <int N> __device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One team = WT waves.  Wave w owns the contiguous block columns
// [w*64*C, (w+1)*64*C) of every row (its "slice"), lane l the columns
// w*64*C + l + 64*c, whose 32 activations each it keeps in registers.
// A tile is up to tile_rows rows of one row block; team b takes tiles
// b, b + T, b + 2T, ... (T teams), so at any moment the grid works on a
// compact band of the matrix.  Each wave streams its slices row after row
// through an LDS ring of NB + 1 slots: before computing a row it issues the
// copy of the row NB ahead (crossing tiles), so NB rows are in flight while
// it decodes.  The team's per-wave row sums meet in LDS and are added in
// wave order.
// The fused transforms a launch applies, fixed at compile time: code for an
// op a launch does not use (even behind a runtime branch) made the plain GEMV
// up to 17% slower.
// kOpSwiglu / kOpRmsSwiglu: the window pairs a gate and an up matrix; its
// "rows" alternate gate row r, up row r (virtual row 2r, 2r + 1), and the
// store writes silu(gate . x) * (up . x) once per pair.
enum GemvOp { kOpNone = 0, kOpRms = 1, kOpRmsGelu = 2, kOpSilu = 3, kOpGelu = 4, kOpSwiglu = 5, kOpRmsSwiglu = 6 };
__host__ __device__ constexpr int op_in(int op) {
  return op == kOpRms || op == kOpRmsGelu || op == kOpRmsSwiglu ? QG_IN_RMS
         : op == kOpSilu                                        ? QG_IN_SILU_MUL
                                                                : QG_IN_X;
}
__host__ __device__ constexpr bool op_gelu(int op) { return op == kOpRmsGelu || op == kOpGelu; }
__host__ __device__ constexpr bool op_pair(int op) { return op == kOpSwiglu || op == kOpRmsSwiglu; }

// NT > 1: NT tokens per launch (a small batch): every block is staged and
// decoded once and dotted with each token's activations, in the one-token
// order, so each token's y has the bits of a one-token launch.
template <int FMT, int WT, int C, int OP, int NT = 1>
__global__ void __launch_bounds__(64 * WT) gemv_kernel(const float *x_first, int32_t nb_first, int32_t tiles_first,
                                                       const GemvArgs a) {
  static_assert(NT == 1 || OP == kOpNone, "fused transforms take one token");
  static_assert(!op_pair(OP) || kGemvTileRows % 2 == 0, "SwiGLU tiles hold whole pairs");
  using G = Geo<FMT, C>;
  constexpr int V = G::V, SLOT = G::SLOT;
  constexpr int NB = gemv_in_flight(FMT, WT), NS = NB + 1;
  constexpr int SB = 64 * C;  // blocks per slice
  __shared__ __attribute__((aligned(16))) uint8_t ring[WT][NS][SLOT];
  __shared__ float red[2][WT][NT * kGemvTileRows];
  __shared__ float ssq[WT * C];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int nb = a.nb;
  const int64_t rb = a.row_bytes;
  const int slice_b0 = wave * SB;
  const int slice_n = max(0, min(SB, nb - slice_b0));  // >= 1 by the choice of WT
  // (a wave's slice is whole blocks: 64 C units are 8 C K-quant super-blocks)
  const int64_t slice_off = (int64_t)(slice_b0 / Fmt<FMT>::kUnits) * Fmt<FMT>::kBytes;
  const uint32_t slice_len = (uint32_t)(slice_n / Fmt<FMT>::kUnits) * Fmt<FMT>::kBytes;
  const int T = gridDim.x;

  // Kernel-argument fields used in the loop are read once into registers, and
  // a window's fields again only when a cursor enters the next window.  The
  // first window's and the tiling fields are all read before any is used, so
  // the launch waits on one round trip to the argument buffer, not a chain.
  const int n_tiles = a.n_tiles;
  const int64_t B = a.block_rows;
  const int TR = a.tile_rows;
  const int tpb = a.tiles_per_block;
  const float eps = a.eps;
  constexpr bool kPair = op_pair(OP);
  struct Win {
    int w, t0, t1;  // window index, its tiles [t0, t1)
    int64_t row_start, row_end;  // (SwiGLU pairs: virtual rows, two per output)
    const uint8_t *base;  // row 0, advanced to the wave's slice
    const uint8_t *base2; // SwiGLU pairs: the up matrix's, likewise
    const float *x, *x2;
    float *y;
  };
  auto load_win = [&](int w, Win &W) {
    W.w = w;
    W.t0 = a.tile_prefix[w];
    W.t1 = a.tile_prefix[w + 1];
    W.row_start = a.win[w].row_start;
    W.row_end = a.win[w].row_end;
    W.base = a.win[w].base + slice_off;
    if constexpr (kPair) W.base2 = a.win[w].base2 + slice_off;
    W.x = a.win[w].x;
    W.x2 = a.win[w].x2;
    W.y = a.win[w].y;
  };
  // The wave's slice of (virtual) row v of window W.
  auto row_ptr = [&](const Win &W, int64_t v) -> const uint8_t * {
    if constexpr (kPair) return ((v & 1) ? W.base2 : W.base) + (v >> 1) * rb;
    return W.base + v * rb;
  };
  struct Tile {
    int t, nrows;
    int64_t r0;
  };
  // Tile t of window W (advanced to the window holding t).
  auto locate = [&](int t, Win &W, Tile &Q) {
    if (t >= W.t1) {
      int w = W.w + 1;
      while (t >= a.tile_prefix[w + 1]) ++w;
      load_win(w, W);
    }
    const int tt = t - W.t0;
    // Row block and tile within it; a window of one row block (block_rows 0)
    // needs no division.
    int blk = 0, tib = tt;
    if (tt >= tpb) {
      blk = tt / tpb;
      tib = tt - blk * tpb;
    }
    Q.t = t;
    Q.r0 = W.row_start + (int64_t)blk * B + (int64_t)tib * TR;
    const int64_t r1 = min(Q.r0 + TR, min(W.row_start + (int64_t)(blk + 1) * B, W.row_end));
    Q.nrows = (int)(r1 - Q.r0);
  };

  const uint32_t lds0 = (uint32_t)(uintptr_t)&ring[wave][0][0];
  const uint32_t lane16 = 16u * lane;
  // Copy the wave's slice of the row at p (any byte alignment) into ring slot s.
  auto issue = [&](const uint8_t *p, int s) {
    const uint32_t ph = (uint32_t)((uintptr_t)p & 15);
    const uint32_t last16 = ((ph + slice_len - 1) >> 4) << 4;
    const uint8_t *pa = p - ph;
    const uint32_t l = lds0 + SLOT * s;
#pragma unroll
    for (int v = 0; v < V; ++v) dma16(pa, min(lane16 + 1024u * v, last16), l + 1024u * v);
  };

  // The team's activations: lane l of wave w holds the 32 inputs of block
  // column w*64*C + l + 64*c in xr[c], zero past the row.  The input
  // transforms are those of the separate calls, in the same order, so a
  // fused launch gives their bits: silu(x) * x2 elementwise as qgemv_silu_mul;
  // rms(x) with the sum of squares formed as qgemv_rms_carry forms it (32
  // consecutive inputs per lane in order, the lanes of a 64-column run by
  // wave_sum63, the runs in column order -- the team's waves cover every
  // column, so no extra read), then one scale per input.
  float xr[C][NT][32];
  float xs[C][NT][2];  // Q4_0, K-quants: the sums of each unit's first and last 16 inputs
  constexpr int in_op = op_in(OP);
  // A launch's first activations are gathered through the wave's LDS ring
  // while it is still idle: the column set's 2048 inputs are read 1 KB per
  // instruction (one cache line per 8 lanes; a lane reading its own 128 bytes
  // touches 64 lines per instruction, and those loads, not HBM, bounded the
  // launch's start: 0.2-1.3 us per launch on MI355X), written to LDS with a
  // rotation inside each 128-byte column, so that the lanes' reads spread over
  // the banks, and read back by the lane owning each column.  SKB KB per pass,
  // as much as the ring holds (less with two columns and a SiLU multiplier,
  // which would otherwise spill registers).  Later windows with other inputs
  // (copies in flight in the ring) load them directly.
  constexpr int kRingBytes = NS * SLOT;
  // A stage of its own for the first gather where the LDS has room for it
  // (one column per lane, one token, no SiLU multiplier): the ring's first
  // weight copies then go out as soon as the activations are written to LDS,
  // before they are read back and normalised (0.4-0.6 us earlier per launch
  // for the Q8_0 k = 6144 projections on MI355X).
  constexpr int kLdsXe = WT * (NS * SLOT + 8192) + 2 * WT * NT * kGemvTileRows * 4 + WT * C * 4;
  constexpr bool kXe = C == 1 && NT == 1 && op_in(OP) != QG_IN_SILU_MUL &&
                       gemv_teams_per_cu(FMT, WT) * kLdsXe <= 160 * 1024;
  __shared__ __attribute__((aligned(16))) uint8_t xst[kXe ? WT : 1][kXe ? 8192 : 16];
  constexpr int kSkbMax = (op_in(OP) == QG_IN_SILU_MUL && C == 2) ? 2 : 8;  // registers: two columns and x2
  constexpr int SKB0 = kXe ? 8 : kRingBytes >= 8192 ? 8 : kRingBytes >= 4096 ? 4 : kRingBytes >= 2048 ? 2 : 1;
  constexpr int SKB = SKB0 < kSkbMax ? SKB0 : kSkbMax;
  uint8_t *const stg = kXe ? &xst[kXe ? wave : 0][0] : &ring[wave][0][0];
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  // put(q, w): inputs 4q .. 4q + 3 of the lane's column
  // The first pass of the first window's gather is issued before the kernel
  // reads its argument block: the launch passes that window's x, nb and the
  // tile count as leading arguments, which the library's build preloads into
  // scalar registers (gfx950 kernel-argument preloading), so the loads go out
  // at the wave's first instructions instead of after a round trip to the
  // argument block in device memory.
  f32x4 pre[SKB];
  bool use_pre = false;
  auto gather = [&](const float *src, int c, auto put, auto after_writes) {
    const int base = 32 * (slice_b0 + 64 * c);
    const int lim = 32 * nb - 4;  // the last 16 bytes of the input vector
#pragma unroll
    for (int p = 0; p < 8 / SKB; ++p) {
      f32x4 v[SKB];
#pragma unroll
      for (int i = 0; i < SKB; ++i) {
        if (p == 0 && c == 0 && use_pre) {
          v[i] = pre[i];
        } else {
          const int f = min(base + 256 * (p * SKB + i) + 4 * lane, lim);
          __builtin_memcpy(&v[i], src + f, 16);
        }
      }
#pragma unroll
      for (int i = 0; i < SKB; ++i) {
        const int col = 8 * i + (lane >> 3);
        *reinterpret_cast<f32x4 *>(stg + 128 * col + 16 * (((lane & 7) + col) & 7)) = v[i];
      }
      if (p == 0 && c == 0) after_writes();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      const int cl = lane - 8 * SKB * p;
      if (cl >= 0 && cl < 8 * SKB) {
#pragma unroll
        for (int q = 0; q < 8; ++q) put(q, *reinterpret_cast<const f32x4 *>(stg + 128 * cl + 16 * ((q + cl) & 7)));
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
  };
  auto load_x_staged = [&](const float *x, const float *x2, auto after_writes) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = slice_b0 + lane + 64 * c;
      const bool ok = j < nb;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float *xt = NT == 1 ? x : x + t * a.x_stride;
        gather(xt, c, [&](int q, f32x4 w) {
          xr[c][t][4 * q + 0] = w.x;
          xr[c][t][4 * q + 1] = w.y;
          xr[c][t][4 * q + 2] = w.z;
          xr[c][t][4 * q + 3] = w.w;
        }, [&]() { if (t == 0) after_writes(); });
        if constexpr (in_op == QG_IN_SILU_MUL) {
          gather(x2, c, [&](int q, f32x4 u) {
            xr[c][t][4 * q + 0] = silu_times(xr[c][t][4 * q + 0], u.x);
            xr[c][t][4 * q + 1] = silu_times(xr[c][t][4 * q + 1], u.y);
            xr[c][t][4 * q + 2] = silu_times(xr[c][t][4 * q + 2], u.z);
            xr[c][t][4 * q + 3] = silu_times(xr[c][t][4 * q + 3], u.w);
          }, [] {});
        }
#pragma unroll
        for (int e = 0; e < 32; ++e) xr[c][t][e] = ok ? xr[c][t][e] : 0.0f;
      }
    }
  };
  auto load_x = [&](const float *x, const float *x2, auto staged, auto after_writes) {
    if constexpr (decltype(staged)::value) {
      load_x_staged(x, x2, after_writes);
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int j = slice_b0 + lane + 64 * c;
        const int jj = min(j, nb - 1);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float *xt = NT == 1 ? x : x + t * a.x_stride;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            float4 v;
            __builtin_memcpy(&v, xt + 32 * jj + 4 * q, 16);
            if constexpr (in_op == QG_IN_SILU_MUL) {
              float4 u;
              __builtin_memcpy(&u, x2 + 32 * jj + 4 * q, 16);
              v.x = silu_times(v.x, u.x);
              v.y = silu_times(v.y, u.y);
              v.z = silu_times(v.z, u.z);
              v.w = silu_times(v.w, u.w);
            }
            const bool ok = j < nb;
            xr[c][t][4 * q + 0] = ok ? v.x : 0.0f;
            xr[c][t][4 * q + 1] = ok ? v.y : 0.0f;
            xr[c][t][4 * q + 2] = ok ? v.z : 0.0f;
            xr[c][t][4 * q + 3] = ok ? v.w : 0.0f;
          }
        }
      }
    }
    if constexpr (in_op == QG_IN_RMS) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; ++e) ss = fmaf(xr[c][0][e], xr[c][0][e], ss);
        ss = wave_sum63(ss);
        if (lane == 63) ssq[C * wave + c] = ss;
      }
      __syncthreads();
      float tot = 0.0f;
#pragma unroll
      for (int v = 0; v < C * WT; ++v) tot += ssq[v];
      const float inv = 1.0f / sqrtf(tot / (float)(32 * nb) + eps);
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int e = 0; e < 32; ++e) xr[c][0][e] *= inv;
      __syncthreads();  // ssq is read before a later window rewrites it
    }
    if constexpr (Fmt<FMT>::kSums) {
      // Sums of the inputs as loaded: no multiply of a fused transform may
      // be contracted into these adds, or a fused launch would not give the
      // bits of the separate calls.
#pragma clang fp contract(off)
#pragma unroll
      for (int c = 0; c < C; ++c) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float lo = 0.0f, hi = 0.0f;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            lo += xr[c][t][e];
            hi += xr[c][t][16 + e];
          }
          xs[c][t][0] = lo;
          xs[c][t][1] = hi;
        }
      }
    }
  };

  // Copy cursor: fp is the wave's slice of the next row to copy, f_left the
  // rows left in its tile (F, window FW); both advance by one row per copy.
  // Past the team's last row the cursor stays on that row, re-copying it into
  // a slot no computation reads, which keeps one fixed count of loads per row.
  Win CW, FW;
  if ((int)blockIdx.x >= tiles_first) return;
  constexpr bool kPre = NT == 1 && op_in(OP) != QG_IN_SILU_MUL;
  if constexpr (kPre) {
    const int lim = 32 * nb_first - 4;
#pragma unroll
    for (int i = 0; i < SKB; ++i) {
      const int f = min(32 * slice_b0 + 256 * i + 4 * lane, lim);
      __builtin_memcpy(&pre[i], x_first + f, 16);
    }
  }
  load_win(0, CW);
  // An empty statement consuming those fields keeps the compiler from
  // sinking their loads past the branches below (one wait, not four); its
  // memory clobber keeps the activation prefetch above it.
  asm volatile("" ::"s"(n_tiles), "s"(B), "s"(TR), "s"(tpb), "s"(eps), "s"(T), "s"(CW.t0), "s"(CW.t1),
               "s"(CW.row_start), "s"(CW.row_end), "s"(CW.base), "s"(CW.x), "s"(CW.x2), "s"(CW.y) : "memory");
  if ((int)blockIdx.x >= n_tiles) return;
  Tile cur, F;
  locate(blockIdx.x, CW, cur);
  FW = CW;
  F = cur;
  const uint8_t *fp = row_ptr(FW, F.r0);
  int64_t f_v = F.r0;  // SwiGLU pairs: the virtual row fp points at
  int f_left = F.nrows;
  bool f_end = false;
  auto advance_fetch = [&]() {
    if (f_end) return;
    if (--f_left > 0) {
      if constexpr (kPair) {
        fp = row_ptr(FW, ++f_v);
      } else {
        fp += rb;
      }
      return;
    }
    if (F.t + T < n_tiles) {
      locate(F.t + T, FW, F);
      fp = row_ptr(FW, F.r0);
      f_v = F.r0;
      f_left = F.nrows;
    } else {
      f_end = true;
    }
  };
  // before the ring's first copies: the loads' wait then drains nothing else
  use_pre = kPre && CW.x == x_first;
  if constexpr (kXe) {
    // the ring is free: its first copies go out once the activations are in
    // their own stage, before they are read back and normalised
    load_x(CW.x, CW.x2, std::true_type{}, [&]() {
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        issue(fp, s);
        advance_fetch();
      }
    });
  } else {
    load_x(CW.x, CW.x2, std::true_type{}, [] {});
    wait_lds_reads();  // the gather's reads of the ring are done before copies land in it
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      issue(fp, s);
      advance_fetch();
    }
  }
  use_pre = false;
  // The activations in registers are those of (x, x2): a tile of another
  // window with the same inputs keeps them (reloading would also wait for
  // every weight copy in flight, since the load counter drains in order).
  const float *cx = CW.x, *cx2 = CW.x2;
  int slot = 0;  // ring slot of the row being computed
  int parity = 0;
  for (;;) {
    if (CW.x != cx || (in_op == QG_IN_SILU_MUL && CW.x2 != cx2)) {
      load_x(CW.x, CW.x2, std::false_type{}, [] {});
      cx = CW.x;
      cx2 = CW.x2;
    }
    const int nrows = cur.nrows;
    // Alignment phase of the tile's rows: row i of the tile sits at
    // (ph0 + i * rb) mod 16 within its first granule.
    const uint32_t ph0 = (uint32_t)((uintptr_t)(CW.base + cur.r0 * rb) & 15);
    const uint32_t rb16 = (uint32_t)(rb & 15);
    float acc[NT][kGemvTileRows];
#pragma unroll
    for (int i = 0; i < kGemvTileRows; ++i) {
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t][i] = 0.0f;
      if (i < nrows) {
        // The slot NB ahead held the previous row, whose LDS reads are done.
        int s2 = slot + NB;
        s2 = s2 >= NS ? s2 - NS : s2;
        wait_lds_reads();
        issue(fp, s2);
        advance_fetch();
        wait_vmcnt<V * NB>();  // this row's copies have landed
        const uint8_t *sb = &ring[wave][slot][0];
        int ph;
        if constexpr (kPair) {
          ph = (int)((uintptr_t)row_ptr(CW, cur.r0 + i) & 15);
        } else {
          ph = (int)((ph0 + (uint32_t)i * rb16) & 15);
        }
        float part[NT];
        row_partial<FMT, C, NT>(sb, ph, lane, slice_n, xr, xs, part);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t][i] = wave_sum63(part[t]);
        slot = slot + 1 == NS ? 0 : slot + 1;
      }
    }
    constexpr bool gelu_out = op_gelu(OP);
    if constexpr (kPair) {
      // tiles start at even virtual rows and hold whole pairs
      float *yt = CW.y + ((cur.r0 - CW.row_start) >> 1);
      const int npair = nrows >> 1;
      if (WT == 1) {
        if (lane == 63) {
#pragma unroll
          for (int j = 0; j < kGemvTileRows / 2; ++j)
            if (j < npair) yt[j] = silu_times(acc[0][2 * j], acc[0][2 * j + 1]);
        }
      } else {
        if (lane == 63) {
#pragma unroll
          for (int i = 0; i < kGemvTileRows; ++i) red[parity][wave][i] = acc[0][i];
        }
        __syncthreads();
        if ((int)threadIdx.x < npair) {
          const int j = threadIdx.x;
          float g = red[parity][0][2 * j], u = red[parity][0][2 * j + 1];
#pragma unroll
          for (int v = 1; v < WT; ++v) {
            g += red[parity][v][2 * j];
            u += red[parity][v][2 * j + 1];
          }
          yt[j] = silu_times(g, u);
        }
        parity ^= 1;
      }
      if (cur.t + T >= n_tiles) break;
      locate(cur.t + T, CW, cur);
      continue;
    }
    float *yt = CW.y + (cur.r0 - CW.row_start);
    if (WT == 1) {
      if (lane == 63) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < kGemvTileRows; ++i)
            if (i < nrows) yt[t * a.y_stride + i] = gelu_out ? gelu_erf(acc[t][i]) : acc[t][i];
      }
    } else {
      if (lane == 63) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < kGemvTileRows; ++i) red[parity][wave][t * kGemvTileRows + i] = acc[t][i];
      }
      __syncthreads();
      if constexpr (NT == 1) {
        if ((int)threadIdx.x < nrows) {
          float s = red[parity][0][threadIdx.x];
#pragma unroll
          for (int v = 1; v < WT; ++v) s += red[parity][v][threadIdx.x];
          yt[threadIdx.x] = gelu_out ? gelu_erf(s) : s;
        }
      } else {
        // thread t * kGemvTileRows + i stores token t's row i (64 WT >= 8 NT)
        const int t = (int)threadIdx.x / kGemvTileRows, i = (int)threadIdx.x % kGemvTileRows;
        if (t < NT && i < nrows) {
          float s = red[parity][0][threadIdx.x];
#pragma unroll
          for (int v = 1; v < WT; ++v) s += red[parity][v][threadIdx.x];
          yt[t * a.y_stride + i] = s;
        }
      }
      parity ^= 1;
    }
    if (cur.t + T >= n_tiles) break;
    locate(cur.t + T, CW, cur);
  }
  // The ring's last copies (re-reads past the end) must land before the
  // workgroup's LDS is released.
  wait_vmcnt<0>();
}

// Team shape (WT waves, C block columns per lane), a function of (format, k).
struct Shape { int wt, c; };

typedef void (*GemvFn)(const float *, int32_t, int32_t, GemvArgs);

template <int FMT, int C, int OP, int... WT>
GemvFn pick_wt(int wt, std::integer_sequence<int, WT...>) {
  GemvFn fn = nullptr;
  ((wt == WT + 1 ? (fn = gemv_kernel<FMT, WT + 1, C, OP>, 0) : 0), ...);
  return fn;
}

template <int FMT, int OP>
GemvFn pick_fmt(Shape s) {
  if (s.c == 1) return pick_wt<FMT, 1, OP>(s.wt, std::make_integer_sequence<int, kMaxWT>{});
  return pick_wt<FMT, 2, OP>(s.wt, std::make_integer_sequence<int, kMaxWT>{});
}

// Several tokens per launch, sized by the activation registers (32 per token
// and column): four tokens with one column per lane and teams of at most 8
// waves (two waves per SIMD), two tokens with one column and any team or two
// columns and at most 8 waves; 0 = no kernel.
__host__ __device__ constexpr int batch_max_wt(int nt, int c) {
  return nt == 4 ? (c == 1 ? 8 : 0) : nt == 2 ? (c == 1 ? kMaxWT : 8) : kMaxWT;
}

template <int FMT, int C, int NT, int... WT>
GemvFn pick_wt_batch(int wt, std::integer_sequence<int, WT...>) {
  GemvFn fn = nullptr;
  ((wt == WT + 1 ? (fn = gemv_kernel<FMT, WT + 1, C, kOpNone, NT>, 0) : 0), ...);
  return fn;
}

template <int FMT, int NT>
GemvFn pick_fmt_batch(Shape s) {
  constexpr int M1 = batch_max_wt(NT, 1), M2 = batch_max_wt(NT, 2);
  if (s.c == 1 && s.wt <= M1) return pick_wt_batch<FMT, 1, NT>(s.wt, std::make_integer_sequence<int, M1>{});
  if constexpr (M2 > 0) {
    if (s.c == 2 && s.wt <= M2) return pick_wt_batch<FMT, 2, NT>(s.wt, std::make_integer_sequence<int, M2>{});
  }
  return nullptr;
}

template <int NT>
GemvFn pick_batch(int32_t fmt, Shape s) {
  switch (fmt) {
    case QG_Q8_0: return pick_fmt_batch<QG_Q8_0, NT>(s);
    case QG_Q4_0: return pick_fmt_batch<QG_Q4_0, NT>(s);
    case QG_Q4_K: return pick_fmt_batch<QG_Q4_K, NT>(s);
    case QG_Q6_K: return pick_fmt_batch<QG_Q6_K, NT>(s);
    default: return pick_fmt_batch<QG_MXFP4, NT>(s);
  }
}

template <int OP>
GemvFn pick_op(int32_t fmt, Shape s) {
  switch (fmt) {
    case QG_Q8_0: return pick_fmt<QG_Q8_0, OP>(s);
    case QG_Q4_0: return pick_fmt<QG_Q4_0, OP>(s);
    case QG_Q4_K: return pick_fmt<QG_Q4_K, OP>(s);
    case QG_Q6_K: return pick_fmt<QG_Q6_K, OP>(s);
    default: return pick_fmt<QG_MXFP4, OP>(s);
  }
}

}  // namespace qgemv_detail
