// gemv_mfma.hip -- the GEMV of up to 16 tokens at once on gfx950's fp32
// matrix cores (v_mfma_f32_16x16x4_f32), for the 32-weight formats.
//
// With 16 tokens the product Y = W X is a dense contraction (16 rows x 16
// tokens x k per tile), so it goes to the matrix cores; the weights are still
// read from HBM once per call and never written out decoded.  One MFMA step
// takes a 16 x 4 slice of W (operand A) and a 4 x 16 slice of X (operand B):
//   A[i][kk] sits in lane i + 16 kk, B[kk][j] in lane j + 16 kk, and the
//   16 x 16 sum D[i][j] in lane j + 16 (i / 4), register i % 4.
// A block of 32 weights is 8 steps.  Lane group g = lane / 16 owns 8 of the
// block's positions, chosen so that one aligned-enough word of the block holds
// them: Q8_0 positions 8g..8g+7 (8 code bytes), Q4_0 and MXFP4 positions
// 4g..4g+3 and 16+4g..16+4g+3 (the low and high nibbles of bytes 4g..4g+3).
// The A values are the weights themselves, scale included: d * q is exact in
// fp32 for Q8_0 and Q4_0 (an 11-bit by 8-bit product) and 2^(e-127) * E2M1 is
// a power-of-two scaling.  The products and sums are the matrix core's fp32
// arithmetic in its own order, so a token's y is within fp32 rounding of
// W x but is not bit-identical to the one-token kernels' results.
//
// Work split: a workgroup of WT waves owns RT tiles of 16 rows; its waves
// take the row blocks' 32-weight blocks in turn (wave w: blocks w, w + WT, ...)
// so that neighbouring waves read neighbouring bytes of each row, and the
// waves' partial sums are added in wave order through LDS.
#include "qgemv_impl.h"

namespace qgemv_detail {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int FMT> struct MfmaFmt;

// Each format: Raw, the lane's loaded bytes of one block (scale field and the
// lane group's code word(s)); load(); scale(), the fp32 scale; w(), the
// weight at the group's position s (0..7) as an fp32 value, scale included.

// Q8_0: fp16 d, 32 int8 codes (RAMforge README, "Milestone 5").
template <> struct MfmaFmt<QG_Q8_0> {
  static constexpr int kBytes = 34;
  struct Raw { uint32_t h; uint2 q; };
  // x offsets of the lane group's two runs of four positions
  __device__ static inline int x0(int g) { return 8 * g; }
  __device__ static inline int x1(int g) { return 8 * g + 4; }
  __device__ static inline Raw load(const uint8_t *blk, int g) {
    uint16_t hb;
    Raw r;
    __builtin_memcpy(&hb, blk, 2);
    __builtin_memcpy(&r.q, blk + 2 + 8 * g, 8);
    r.h = hb;
    return r;
  }
  __device__ static inline float scale(const Raw &r) { return __half2float(__ushort_as_half((uint16_t)r.h)); }
  template <int S> __device__ static inline float w(const Raw &r, float d) {
    return d * (float)(int8_t)((S < 4 ? r.q.x : r.q.y) >> (8 * (S & 3)));
  }
};

// Q4_0: fp16 d, 16 bytes; position j < 16 is the low nibble of byte j,
// j + 16 its high nibble; w = d (q - 8) (RAMforge README, "Milestone 5").
template <> struct MfmaFmt<QG_Q4_0> {
  static constexpr int kBytes = 18;
  struct Raw { uint32_t h, q; };
  __device__ static inline int x0(int g) { return 4 * g; }
  __device__ static inline int x1(int g) { return 16 + 4 * g; }
  __device__ static inline Raw load(const uint8_t *blk, int g) {
    uint16_t hb;
    Raw r;
    __builtin_memcpy(&hb, blk, 2);
    __builtin_memcpy(&r.q, blk + 2 + 4 * g, 4);
    r.h = hb;
    return r;
  }
  __device__ static inline float scale(const Raw &r) { return __half2float(__ushort_as_half((uint16_t)r.h)); }
  template <int S> __device__ static inline float w(const Raw &r, float d) {
    return d * (float)((int)((r.q >> (8 * (S & 3) + 4 * (S >> 2))) & 15u) - 8);
  }
};

// MXFP4: E8M0 e, 16 bytes of E2M1 codes in the Q4_0 nibble order;
// w = 2^(e-127) E2M1(q), e = 255 is NaN (neurostream README, "The idea").
template <> struct MfmaFmt<QG_MXFP4> {
  static constexpr int kBytes = 17;
  struct Raw { uint32_t e, q; };
  __device__ static inline int x0(int g) { return 4 * g; }
  __device__ static inline int x1(int g) { return 16 + 4 * g; }
  __device__ static inline Raw load(const uint8_t *blk, int g) {
    Raw r;
    __builtin_memcpy(&r.q, blk + 1 + 4 * g, 4);
    r.e = blk[0];
    return r;
  }
  // 2^(e-127) as an fp32 bit pattern: normal for e >= 1, the subnormal
  // 2^-127 for e = 0
  __device__ static inline float scale(const Raw &r) {
    return r.e == 255u ? __builtin_nanf("") : __uint_as_float(r.e ? r.e << 23 : 0x00400000u);
  }
  // E2M1 value of byte S & 3's low (S < 4) or high nibble (scale 1: exact)
  template <int S> __device__ static inline float w(const Raw &r, float sc) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.q, 1.0f, S & 3)[S >> 2] * sc;
  }
};

template <int FMT, int S, int RT>
__device__ __forceinline__ void mfma_steps(const typename MfmaFmt<FMT>::Raw (&r)[RT], const float (&sc)[RT],
                                           const float (&xv)[8], f32x4 (&acc)[RT]) {
  if constexpr (S < 8) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(MfmaFmt<FMT>::template w<S>(r[t], sc[t]), xv[S], acc[t], 0,
                                                    0, 0);
    mfma_steps<FMT, S + 1, RT>(r, sc, xv, acc);
  }
}

template <int FMT, int RT, int WT, int P>
__global__ void __launch_bounds__(64 * WT) gemv_mfma_kernel(const MfmaArgs a) {
  using F = MfmaFmt<FMT>;
  using Raw = typename F::Raw;
  __shared__ f32x4 red[WT][RT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15;  // A: tile row; B, D: token
  const int g = lane >> 4;  // lane group: the block positions of the lane
  const int nb = a.nb;
  const int64_t rb = a.row_bytes;
  const int64_t r0 = (int64_t)blockIdx.x * (16 * RT);
  const uint8_t *rowp[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    // rows past the window read its last row; their sums are not stored
    const int64_t r = min(r0 + 16 * t + i, a.n_rows - 1);
    rowp[t] = a.w + r * rb;
  }
  const bool tok = i < a.n_tok;
  const float *xp = a.x + (int64_t)(tok ? i : 0) * a.x_stride;
  const int xo0 = F::x0(g), xo1 = F::x1(g);

  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Software pipeline: the loads of round m + P are in flight while round m
  // is decoded and multiplied.  Block b of the wave's round slot is
  // wave + WT (m + p); past the row it is clamped to the last block and its
  // x and scale are zeroed (exact zeros, never 0 * NaN).
  Raw rw[P][RT];
  float4 xa[P], xb[P];
  auto fetch = [&](int m, Raw (&r)[P][RT], float4 (&u)[P], float4 (&v)[P]) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int bb = min(wave + WT * (m + p), nb - 1);
      u[p] = float4{0.0f, 0.0f, 0.0f, 0.0f};
      v[p] = float4{0.0f, 0.0f, 0.0f, 0.0f};
      if (tok) {
        __builtin_memcpy(&u[p], xp + 32 * bb + xo0, 16);
        __builtin_memcpy(&v[p], xp + 32 * bb + xo1, 16);
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) r[p][t] = F::load(rowp[t] + (int64_t)bb * F::kBytes, g);
    }
  };
  const int rounds = (nb + WT - 1) / WT;  // blocks per wave, rounded up
  fetch(0, rw, xa, xb);
  for (int m = 0; m < rounds; m += P) {
    Raw rn[P][RT];
    float4 xan[P], xbn[P];
    const bool more = m + P < rounds;
    if (more) fetch(m + P, rn, xan, xbn);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const bool ok = wave + WT * (m + p) < nb;
      const float xv[8] = {ok ? xa[p].x : 0.0f, ok ? xa[p].y : 0.0f, ok ? xa[p].z : 0.0f, ok ? xa[p].w : 0.0f,
                           ok ? xb[p].x : 0.0f, ok ? xb[p].y : 0.0f, ok ? xb[p].z : 0.0f, ok ? xb[p].w : 0.0f};
      float sc[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) sc[t] = ok ? F::scale(rw[p][t]) : 0.0f;
      mfma_steps<FMT, 0, RT>(rw[p], sc, xv, acc);
    }
    if (!more) break;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      xa[p] = xan[p];
      xb[p] = xbn[p];
#pragma unroll
      for (int t = 0; t < RT; ++t) rw[p][t] = rn[p][t];
    }
  }

  // Add the waves' sums in wave order; thread q stores token q / (16 RT),
  // tile row q % (16 RT), so consecutive threads write consecutive rows.
#pragma unroll
  for (int t = 0; t < RT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  for (int q = threadIdx.x; q < 256 * RT; q += 64 * WT) {
    const int j = q / (16 * RT), rr = q % (16 * RT);
    const int t = rr >> 4, ii = rr & 15;
    const int64_t r = r0 + rr;
    if (j < a.n_tok && r < a.n_rows) {
      const int l = j + 16 * (ii >> 2), e = ii & 3;
      float s = red[0][t][l][e];
#pragma unroll
      for (int v = 1; v < WT; ++v) s += red[v][t][l][e];
      a.y[(int64_t)j * a.y_stride + r] = s;
    }
  }
}

// Two 16-row tiles per workgroup (each x value loaded once for 32 rows), 8
// waves, 2 blocks per round: of the shapes measured on the 20B-class pass
// (1-2 tiles, 8-16 waves, 2-8 blocks per round) the fastest.
template <int FMT>
static int launch_fmt(const MfmaArgs &a, hipStream_t stream) {
  constexpr int RT = 2, WT = 8, P = 2;
  const int64_t tiles = (a.n_rows + 16 * RT - 1) / (16 * RT);
  if (tiles > 0x7fffffff) return QG_E_SHAPE;
  hipLaunchKernelGGL((gemv_mfma_kernel<FMT, RT, WT, P>), dim3((unsigned)tiles), dim3(64 * WT), 0, stream, a);
  return QG_OK;
}

int launch_gemv_mfma(int32_t fmt, const MfmaArgs &a, hipStream_t stream) {
  switch (fmt) {
    case QG_Q8_0: return launch_fmt<QG_Q8_0>(a, stream);
    case QG_Q4_0: return launch_fmt<QG_Q4_0>(a, stream);
    case QG_MXFP4: return launch_fmt<QG_MXFP4>(a, stream);
    default: return QG_E_FMT;
  }
}

}  // namespace qgemv_detail
