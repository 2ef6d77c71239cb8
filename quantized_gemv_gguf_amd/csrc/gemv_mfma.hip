// gemv_mfma.hip -- the GEMV of up to 16 tokens at once on gfx950's fp32
// matrix cores (v_mfma_f32_16x16x4_f32), for every format.
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
// take the rows' blocks in turn (the LDS kernel: chunks of kCB blocks, wave
// w: chunks w, w + WT, ...; the register kernel: single blocks), and the
// waves' partial sums are added in wave order through LDS.
#include "qgemv_impl.h"

namespace qgemv_detail {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef u32x4 __attribute__((aligned(1))) u32x4_u1;  // 16 bytes at any address

template <int FMT> struct MfmaFmt;

// Each format: Raw, the lane's loaded bytes of one block (scale field and the
// lane group's code word(s)); load(); scale(), the fp32 scale; w(), the
// weight at the group's position s (0..7) as an fp32 value, scale included.

// Q8_0: fp16 d, 32 int8 codes (RAMforge README, "Milestone 5").
template <> struct MfmaFmt<QG_Q8_0> {
  static constexpr int kBytes = 34, kCB = 8;  // kCB blocks: 17 granules of 16 bytes
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
  __device__ static inline Raw load_unit(const uint8_t *row, int c, int g) { return load(row + c * kBytes, g); }
  __device__ static inline float scale(const Raw &r) { return __half2float(__ushort_as_half((uint16_t)r.h)); }
  template <int S> __device__ static inline float w(const Raw &r, float d) {
    return d * (float)(int8_t)((S < 4 ? r.q.x : r.q.y) >> (8 * (S & 3)));
  }
};

// Q4_0: fp16 d, 16 bytes; position j < 16 is the low nibble of byte j,
// j + 16 its high nibble; w = d (q - 8) (RAMforge README, "Milestone 5").
template <> struct MfmaFmt<QG_Q4_0> {
  static constexpr int kBytes = 18, kCB = 16;  // 18 granules
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
  __device__ static inline Raw load_unit(const uint8_t *row, int c, int g) { return load(row + c * kBytes, g); }
  __device__ static inline float scale(const Raw &r) { return __half2float(__ushort_as_half((uint16_t)r.h)); }
  template <int S> __device__ static inline float w(const Raw &r, float d) {
    return d * (float)((int)((r.q >> (8 * (S & 3) + 4 * (S >> 2))) & 15u) - 8);
  }
};

// MXFP4: E8M0 e, 16 bytes of E2M1 codes in the Q4_0 nibble order;
// w = 2^(e-127) E2M1(q), e = 255 is NaN (neurostream README, "The idea").
template <> struct MfmaFmt<QG_MXFP4> {
  static constexpr int kBytes = 17, kCB = 16;  // 17 granules
  struct Raw { uint32_t e, q; };
  __device__ static inline int x0(int g) { return 4 * g; }
  __device__ static inline int x1(int g) { return 16 + 4 * g; }
  __device__ static inline Raw load(const uint8_t *blk, int g) {
    Raw r;
    __builtin_memcpy(&r.q, blk + 1 + 4 * g, 4);
    r.e = blk[0];
    return r;
  }
  __device__ static inline Raw load_unit(const uint8_t *row, int c, int g) { return load(row + c * kBytes, g); }
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

// Q4_K: 144-byte super-blocks of 8 units of 32 weights (fp16 d, fp16 dmin,
// 12 bytes of 6-bit scales and mins, 128 bytes of nibbles); unit s's weights
// are d sc_s q - dmin m_s, q the low (even s) or high (odd s) nibbles of bytes
// 32 (s / 2) .. 32 (s / 2) + 31 (RAMforge README, "Milestone 5", Q4_K line).
// Here kBytes is the bytes per unit (144 / 8), so a chunk of 8 units is one
// super-block of 9 granules; k is a multiple of 256, so no chunk is ever
// moved back and every unit's gate is 1.  The weight d sc q - dmin m is one
// fused multiply-add of exact products, rounded once, as the oracle's.
template <> struct MfmaFmt<QG_Q4_K> {
  static constexpr int kBytes = 18, kCB = 8;
  struct Raw { uint2 q; float dsc, dm; uint32_t sh; };
  __device__ static inline int x0(int g) { return 8 * g; }
  __device__ static inline int x1(int g) { return 8 * g + 4; }
  __device__ static inline Raw load_unit(const uint8_t *row, int c, int g) {
    const uint8_t *sb = row + (c >> 3) * 144;
    const int s = c & 7;
    int sc, m;
    Fmt<QG_Q4_K>::scale_min(sb, s, sc, m);
    uint16_t hd, hm;
    __builtin_memcpy(&hd, sb, 2);
    __builtin_memcpy(&hm, sb + 2, 2);
    Raw r;
    r.dsc = __half2float(__ushort_as_half(hd)) * (float)sc;
    r.dm = __half2float(__ushort_as_half(hm)) * (float)m;
    __builtin_memcpy(&r.q, sb + 16 + 32 * (s >> 1) + 8 * g, 8);
    r.sh = 4u * (uint32_t)(s & 1);
    return r;
  }
  __device__ static inline float scale(const Raw &) { return 1.0f; }
  template <int S> __device__ static inline float w(const Raw &r, float gate) {
    const float q = (float)(((S < 4 ? r.q.x : r.q.y) >> (8 * (S & 3) + r.sh)) & 15u);
    return gate * fmaf(r.dsc, q, -r.dm);
  }
};

// Q6_K: 210-byte super-blocks (128 bytes of low nibbles ql, 64 of high bit
// pairs qh, 16 int8 scales, fp16 d); element e's code is the nibble of
// ql[64 h + 32 (i % 2) + l] at 4 (i / 2) with the bit pair of qh[32 h + l] at
// 2 i above it (h = e / 128, i = e % 128 / 32, l = e % 32), and its weight
// d scale[e / 16] (q - 32), exact in fp32 (11 + 7 + 6 significant bits).
// A lane group's 8 positions of a unit lie in one scale's run of 16 and read
// 8 consecutive bytes of ql and of qh.  210-byte blocks are no whole number
// of granules per chunk, so Q6_K takes the register kernel.
template <> struct MfmaFmt<QG_Q6_K> {
  static constexpr int kBytes = 210, kCB = 0;
  struct Raw { uint2 ql, qh; float dsc; uint32_t shl, shh; };
  __device__ static inline int x0(int g) { return 8 * g; }
  __device__ static inline int x1(int g) { return 8 * g + 4; }
  __device__ static inline Raw load_unit(const uint8_t *row, int u, int g) {
    const uint8_t *sb = row + (int64_t)(u >> 3) * 210;
    const int uu = u & 7, h = uu >> 2, i = uu & 3;
    Raw r;
    __builtin_memcpy(&r.ql, sb + 64 * h + 32 * (i & 1) + 8 * g, 8);
    __builtin_memcpy(&r.qh, sb + 128 + 32 * h + 8 * g, 8);
    uint16_t hd;
    __builtin_memcpy(&hd, sb + 208, 2);
    r.dsc = __half2float(__ushort_as_half(hd)) * (float)(int8_t)sb[192 + 2 * uu + (g >> 1)];
    r.shl = 4u * (uint32_t)(i >> 1);
    r.shh = 2u * (uint32_t)i;
    return r;
  }
  __device__ static inline float scale(const Raw &r) { return r.dsc; }
  template <int S> __device__ static inline float w(const Raw &r, float dsc) {
    const uint32_t lo = ((S < 4 ? r.ql.x : r.ql.y) >> (8 * (S & 3) + r.shl)) & 15u;
    const uint32_t hi = ((S < 4 ? r.qh.x : r.qh.y) >> (8 * (S & 3) + r.shh)) & 3u;
    return dsc * (float)((int)(lo | (hi << 4)) - 32);
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
      for (int t = 0; t < RT; ++t) r[p][t] = F::load_unit(rowp[t], bb, g);
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

// The same product with the weights staged through LDS.  A wave's k range
// is a run of chunks of kCB blocks (wave w: chunks w, w + WT, ...); a chunk
// of one row is GR 16-byte granules, and the wave reads its 16 RT rows' chunk
// with contiguous 16-byte loads (lane l of load v: granule 64 v + l, in row
// order), so each load instruction covers whole cache lines.  The granules
// land in the wave's own LDS region (row stride an odd number of granules,
// so the 16 rows of a tile fall in distinct banks) and the lanes read their
// MFMA operands back from there; the next chunk's loads are in flight while
// the current chunk is multiplied, and each block's x two blocks ahead.
template <int FMT, int RT, int WT>
__global__ void __launch_bounds__(64 * WT) gemv_mfma_lds_kernel(const MfmaArgs a) {
  using F = MfmaFmt<FMT>;
  using Raw = typename F::Raw;
  constexpr int CB = F::kCB;
  constexpr int CBYTES = CB * F::kBytes;  // bytes of a row's chunk
  static_assert(CBYTES % 16 == 0, "a row's chunk is whole granules");
  constexpr int GR = CBYTES / 16;         // granules per row's chunk
  constexpr int GRP = GR | 1;             // LDS row stride in granules
  constexpr int ROWS = 16 * RT;
  constexpr int NG = ROWS * GR;           // granules per chunk
  constexpr int NV = (NG + 63) / 64;      // loads per lane per chunk
  constexpr int STAGE = ROWS * GRP * 16;  // LDS bytes per wave
  constexpr int RED = WT * RT * 64 * 16;  // the final reduction's bytes
  __shared__ __attribute__((aligned(16))) uint8_t lds[(WT * STAGE > RED) ? WT * STAGE : RED];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15;  // A: tile row; B, D: token
  const int g = lane >> 4;  // lane group: the block positions of the lane
  const int nb = a.nb;
  const int64_t rb = a.row_bytes;
  const int64_t r0 = (int64_t)blockIdx.x * ROWS;
  uint8_t *stage = lds + wave * STAGE;

  // This lane's granules of every chunk: row base and offset within the
  // chunk, and the LDS slot.  Rows past the window read its last row.
  const uint8_t *gbase[NV];
  uint32_t goff[NV], gslot[NV];
  bool gon[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int G = 64 * v + lane;
    const int row = G / GR, q = G - (G / GR) * GR;
    // (a lane past the chunk's granules loads granule 0 and stores nothing)
    gon[v] = G < NG;
    gbase[v] = a.w + min(r0 + (gon[v] ? row : 0), a.n_rows - 1) * rb;
    goff[v] = gon[v] ? 16u * (uint32_t)q : 0u;  // + 16 <= CBYTES
    gslot[v] = 16u * (uint32_t)(row * GRP + q);
  }
  // Chunk c holds blocks [CB c, CB c + CB) of the row; the last one, when nb
  // is not a multiple of CB, is moved back to end at the row's end (nb >= CB:
  // the host's choice), so every load stays inside the row, and its blocks
  // below CB c, counted in the chunk before, are zeroed.
  const int nch = (nb + CB - 1) / CB;            // chunks of the row
  const int mine = nch > wave ? (nch - wave + WT - 1) / WT : 0;  // this wave's chunks
  auto chunk_base = [&](int c) { return min(CB * c, nb - CB); };
  u32x4 gr[NV];
  auto fetch = [&](int c) {
    const int64_t off = (int64_t)chunk_base(c) * F::kBytes;
#pragma unroll
    for (int v = 0; v < NV; ++v) gr[v] = *reinterpret_cast<const u32x4_u1 *>(gbase[v] + off + goff[v]);
  };
  const bool tok = i < a.n_tok;
  const float *xp = a.x + (int64_t)(tok ? i : 0) * a.x_stride;
  const int xo0 = F::x0(g), xo1 = F::x1(g);
  // x of the wave's u-th block (u counts blocks over the wave's chunks; past
  // its last chunk, zeros)
  auto xload = [&](int u, float (&xv)[8]) {
    const int c = wave + WT * (u / CB);
    const int bb = chunk_base(c) + (u % CB);
    const bool ok = bb >= CB * c && tok;
    float4 p = float4{0.0f, 0.0f, 0.0f, 0.0f}, q = float4{0.0f, 0.0f, 0.0f, 0.0f};
    if (tok) {
      __builtin_memcpy(&p, xp + 32 * bb + xo0, 16);
      __builtin_memcpy(&q, xp + 32 * bb + xo1, 16);
    }
    xv[0] = ok ? p.x : 0.0f;
    xv[1] = ok ? p.y : 0.0f;
    xv[2] = ok ? p.z : 0.0f;
    xv[3] = ok ? p.w : 0.0f;
    xv[4] = ok ? q.x : 0.0f;
    xv[5] = ok ? q.y : 0.0f;
    xv[6] = ok ? q.z : 0.0f;
    xv[7] = ok ? q.w : 0.0f;
  };

  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  if (mine > 0) {
    float xr[4][8];  // x ring: block u in slot u % 4 (CB is a multiple of 4)
    fetch(wave);
    xload(0, xr[0]);
    xload(1, xr[1]);
    for (int n = 0; n < mine; ++n) {
      // chunk n's granules to LDS (the previous chunk's reads are done: one
      // wave's LDS operations complete in order), then chunk n + 1's loads
#pragma unroll
      for (int v = 0; v < NV; ++v)
        if (gon[v]) *reinterpret_cast<u32x4 *>(stage + gslot[v]) = gr[v];
      if (n + 1 < mine) fetch(wave + WT * (n + 1));
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const int u = CB * n + c;
        xload(u + 2, xr[(c + 2) & 3]);
        const int cw = wave + WT * n;
        const bool ok = chunk_base(cw) + c >= CB * cw;
        Raw rw[RT];
        float sc[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          rw[t] = F::load_unit(stage + (16 * t + i) * (GRP * 16), c, g);
          sc[t] = ok ? F::scale(rw[t]) : 0.0f;
        }
        mfma_steps<FMT, 0, RT>(rw, sc, xr[c & 3], acc);
      }
    }
  }

  // Add the waves' sums in wave order (the staging area is reused);
  // thread q stores token q / (16 RT), tile row q % (16 RT), so consecutive
  // threads write consecutive rows.
  __syncthreads();
  f32x4 *red = reinterpret_cast<f32x4 *>(lds);  // [WT][RT][64]
#pragma unroll
  for (int t = 0; t < RT; ++t) red[(wave * RT + t) * 64 + lane] = acc[t];
  __syncthreads();
  for (int q = threadIdx.x; q < 256 * RT; q += 64 * WT) {
    const int j = q / (16 * RT), rr = q % (16 * RT);
    const int t = rr >> 4, ii = rr & 15;
    const int64_t r = r0 + rr;
    if (j < a.n_tok && r < a.n_rows) {
      const int l = j + 16 * (ii >> 2), e = ii & 3;
      float s = red[t * 64 + l][e];
#pragma unroll
      for (int v = 1; v < WT; ++v) s += red[(v * RT + t) * 64 + l][e];
      a.y[(int64_t)j * a.y_stride + r] = s;
    }
  }
}

// Launch shape: two 16-row tiles per workgroup (each x value loaded once for
// 32 rows) and 8 waves; of the shapes measured on the 20B-class pass (1-2
// tiles, 4-16 waves, with and without LDS staging) the fastest.  A matrix
// shorter than one chunk (k < 32 kCB), and Q6_K, take the register kernel.
template <int FMT>
static int launch_fmt(const MfmaArgs &a, hipStream_t stream) {
  constexpr int RT = 2, WT = 8;
  const int64_t tiles = (a.n_rows + 16 * RT - 1) / (16 * RT);
  if (tiles > 0x7fffffff) return QG_E_SHAPE;
  if constexpr (FMT == QG_Q6_K) {
    hipLaunchKernelGGL((gemv_mfma_kernel<FMT, RT, WT, 2>), dim3((unsigned)tiles), dim3(64 * WT), 0, stream, a);
  } else {
    if (a.nb >= MfmaFmt<FMT>::kCB) {
      hipLaunchKernelGGL((gemv_mfma_lds_kernel<FMT, RT, WT>), dim3((unsigned)tiles), dim3(64 * WT), 0, stream, a);
    } else if constexpr (FMT != QG_Q4_K) {  // (a Q4_K row is at least one chunk)
      hipLaunchKernelGGL((gemv_mfma_kernel<FMT, RT, WT, 2>), dim3((unsigned)tiles), dim3(64 * WT), 0, stream, a);
    }
  }
  return QG_OK;
}

int launch_gemv_mfma(int32_t fmt, const MfmaArgs &a, hipStream_t stream) {
  switch (fmt) {
    case QG_Q8_0: return launch_fmt<QG_Q8_0>(a, stream);
    case QG_Q4_0: return launch_fmt<QG_Q4_0>(a, stream);
    case QG_MXFP4: return launch_fmt<QG_MXFP4>(a, stream);
    case QG_Q4_K: return launch_fmt<QG_Q4_K>(a, stream);
    case QG_Q6_K: return launch_fmt<QG_Q6_K>(a, stream);
    default: return QG_E_FMT;
  }
}

}  // namespace qgemv_detail
