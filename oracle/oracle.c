/*
 * oracle.c -- plain, slow, scalar CPU oracle for the batch-1 dequant-GEMV over
 * GGUF block-quantized weights (Q8_0, Q4_0, MXFP4, Q4_K, Q6_K).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only the test suite, the package's smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no header, constant, table or helper
 * with the HIP library; every format fact below is restated here from the pages.
 *
 * What it computes (all sums in fp64, sequential in the column index):
 *
 *   y[j] = sum_{i<K} dec(W)[row_start + j, i] * x[i],   j < row_end - row_start
 *
 * with W stored row-major as [n_rows][K/QK blocks] (QK = 32 weights per
 * block; 256 for the K-quants) -- the GGML/GGUF matrix
 * convention that RAMforge's README states under "Milestone 6 - True
 * Out-of-Core Integrity" (shape [in, out], buffer [out][in], y[o] = sum_i
 * W[o*in + i] * x[i]).  Each row is a whole number of quantization blocks
 * (neurostream README, "The idea"), so a row window is one contiguous byte
 * range and rows are independent.
 *
 * Block formats (RAMforge README, "Milestone 5 - Native Quantized Tensor
 * Support"):
 *   Q8_0 : 34 bytes = fp16 scale d, then 32 int8 q;           w = d * q
 *   Q4_0 : 18 bytes = fp16 scale d, then 16 bytes of nibbles;  w = d * (q - 8)
 * MXFP4 (neurostream README, "The idea": one 2,880-row expert of 2,880 inputs
 * is 4.41 MB, i.e. 17 bytes per 32 weights; GPT-OSS's expert format):
 *   MXFP4: 17 bytes = E8M0 scale byte e, then 16 bytes of E2M1 nibbles;
 *          w = 2^(e-127) * E2M1(code)
 *
 * K-quants, 256-weight super-blocks of eight 32-weight sub-blocks:
 *   Q4_K : 144 bytes = fp16 d, fp16 dmin, 12 bytes holding eight 6-bit
 *          sub-block scales sc and eight 6-bit mins m, 128 bytes of nibbles;
 *          w = d * sc * q - dmin * m  (RAMforge README, "Milestone 5", Q4_K)
 *   Q6_K : 210 bytes = 128 bytes of low nibbles, 64 bytes of 2-bit high
 *          parts, sixteen int8 scales (one per 16 weights), fp16 d;
 *          w = d * scale * (q - 32), q the 6-bit code (named by RAMforge README
 *          "Milestone 5" and neurostream README "Supported"; the pages print
 *          no layout for it)
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *   - nibble order: element j (j < 16) is the low nibble of qs[j], element
 *     j + 16 is the high nibble of qs[j] (the GGUF split-half order);
 *   - E2M1 is the OCP MX 4-bit float: 1 sign bit (bit 3), 2 exponent bits
 *     (bias 1), 1 mantissa bit; E8M0 is a bare biased exponent 2^(e-127) with
 *     e = 255 meaning NaN;
 *   - the fp16 scale is IEEE binary16, decoded here from its bit fields;
 *   - K-quant byte layouts are GGUF's (neurostream states its K-quant decode
 *     is bit-exact against the reference gguf implementation): in Q4_K,
 *     sub-block j < 4 takes scale = low 6 bits of scale byte j and min = low
 *     6 bits of byte j + 4; j >= 4 takes scale = low nibble of byte j + 4 with
 *     the top 2 bits of byte j - 4 above it, min = high nibble of byte j + 4
 *     with the top 2 bits of byte j above it; nibble byte 32 c + l holds
 *     element l of sub-block 2 c (low nibble) and of sub-block 2 c + 1 (high).
 *     In Q6_K, element e = 128 h + 32 i + l (l < 32) takes the nibble
 *     (i < 2 ? low : high) of low byte 64 h + 32 (i & 1) + l, bits 2 i, 2 i + 1
 *     of high byte 32 h + l as its top two bits, and scale e / 16.
 *
 * Every decoded weight of the 32-weight formats is exactly representable in
 * fp32 for finite scales (an fp16 has 11 significant bits, |q| <= 128 adds 8;
 * E2M1 values have 2).  K-quant weights are exact in fp64 and rounded once to
 * fp32 (Q4_K: d sc q and dmin m are exact, their difference is not always;
 * Q6_K: d scale (q - 32) can need 25 bits).  The decoder returns fp32 and the
 * dot product multiplies those fp32 values by the fp32 x in fp64, where each
 * product is exact.
 *
 * Threads split rows only; each row's sum is the same sequence of fp64
 * operations whatever the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Format identifiers: the same small integers the boundary uses, restated. */
#define ORC_Q8_0 1
#define ORC_Q4_0 2
#define ORC_MXFP4 3
#define ORC_Q4_K 4
#define ORC_Q6_K 5

#define ORC_OK 0
#define ORC_EBAD (-1)

int64_t orc_block_bytes(int32_t fmt) {
  switch (fmt) {
    case ORC_Q8_0: return 2 + 32;   /* fp16 d + 32 x int8 */
    case ORC_Q4_0: return 2 + 16;   /* fp16 d + 32 nibbles */
    case ORC_MXFP4: return 1 + 16;  /* E8M0 e + 32 nibbles */
    case ORC_Q4_K: return 2 + 2 + 12 + 128;  /* d, dmin, packed scales/mins, 256 nibbles */
    case ORC_Q6_K: return 128 + 64 + 16 + 2; /* low nibbles, high bit pairs, scales, d */
    default: return ORC_EBAD;
  }
}

/* Weights per block. */
int64_t orc_block_weights(int32_t fmt) {
  if (orc_block_bytes(fmt) < 0) return ORC_EBAD;
  return (fmt == ORC_Q4_K || fmt == ORC_Q6_K) ? 256 : 32;
}

int64_t orc_row_bytes(int32_t fmt, int64_t k) {
  int64_t bb = orc_block_bytes(fmt), qk = orc_block_weights(fmt);
  if (bb < 0 || k <= 0 || k % qk != 0) return ORC_EBAD;
  return (k / qk) * bb;
}

/* IEEE 754 binary16 -> double, from the bit fields (no host half type). */
double orc_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int exp = (h >> 10) & 0x1f;
  int man = h & 0x3ff;
  double v;
  if (exp == 0) {
    v = ldexp((double)man, -24);             /* zero or subnormal: man * 2^-24 */
  } else if (exp == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + man), exp - 25); /* (1 + man/1024) * 2^(exp-15) */
  }
  return sign ? -v : v;
}

void orc_half_to_double_n(const uint16_t *h, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_half_to_double(h[i]);
}

/* OCP MX E2M1 code (0..15) -> value, from its fields. */
static double e2m1_value(int code) {
  int s = (code >> 3) & 1;
  int e = (code >> 1) & 3;
  int m = code & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* E8M0 scale byte -> value. */
static double e8m0_value(int e) {
  if (e == 255) return NAN;
  return ldexp(1.0, e - 127);
}

/* Q4_K's twelve scale bytes -> the 6-bit scale sc[j] and min m[j] of each
 * sub-block j: the first four sub-blocks keep both fields whole in the low six
 * bits of bytes 0..7; the last four keep their low four bits in the nibbles
 * of bytes 8..11 and their top two bits in the spare top bits of bytes 0..7. */
static void q4_k_scales_mins(const uint8_t s[12], int sc[8], int m[8]) {
  for (int j = 0; j < 4; ++j) {
    sc[j] = s[j] & 63;
    m[j] = s[j + 4] & 63;
  }
  for (int j = 4; j < 8; ++j) {
    sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
    m[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
  }
}

/* One Q4_K super-block into 256 weights. */
static void decode_q4_k(const uint8_t *b, float w[256]) {
  double d = orc_half_to_double((uint16_t)(b[0] | (b[1] << 8)));
  double dmin = orc_half_to_double((uint16_t)(b[2] | (b[3] << 8)));
  int sc[8], m[8];
  q4_k_scales_mins(b + 4, sc, m);
  const uint8_t *qs = b + 16;
  for (int j = 0; j < 8; ++j) {
    for (int l = 0; l < 32; ++l) {
      int byte = qs[32 * (j / 2) + l];
      int q = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
      w[32 * j + l] = (float)(d * sc[j] * q - dmin * m[j]);
    }
  }
}

/* One Q6_K super-block into 256 weights. */
static void decode_q6_k(const uint8_t *b, float w[256]) {
  const uint8_t *ql = b, *qh = b + 128;
  const int8_t *scale = (const int8_t *)(b + 192);
  double d = orc_half_to_double((uint16_t)(b[208] | (b[209] << 8)));
  for (int e = 0; e < 256; ++e) {
    int h = e / 128, i = (e % 128) / 32, l = e % 32;
    int low = (ql[64 * h + 32 * (i % 2) + l] >> (4 * (i / 2))) & 15;
    int high = (qh[32 * h + l] >> (2 * i)) & 3;
    int q = low | (high << 4);
    w[e] = (float)(d * scale[e / 16] * (q - 32));
  }
}

/* Decode one block into its 32 (or 256) fp32 weights, in element order. */
static void decode_block(int32_t fmt, const uint8_t *b, float *w) {
  if (fmt == ORC_Q4_K) {
    decode_q4_k(b, w);
  } else if (fmt == ORC_Q6_K) {
    decode_q6_k(b, w);
  } else if (fmt == ORC_Q8_0) {
    double d = orc_half_to_double((uint16_t)(b[0] | (b[1] << 8)));
    for (int j = 0; j < 32; ++j) w[j] = (float)(d * (double)(int8_t)b[2 + j]);
  } else if (fmt == ORC_Q4_0) {
    double d = orc_half_to_double((uint16_t)(b[0] | (b[1] << 8)));
    for (int j = 0; j < 16; ++j) {
      int lo = b[2 + j] & 0x0f;
      int hi = b[2 + j] >> 4;
      w[j] = (float)(d * (double)(lo - 8));
      w[j + 16] = (float)(d * (double)(hi - 8));
    }
  } else { /* ORC_MXFP4 */
    double s = e8m0_value(b[0]);
    for (int j = 0; j < 16; ++j) {
      int lo = b[1 + j] & 0x0f;
      int hi = b[1 + j] >> 4;
      w[j] = (float)(s * e2m1_value(lo));
      w[j + 16] = (float)(s * e2m1_value(hi));
    }
  }
}

static int check_args(int32_t fmt, int64_t n_rows, int64_t k, int64_t r0, int64_t r1) {
  if (orc_row_bytes(fmt, k) < 0) return ORC_EBAD;
  if (n_rows < 0 || r0 < 0 || r0 > r1 || r1 > n_rows) return ORC_EBAD;
  return ORC_OK;
}

/* Decoded fp32 weights of rows [r0, r1): out is (r1 - r0) x k, row-major. */
int orc_dequant_rows(int32_t fmt, const uint8_t *w, int64_t n_rows, int64_t k,
                     int64_t r0, int64_t r1, float *out) {
  if (check_args(fmt, n_rows, k, r0, r1) != ORC_OK) return ORC_EBAD;
  int64_t bb = orc_block_bytes(fmt), rb = orc_row_bytes(fmt, k), qk = orc_block_weights(fmt), nb = k / qk;
  for (int64_t r = r0; r < r1; ++r)
    for (int64_t b = 0; b < nb; ++b)
      decode_block(fmt, w + r * rb + b * bb, out + (r - r0) * k + b * qk);
  return ORC_OK;
}

/* One row: y = sum_i w_i * x_i and a = sum_i |w_i * x_i| (the second is the
 * scale a componentwise error bound is measured against). */
static void gemv_row(int32_t fmt, const uint8_t *row, int64_t k, const float *x,
                     double *y, double *a) {
  int64_t bb = orc_block_bytes(fmt), qk = orc_block_weights(fmt), nb = k / qk;
  float w[256];
  double acc = 0.0, aacc = 0.0;
  for (int64_t b = 0; b < nb; ++b) {
    decode_block(fmt, row + b * bb, w);
    for (int j = 0; j < qk; ++j) {
      double p = (double)w[j] * (double)x[b * qk + j];
      acc += p;
      aacc += fabs(p);
    }
  }
  *y = acc;
  if (a) *a = aacc;
}

typedef struct {
  int32_t fmt;
  const uint8_t *w;
  int64_t k, rb, r_lo, r_hi, r0;
  const float *x;
  double *y, *a;
} gemv_job;

static void *gemv_worker(void *p) {
  gemv_job *j = (gemv_job *)p;
  for (int64_t r = j->r_lo; r < j->r_hi; ++r)
    gemv_row(j->fmt, j->w + r * j->rb, j->k, j->x, j->y + (r - j->r0),
             j->a ? j->a + (r - j->r0) : NULL);
  return NULL;
}

/* y[j] (and a[j] if a != NULL) for rows [r0, r1), split over nthreads. */
int orc_gemv_rows(int32_t fmt, const uint8_t *w, int64_t n_rows, int64_t k,
                  int64_t r0, int64_t r1, const float *x, double *y, double *a,
                  int32_t nthreads) {
  if (check_args(fmt, n_rows, k, r0, r1) != ORC_OK) return ORC_EBAD;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  int64_t rb = orc_row_bytes(fmt, k), n = r1 - r0;
  if (n == 0) return ORC_OK;
  if (nthreads > n) nthreads = (int32_t)n;
  pthread_t th[256];
  gemv_job jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].fmt = fmt; jobs[t].w = w; jobs[t].k = k; jobs[t].rb = rb;
    jobs[t].r_lo = r0 + n * t / nthreads;
    jobs[t].r_hi = r0 + n * (t + 1) / nthreads;
    jobs[t].r0 = r0; jobs[t].x = x; jobs[t].y = y; jobs[t].a = a;
  }
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, gemv_worker, &jobs[t]) != 0) break;
    started = t;
  }
  gemv_worker(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  for (int t = started + 1; t < nthreads; ++t) gemv_worker(&jobs[t]);
  return ORC_OK;
}

/* h = silu(g) * u, silu(g) = g / (1 + exp(-g)), in fp64 (the between-phase
 * activation of a SwiGLU FFN: hipfire PR "Design notes" runs it as a GPU
 * elementwise step; neurostream "How it works" materialises it between the
 * row-contiguous gate/up and down phases). */
void orc_silu_mul(const double *g, const double *u, double *h, int64_t n) {
  for (int64_t i = 0; i < n; ++i) h[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}

/* Carry step of the synthetic dense decode pass: optional exact GELU
 * (0.5 v (1 + erf(v / sqrt 2)), GPT-NeoX's activation), then RMS
 * normalisation v / sqrt(mean(v^2) + eps) with no gain.  The GELU is written
 * with erfc, since 1 + erf(z) = erfc(-z) exactly: erfc keeps its relative
 * accuracy for v far below 0, where 1 + erf cancels to nothing. */
void orc_rms_carry(const double *v, double *out, int64_t n, double eps, int32_t gelu) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double t = gelu ? 0.5 * v[i] * erfc(-v[i] / sqrt(2.0)) : v[i];
    out[i] = t;
    ss += t * t;
  }
  double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) out[i] *= inv;
}

/* Router-weighted combine of per-expert outputs: out[i] = sum_s w[s] *
 * y[s * y_stride + i], in fp64 (neurostream README, "How it works": the
 * router's active experts are mixed back into one vector). */
void orc_combine(const double *y, int64_t y_stride, int32_t n_sel, const double *w, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) {
    double acc = 0.0;
    for (int32_t s = 0; s < n_sel; ++s) acc += w[s] * y[s * y_stride + i];
    out[i] = acc;
  }
}
