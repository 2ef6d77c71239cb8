/*
 * synth.c -- seeded synthetic GGUF blocks, written straight as bytes.
 *
 * Input generation only: no decoding, no products, no value tables.  The
 * tests, the benchmark and the oracle's inputs all come from here.
 *
 * Randomness is counter-based: word i of stream s under key `seed` is
 * SplitMix64's output function applied to seed + 0x9E3779B97F4A7C15 * (1 + c),
 * c = s * 2^40 + i (Steele, Lea & Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014; the constants are those of the published
 * SplitMix64).  Block b of a matrix (b = row * blocks_per_row + column) reads
 * only its own words, so any row range can be regenerated on its own and the
 * result does not depend on the thread count.
 *
 * Distributions per block:
 *   Q8_0 : d = binary16(lo + (hi - lo) u), u uniform in [0,1) (53 bits), rounded
 *          to nearest even; optional sign from one more bit; 32 codes uniform
 *          over {-127..127} (Lemire's multiply-shift on 32-bit words).
 *   Q4_0 : d as above; 16 code bytes uniform over 0..255.
 *   MXFP4: scale byte uniform over {e_lo..e_hi}; 16 code bytes uniform.
 * and per 256-weight super-block:
 *   Q4_K : d as above, dmin = 8 d (exact: three more in the fp16 exponent);
 *          eight 6-bit sub-block scales sc uniform over 0..63, each min
 *          m = round(15 sc / 16), so that every sub-block's weights centre on
 *          zero as a quantiser's blocks do (d sc q - 8 d m ~ d sc (q - 7.5));
 *          the 16 fields packed into 12 bytes in GGUF's layout (fields 0..3
 *          in the low six bits of bytes 0..3 / 4..7, fields 4..7 as nibbles of
 *          bytes 8..11 with their top two bits in the top bits of bytes
 *          0..3 / 4..7); 128 code bytes uniform over 0..255.
 *   Q6_K : d as above (stored last); 192 low/high code bytes uniform over
 *          0..255; 16 int8 scales uniform over {-127..127}.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define SY_Q8_0 1
#define SY_Q4_0 2
#define SY_MXFP4 3
#define SY_Q4_K 4
#define SY_Q6_K 5

static inline uint64_t sm64(uint64_t seed, uint64_t s, uint64_t i) {
  uint64_t z = seed + 0x9E3779B97F4A7C15ULL * (1 + ((s << 40) + i));
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_word(uint64_t seed, uint64_t s, uint64_t i) { return sm64(seed, s, i); }

/* binary16 bits of a positive normal value (round to nearest even). */
uint16_t synth_half_bits(double v) {
  int e;
  double m = frexp(v, &e);               /* v = m 2^e, m in [0.5, 1) */
  double t = nearbyint(ldexp(m, 11));    /* 11 significant bits */
  if (t >= 2048.0) { t = 1024.0; e += 1; }
  int ex = e - 1 + 15;                   /* biased exponent of 1.xxx * 2^(e-1) */
  return (uint16_t)((ex << 10) | ((int)t - 1024));
}

static inline uint32_t bounded(uint32_t r, uint32_t n) { return (uint32_t)(((uint64_t)r * n) >> 32); }

typedef struct {
  int32_t fmt;
  uint8_t *out;
  int64_t nb_row, bb, r0, r_lo, r_hi;
  uint64_t seed;
  double lo, hi;
  int32_t random_sign, e_lo, e_hi;
} job_t;

static uint16_t draw_half(const job_t *j, uint64_t s, uint64_t b) {
  uint64_t r = sm64(j->seed, s, b);
  double u = (double)(r >> 11) * 0x1.0p-53;
  return synth_half_bits(j->lo + (j->hi - j->lo) * u);
}

static void put_half(uint8_t *p, uint16_t h) {
  p[0] = (uint8_t)(h & 0xff);
  p[1] = (uint8_t)(h >> 8);
}

static void fill_block(const job_t *j, uint64_t b, uint8_t *p) {
  /* stream 0: scale, stream 1: codes, stream 3: Q4_K's sub-block scales, stream 4: Q6_K's scales */
  if (j->fmt == SY_Q4_K) {
    uint16_t d = draw_half(j, 0, b);
    put_half(p, d);
    put_half(p + 2, (uint16_t)(d + (3 << 10)));
    uint64_t r = sm64(j->seed, 3, b);
    int sc[8], m[8];
    for (int f = 0; f < 8; ++f) {
      sc[f] = (int)((r >> (6 * f)) & 63);
      m[f] = (15 * sc[f] + 8) >> 4;
    }
    for (int f = 0; f < 4; ++f) {
      p[4 + f] = (uint8_t)((sc[f] & 63) | ((sc[f + 4] >> 4) << 6));
      p[8 + f] = (uint8_t)((m[f] & 63) | ((m[f + 4] >> 4) << 6));
      p[12 + f] = (uint8_t)((sc[f + 4] & 15) | ((m[f + 4] & 15) << 4));
    }
    for (int i = 0; i < 16; ++i) {  /* 128 code bytes */
      uint64_t w = sm64(j->seed, 1, 16 * b + i);
      memcpy(p + 16 + 8 * i, &w, 8);
    }
    return;
  }
  if (j->fmt == SY_Q6_K) {
    for (int i = 0; i < 24; ++i) {  /* 192 code bytes */
      uint64_t w = sm64(j->seed, 1, 24 * b + i);
      memcpy(p + 8 * i, &w, 8);
    }
    for (int i = 0; i < 8; ++i) {
      uint64_t w = sm64(j->seed, 4, 8 * b + i);
      p[192 + 2 * i] = (uint8_t)(int8_t)((int)bounded((uint32_t)w, 255u) - 127);
      p[193 + 2 * i] = (uint8_t)(int8_t)((int)bounded((uint32_t)(w >> 32), 255u) - 127);
    }
    put_half(p + 208, draw_half(j, 0, b));
    return;
  }
  if (j->fmt == SY_MXFP4) {
    uint32_t r = (uint32_t)sm64(j->seed, 0, b);
    p[0] = (uint8_t)(j->e_lo + bounded(r, (uint32_t)(j->e_hi - j->e_lo + 1)));
    uint64_t w0 = sm64(j->seed, 1, 2 * b), w1 = sm64(j->seed, 1, 2 * b + 1);
    memcpy(p + 1, &w0, 8);
    memcpy(p + 9, &w1, 8);
    return;
  }
  uint64_t r = sm64(j->seed, 0, b);
  double u = (double)(r >> 11) * 0x1.0p-53;
  uint16_t h = synth_half_bits(j->lo + (j->hi - j->lo) * u);
  if (j->random_sign && (sm64(j->seed, 2, b) & 1)) h |= 0x8000;
  p[0] = (uint8_t)(h & 0xff);
  p[1] = (uint8_t)(h >> 8);
  if (j->fmt == SY_Q4_0) {
    uint64_t w0 = sm64(j->seed, 1, 2 * b), w1 = sm64(j->seed, 1, 2 * b + 1);
    memcpy(p + 2, &w0, 8);
    memcpy(p + 10, &w1, 8);
  } else { /* Q8_0 */
    for (int i = 0; i < 16; ++i) {
      uint64_t w = sm64(j->seed, 1, 16 * b + i);
      p[2 + 2 * i] = (uint8_t)(int8_t)((int)bounded((uint32_t)w, 255u) - 127);
      p[3 + 2 * i] = (uint8_t)(int8_t)((int)bounded((uint32_t)(w >> 32), 255u) - 127);
    }
  }
}

static void *worker(void *arg) {
  const job_t *j = (const job_t *)arg;
  for (int64_t r = j->r_lo; r < j->r_hi; ++r) {
    uint8_t *row = j->out + (r - j->r0) * j->nb_row * j->bb;
    for (int64_t c = 0; c < j->nb_row; ++c)
      fill_block(j, (uint64_t)(r * j->nb_row + c), row + c * j->bb);
  }
  return NULL;
}

/* Rows [r0, r1) of a seeded matrix of k inputs into out ((r1-r0) rows of
 * k/32 blocks, or k/256 super-blocks).  Returns 0, or -1 on bad arguments. */
int synth_fill(int32_t fmt, uint8_t *out, int64_t k, int64_t r0, int64_t r1, uint64_t seed,
               double scale_lo, double scale_hi, int32_t random_sign, int32_t e_lo, int32_t e_hi,
               int32_t nthreads) {
  int64_t bb = fmt == SY_Q8_0 ? 34 : fmt == SY_Q4_0 ? 18 : fmt == SY_MXFP4 ? 17
             : fmt == SY_Q4_K ? 144 : fmt == SY_Q6_K ? 210 : -1;
  int64_t qk = (fmt == SY_Q4_K || fmt == SY_Q6_K) ? 256 : 32;
  if (bb < 0 || k <= 0 || k % qk || r0 < 0 || r1 < r0) return -1;
  if (fmt != SY_MXFP4 && !(scale_lo > 6.2e-5 && scale_hi > scale_lo && scale_hi < 65504.0)) return -1;
  if (fmt == SY_MXFP4 && !(0 <= e_lo && e_lo <= e_hi && e_hi <= 255)) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  int64_t n = r1 - r0;
  if (n == 0) return 0;
  if (nthreads > n) nthreads = (int32_t)n;
  job_t jobs[64];
  pthread_t th[64];
  for (int t = 0; t < nthreads; ++t) {
    job_t j = {fmt, out, k / qk, bb, r0, r0 + n * t / nthreads, r0 + n * (t + 1) / nthreads,
               seed, scale_lo, scale_hi, random_sign, e_lo, e_hi};
    jobs[t] = j;
  }
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) break;
    started = t;
  }
  worker(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  for (int t = started + 1; t < nthreads; ++t) worker(&jobs[t]);
  return 0;
}
