/*
 * qgemv.h -- C ABI of libqgemv.so: batch-1 dequant-GEMV over GGUF
 * block-quantized weights (Q8_0, Q4_0, MXFP4, Q4_K, Q6_K) on an AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (RAMforge README, "Milestone 6 - True Out-of-Core Integrity",
 * matrix layout): a weight matrix of n_rows output rows and k inputs is stored
 * row-major, [n_rows][k/QK blocks], each row a whole number of quant blocks
 * (neurostream README, "The idea"; QK = 32 weights per block, 256 for the
 * K-quant super-blocks), and
 *
 *     y[j] = sum_{i<k} W[row_start + j, i] * x[i],   0 <= j < row_end - row_start
 *
 * with every block dequantized in registers and never written out, fp32
 * activations and fp32 accumulation.
 *
 * Block formats (RAMforge README, "Milestone 5 - Native Quantized Tensor
 * Support"; MXFP4 from neurostream README, "The idea", 4.41 MB per 2,880 x 2,880
 * expert = 17 bytes per 32 weights):
 *   QG_Q8_0  34 B: fp16 d, int8 q[32];              w_j = d * q_j
 *   QG_Q4_0  18 B: fp16 d, uint8 qs[16];            w_j = d * (nib_j - 8)
 *   QG_MXFP4 17 B: uint8 e (E8M0), uint8 qs[16];    w_j = 2^(e-127) * E2M1(nib_j)
 * Nibble order: element j < 16 is the low nibble of qs[j], element j + 16 the
 * high nibble (the GGUF split-half order).  E2M1 is the OCP MX 4-bit float
 * (sign bit 3, two exponent bits with bias 1, one mantissa bit); e = 255 is NaN.
 *
 * K-quants: 256-weight super-blocks of eight 32-weight sub-blocks, in GGUF's
 * byte layout (neurostream README, "Supported": Q4_K and Q6_K decode
 * bit-exact against the reference gguf implementation):
 *   QG_Q4_K 144 B: fp16 d, fp16 dmin, uint8 scales[12], uint8 qs[128];
 *                  w = d * sc_s * q - dmin * m_s, sub-block s of 32 weights
 *                  (RAMforge README, "Milestone 5", Q4_K line).  scales[]
 *                  packs eight 6-bit sc and eight 6-bit m: s < 4 keeps
 *                  sc_s = scales[s] & 63, m_s = scales[s+4] & 63; s >= 4 keeps
 *                  their low nibbles in scales[s+4] (sc low, m high) and their
 *                  top two bits in the top bits of scales[s-4] (sc) and
 *                  scales[s] (m).  qs[32c + l] holds element l of sub-block 2c
 *                  (low nibble) and of sub-block 2c + 1 (high nibble).
 *   QG_Q6_K 210 B: uint8 ql[128], uint8 qh[64], int8 scales[16], fp16 d;
 *                  w_e = d * scales[e/16] * (q_e - 32) with the 6-bit code of
 *                  element e = 128h + 32i + l (l < 32): low four bits from
 *                  ql[64h + 32(i&1) + l] (low nibble for i < 2, else high),
 *                  top two bits from bits 2i, 2i+1 of qh[32h + l].
 *
 * Conventions shared by every entry point
 *  - Status: 0 (QG_OK) or a negative qg_status.  Arguments are validated on the
 *    host before any HIP call; a call that fails validation enqueues nothing and
 *    leaves every output untouched (fail closed: hipfire PR, "Design notes").
 *  - Memory: the caller owns every weight, activation and output buffer and
 *    every stream.  Pointers marked "device" are device (HBM) addresses; the
 *    streamed entry points take weights in page-locked host memory
 *    (hipHostMalloc / pinned), checked, never pageable.
 *  - Asynchrony: compute entry points (the GEMVs, the elementwise steps,
 *    qgemv_stream_rows / _windows / _rows_noalloc, qgemv_stream_plan_run and
 *    qgemv_chain_run) enqueue on `stream` (NULL = the default stream) and
 *    return without waiting.  qgemv_stream_create / _destroy,
 *    qgemv_stream_plan_destroy and qgemv_chain_create / _check /
 *    _set_spin_limit / _destroy wait for the device.
 *  - Outputs: y receives exactly row_end - row_start values; nothing outside
 *    that range is written.
 *  - Determinism: a row's result depends only on its own bytes, x, the format
 *    and k.  It does not depend on the window, block_rows, the grid, the stream
 *    or whether the weights were streamed, so all those give identical bits.
 *  - Threads: stateless calls are re-entrant; a qg_streamer is not thread-safe.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t. */
typedef struct ihipStream_t *qg_stream_t;

enum qg_format { QG_Q8_0 = 1, QG_Q4_0 = 2, QG_MXFP4 = 3, QG_Q4_K = 4, QG_Q6_K = 5 };

enum qg_status {
  QG_OK = 0,
  QG_E_NULL = -1,       /* a required pointer is NULL */
  QG_E_FMT = -2,        /* unknown format (RAMforge README, "Capability registry":
                           unsupported types are an explicit error) */
  QG_E_SHAPE = -3,      /* k <= 0, k % QK != 0, k > QG_MAX_K, n_rows < 0,
                           n_expert <= 0, rows not a multiple of n_expert */
  QG_E_RANGE = -4,      /* row_start < 0, row_start > row_end, row_end > n_rows,
                           expert id outside [0, n_expert) */
  QG_E_SIZE = -5,       /* n_bytes != n_rows * (k/QK) * block bytes (truncated or
                           oversized tensors are rejected: RAMforge README,
                           "Build & Test", quant.rs unit tests) */
  QG_E_ARG = -6,        /* block_rows < 0, lookahead < 1, n_win < 0 or above
                           QG_MAX_WINDOWS, n < 0, bad eps, x_stride < 0,
                           weight data not 16-byte aligned */
  QG_E_NOT_PINNED = -7, /* streamed weights not in page-locked host memory */
  QG_E_CAPACITY = -8,   /* a streamed row block is larger than a ring slot */
  QG_E_BARRIER = -9,    /* a chain's device-wide barrier gave up waiting */
  QG_E_HIP = -100       /* a HIP runtime call failed; see qgemv_last_hip_error */
};

/* Most windows one grid takes (the window table travels in kernel arguments). */
#define QG_MAX_WINDOWS 64

/* Largest k: a row's block columns are spread over at most 12 wavefronts with
 * at most 2 columns per lane, each lane holding its activations in registers. */
#define QG_MAX_K 49152

/* Largest k of a chain step: 12 wavefronts, one column per lane. */
#define QG_CHAIN_MAX_K 24576

/* A whole quantized weight matrix: the compact resident representation of a
 * quantized tensor (RAMforge README, "Milestone 5", QuantizedTensor: raw block
 * bytes plus type and shape). */
typedef struct qg_matrix {
  const void *data; /* n_bytes of blocks, row-major [n_rows][k/QK]; 16-byte
                       aligned.  Kernels fetch whole aligned 16-byte granules,
                       so they may read up to 15 bytes past the last row
                       inside the granule holding its last byte. */
  int32_t fmt;      /* enum qg_format */
  int32_t reserved; /* must be 0 */
  int64_t n_rows;   /* output rows */
  int64_t k;        /* inputs per row, a multiple of 32 (256 for K-quants) */
  int64_t n_bytes;  /* must equal qgemv_weight_bytes(fmt, n_rows, k) */
} qg_matrix;

/* A row window of one matrix with its own activation and output vectors
 * (neurostream README, "How it works", step 4: row_start/row_end bound the
 * walk over a weight matrix).  All windows of one call share fmt and k. */
typedef struct qg_window {
  const void *data;  /* the matrix's row 0 (not the window's first row); 16-byte aligned */
  int64_t n_rows;    /* rows of that matrix, for range checks */
  int64_t row_start; /* first row of the window */
  int64_t row_end;   /* one past the last row */
  const float *x;    /* device, k values */
  float *y;          /* device, row_end - row_start values: y[j] <-> row row_start + j */
} qg_window;

/* Bytes per block: 34, 18, 17, 144 or 210; QG_E_FMT for an unknown format. */
int64_t qgemv_block_bytes(int32_t fmt);

/* Weights per block (QK): 32, or 256 for Q4_K and Q6_K (RAMforge README,
 * "Milestone 5": 32-weight Q8_0/Q4_0 blocks, the 256-weight Q4_K
 * super-block); QG_E_FMT for an unknown format. */
int64_t qgemv_block_weights(int32_t fmt);

/* Bytes of an n_rows x k matrix, or a negative status (QG_E_FMT, QG_E_SHAPE). */
int64_t qgemv_weight_bytes(int32_t fmt, int64_t n_rows, int64_t k);

/* y = W[row_start:row_end] . x, weights resident in device memory.
 * w->data, x (k floats) and y (row_end - row_start floats) are device pointers.
 * block_rows = B > 0 splits the window into row blocks
 * [row_start + iB, min(row_start + (i+1)B, row_end)) (neurostream README,
 * "The idea": --block-rows; 0 keeps the whole window as one block); all blocks
 * are computed by one grid and the result does not depend on B. */
int qgemv_rows(const qg_matrix *w, int64_t row_start, int64_t row_end,
               const float *x, float *y, int64_t block_rows, qg_stream_t stream);

/* A small batch: y_t = W[row_start:row_end] . x_t for n_tok tokens t, with
 * every weight block read from memory and decoded once per pass for several
 * tokens (neurostream README, "What the numbers taught us": tokens that share
 * one pass over the weights cost about one token's weight traffic).  Token
 * t's x is the k floats at x + t * x_stride, its y the row_end - row_start
 * floats at y + t * y_stride (device pointers; y_stride >= row_end -
 * row_start when n_tok > 1, so outputs never overlap; x_stride >= 0).  A
 * pass takes four tokens while the row fits one 32-weight column per lane in
 * at most 8 waves (Q8_0, Q4_K, Q6_K: k <= 16384), else two while it fits one
 * column in 12 waves or two columns in 8 (every format up to k = 32768),
 * else one; the weights are read once per pass.  Each
 * y_t has the bits qgemv_rows gives for x_t alone.  n_tok = 0 or an empty
 * window does nothing; block_rows as in qgemv_rows. */
int qgemv_rows_batch(const qg_matrix *w, int64_t row_start, int64_t row_end,
                     const float *x, int64_t x_stride, int32_t n_tok, float *y,
                     int64_t y_stride, int64_t block_rows, qg_stream_t stream);

/* Rows [row_start, row_end) of w for n_tok tokens at once on the fp32 matrix
 * cores: y_t[r - row_start] = sum_c W[r][c] x_t[c].  With several tokens the
 * product is a dense contraction over the shared weights (neurostream README,
 * "What the numbers taught us": tokens that share one pass over the weights
 * cost about one token's weight traffic); passes of 16 tokens each read the
 * weights once.  Every format (Q4_K's weight d sc q - dmin m is formed with
 * one rounding, the others' exactly).  x, y:
 * device, token t at x + t x_stride and y + t y_stride (y_stride >=
 * row_end - row_start when n_tok > 1).  Each weight is formed exactly in fp32
 * and the sums are fp32, in the matrix cores' order: y_t is within fp32
 * rounding of W x_t, not bit-identical to qgemv_rows (qgemv_rows_batch is).
 * n_tok = 0 or an empty window does nothing; other errors as qgemv_rows_batch. */
int qgemv_rows_mfma(const qg_matrix *w, int64_t row_start, int64_t row_end,
                    const float *x, int64_t x_stride, int32_t n_tok, float *y,
                    int64_t y_stride, qg_stream_t stream);

/* Input transforms (qgemv_rows_op, chain steps) and output transforms
 * (qgemv_rows_op). */
enum qg_in_op { QG_IN_X = 0, QG_IN_RMS = 1, QG_IN_GELU_RMS = 2, QG_IN_SILU_MUL = 3 };
enum qg_out_op { QG_OUT_Y = 0, QG_OUT_GELU = 1 };

/* As qgemv_rows, with the activation transformed as it is loaded and each
 * output as it is stored, so that a decode pass needs no elementwise launch
 * between its GEMVs (neurostream README, "What the numbers taught us": the
 * time per step went to drains and small launches, not to bytes):
 *   in_op  QG_IN_X         x
 *          QG_IN_RMS       rms(x) = x / sqrt(mean(x^2) + eps), as
 *                          qgemv_rms_carry(gelu = 0); k <= 32768
 *          QG_IN_SILU_MUL  silu(x) * x2 elementwise, as qgemv_silu_mul
 *   out_op QG_OUT_Y        y = W x'
 *          QG_OUT_GELU     y = gelu(W x'), the exact (erf) GELU, once per row
 * (QG_IN_GELU_RMS is not an input op here: store the producer's output with
 * QG_OUT_GELU and normalise it with QG_IN_RMS.)  Each transform is computed
 * in the order the separate calls use, so the result has their bits: e.g.
 * qgemv_rows_op(..., QG_IN_RMS, eps, QG_OUT_Y, y) equals qgemv_rms_carry(x,
 * t, eps, 0) followed by qgemv_rows(t -> y), and GELU-stored y normalised by
 * QG_IN_RMS equals qgemv_rms_carry(y, t, eps, 1).  x2: device, k values,
 * required for QG_IN_SILU_MUL only.  Errors: an unknown op, eps < 0 or not
 * finite, or k > 32768 with QG_IN_RMS give QG_E_ARG; otherwise as qgemv_rows. */
int qgemv_rows_op(const qg_matrix *w, int64_t row_start, int64_t row_end, const float *x,
                  const float *x2, int32_t in_op, float eps, int32_t out_op, float *y,
                  int64_t block_rows, qg_stream_t stream);

/* Several row windows (any matrices of the same fmt and k, each with its own
 * x and y) computed by ONE grid: the row-bounded walks of neurostream README,
 * "How it works" (stream_linear over [row_start, row_end), for example the
 * selected experts' rows), launched together instead of one after another.
 * win is a host array of n_win entries, 0 <= n_win <= QG_MAX_WINDOWS;
 * n_win = 0 is a no-op. */
int qgemv_windows(int32_t fmt, int64_t k, const qg_window *win, int32_t n_win,
                  int64_t block_rows, qg_stream_t stream);

/* Selected experts of stacked (n_expert, out, k) tensors (neurostream README,
 * "The idea" and "How it works" step 2: expert e owns rows [e*out, (e+1)*out)
 * and only router-named experts are read).  mats is a host array of n_mat
 * matrices of the same fmt, k and n_rows = n_expert * out; ids is a host array
 * of n_sel expert ids.  All n_mat * n_sel windows run in ONE grid.
 * Input of selected expert s: x + s * x_stride (x_stride = 0: one shared x).
 * Output of matrix m, selected expert s: y + (m * n_sel + s) * out.
 * n_mat * n_sel must not exceed QG_MAX_WINDOWS. */
int qgemv_expert_windows(const qg_matrix *mats, int32_t n_mat, int64_t n_expert,
                         const int32_t *ids, int32_t n_sel, const float *x,
                         int64_t x_stride, float *y, int64_t block_rows,
                         qg_stream_t stream);

/* h[i] = silu(g[i]) * u[i], silu(v) = v / (1 + exp(-v)), fp32, device
 * pointers, n >= 0 (the SwiGLU activation between the row-contiguous gate/up
 * and down phases: neurostream README, "How it works"; run on the GPU as in
 * hipfire PR, "Design notes", silu_mul).  exp and the division use the
 * hardware exp2 and reciprocal: within about (|g| + 4) * 2^-24 of the exact
 * value, relative; the fused QG_IN_SILU_MUL loads give the same bits. */
int qgemv_silu_mul(const float *g, const float *u, float *h, int64_t n, qg_stream_t stream);

/* As qgemv_expert_windows, with qgemv_rows_op's fused transforms applied per
 * window: selected expert s reads x + s * x_stride and, for QG_IN_SILU_MUL,
 * x2 + s * x_stride.  With the gate outputs as x and the up outputs as x2 the
 * down grid takes silu(gate) * up as it loads it, so an MoE token is two
 * grids with no elementwise launch between them (neurostream README, "What
 * the numbers taught us": drains and small launches, not bytes, set the time
 * per step; hipfire PR, "Design notes": the fused SwiGLU GEMV).  in_op,
 * out_op, eps and their errors as qgemv_rows_op (QG_IN_RMS needs k <= 32768
 * and normalises each window's own x).  Results equal the separate calls'
 * bits. */
int qgemv_expert_windows_op(const qg_matrix *mats, int32_t n_mat, int64_t n_expert,
                            const int32_t *ids, int32_t n_sel, const float *x,
                            const float *x2, int64_t x_stride, int32_t in_op, float eps,
                            int32_t out_op, float *y, int64_t block_rows, qg_stream_t stream);

/* SwiGLU gate and up projections in one grid: h[j] = silu(gate_j . x') *
 * (up_j . x') for rows j in [row_start, row_end), x' = x or rms(x) (in_op
 * QG_IN_X or QG_IN_RMS, eps and k <= 32768 as qgemv_rows_op).  Each team
 * computes a gate row and the up row of the same index back to back and
 * stores only their SwiGLU product (neurostream README, "How it works": the
 * two-phase FFN whose first phase is gate and up; hipfire PR, "Design
 * notes": the fused weight_gemv_swiglu step), so neither projection is
 * written out and no elementwise launch follows.  gate and up must match in
 * fmt, k and n_rows (else QG_E_SHAPE); h is device, row_end - row_start
 * floats.  Bits equal qgemv_rows (or _op) of each, then qgemv_silu_mul. */
int qgemv_rows_swiglu(const qg_matrix *gate, const qg_matrix *up, int64_t row_start,
                      int64_t row_end, const float *x, int32_t in_op, float eps, float *h,
                      int64_t block_rows, qg_stream_t stream);

/* The same for selected experts of stacked (n_expert, out, k) gate and up
 * tensors (as qgemv_expert_windows): expert s reads x + s * x_stride and
 * writes h + s * out; all n_sel <= QG_MAX_WINDOWS experts in one grid. */
int qgemv_expert_swiglu(const qg_matrix *gate, const qg_matrix *up, int64_t n_expert,
                        const int32_t *ids, int32_t n_sel, const float *x, int64_t x_stride,
                        int32_t in_op, float eps, float *h, int64_t block_rows,
                        qg_stream_t stream);

/* Router-weighted combine of the selected experts' outputs: out[i] =
 * sum_{s < n_sel} w[s] * y[s * y_stride + i], one fp32 fma per term in s
 * order (neurostream README, "How it works": the router names the active
 * experts and their outputs are mixed back into one vector).  y (n_sel
 * vectors of n floats, y_stride >= n when n_sel > 1), w (n_sel weights) and
 * out (n floats, not overlapping y) are device pointers.  n_sel = 0 writes
 * zeros; n = 0 does nothing. */
int qgemv_combine(const float *y, int64_t y_stride, int32_t n_sel, const float *w, int64_t n,
                  float *out, qg_stream_t stream);

/* out = rms(act(v)), act = identity (gelu = 0) or exact erf GELU (gelu = 1),
 * rms(t) = t / sqrt(mean(t^2) + eps), no gain; fp32, device pointers, n >= 1,
 * eps >= 0.  The activation carry between the GEMVs of the synthetic dense
 * decode pass. */
int qgemv_rms_carry(const float *v, float *out, int64_t n, float eps, int32_t gelu,
                    qg_stream_t stream);

/* A measurement aid: one plain streaming read of n_bytes of device memory at
 * data (a positive multiple of 16 bytes, 16-byte aligned), 2048 workgroups of
 * 256 lanes each reading one 16-byte granule per step with the weights'
 * non-temporal hint; an xor of everything read is xor-ed into *sink (device
 * uint32), so the loads cannot be dropped.  Its rate is the read ceiling the
 * GEMV's weight stream is compared with: the bandwidth term of neurostream
 * README, "The idea" (tokens/sec = effective bandwidth / active bytes per
 * token), measured rather than taken from the specification.  QG_E_NULL,
 * QG_E_ARG (size or alignment); asynchronous on `stream`. */
int qgemv_read_ceiling(const void *data, int64_t n_bytes, uint32_t *sink, qg_stream_t stream);

/* Decoded fp32 weights of rows [row_start, row_end): out is device memory of
 * (row_end - row_start) * k floats, row-major; each weight is the format's
 * value (RAMforge README, "Milestone 5") rounded once to fp32, which for
 * every generated block is exact.  A test aid for the bit-exact decode check
 * (neurostream README, "Supported": bit-exact decode against the reference
 * gguf implementation): Q4_0 and the K-quants build the weights from the same
 * code formation as the GEMV's dot, Q8_0 and MXFP4 from the same decoder. */
int qgemv_dequant_rows(const qg_matrix *w, int64_t row_start, int64_t row_end,
                       float *out, qg_stream_t stream);

/* ---- streamed weights: pinned host memory -> device ring -> same kernels ----
 * A streamer owns lookahead + 1 device slots of slot_bytes each and per-slot
 * events (neurostream README, "The idea": blocks sized so
 * that lookahead + 1 buffers fit; "Bugs worth knowing about": the pipeline
 * holds depth + 1 blocks, because the block being multiplied keeps its
 * buffer until its output exists).  Block k is copied into slot
 * k mod (lookahead + 1) once the kernel of block k - lookahead - 1 has
 * released that slot, on one of min(lookahead, 2) copy streams taken in turn
 * (so that two copies can be in flight at once; the copy streams are shared
 * by the process's streamers on a device and kept until it exits); its
 * kernel runs on the caller's stream after the copy. */
typedef struct qg_streamer qg_streamer;

/* slot_bytes >= 1, lookahead >= 1.  Allocates (lookahead + 1) * slot_bytes of
 * device memory.  Synchronising. */
int qgemv_stream_create(int64_t slot_bytes, int32_t lookahead, qg_streamer **out);

/* Device bytes the ring holds: (lookahead + 1) * slot_bytes; negative status on
 * a NULL streamer. */
int64_t qgemv_stream_ring_bytes(const qg_streamer *st);

/* As qgemv_rows, with w->data in pinned host memory: the window is walked in
 * row blocks of block_rows (0 = whole window), each copied into the ring and
 * multiplied there.  Every block must fit one slot (else QG_E_CAPACITY).
 * x and y are device pointers.  `stream` waits for the last block's kernel. */
int qgemv_stream_rows(qg_streamer *st, const qg_matrix *w, int64_t row_start,
                      int64_t row_end, int64_t block_rows, const float *x, float *y,
                      qg_stream_t stream);

/* As qgemv_windows, with every win[i].data in pinned host memory; the blocks
 * of all windows go through the ring in window order. */
int qgemv_stream_windows(qg_streamer *st, int32_t fmt, int64_t k, const qg_window *win,
                         int32_t n_win, int64_t block_rows, qg_stream_t stream);

/* ---- streamed plans: a layer's streamed steps as one replayed graph ----
 * neurostream README, "What the numbers taught us": a plan that spans the
 * layer's projections and experts, instead of one prefetcher per
 * projection, removed the pipeline drains between them.  A plan is a fixed
 * list of steps: streamed GEMV steps (windows of pinned host matrices walked
 * in row blocks through the plan's own ring of lookahead + 1 device slots of
 * slot_bytes, as qgemv_stream_windows) and elementwise steps between them
 * (SiLU * up, router-weighted combine).  qgemv_stream_plan_create builds the
 * whole walk once, as a HIP graph: block b's copy waits only for the kernel
 * that last read its slot (block b - lookahead - 1), so copies run ahead
 * across steps while the kernels and elementwise steps run in order.  A run
 * replays it with one launch, with no per-block host work.  Every kernel is
 * the qgemv_rows kernel on the ring slot, so every y has the bits of the
 * resident computation. */
enum qg_plan_op { QG_PLAN_GEMV = 1, QG_PLAN_SILU_MUL = 2, QG_PLAN_COMBINE = 3 };

typedef struct qg_plan_step {
  int32_t op;          /* enum qg_plan_op */
  int32_t fmt;         /* GEMV: format of the step's windows */
  int64_t k;           /* GEMV: inputs per row */
  int32_t first_win;   /* GEMV: windows [first_win, first_win + n_win) of the */
  int32_t n_win;       /*   plan's table; each window belongs to one step */
  int64_t block_rows;  /* GEMV: rows per streamed block, 0 = whole window */
  const float *a;      /* SILU_MUL: g;  COMBINE: y, n_sel vectors stride floats apart */
  const float *b;      /* SILU_MUL: u;  COMBINE: the n_sel weights */
  float *out;          /* SILU_MUL: h;  COMBINE: out (as qgemv_combine) */
  int64_t n;           /* SILU_MUL, COMBINE: outputs */
  int64_t stride;      /* COMBINE: y stride */
  int32_t n_sel;       /* COMBINE */
  int32_t reserved;    /* 0 */
} qg_plan_step;

typedef struct qg_stream_plan qg_stream_plan;

/* Validates the steps against the host window table win (x and y device
 * pointers; data in pinned host memory, QG_E_NOT_PINNED otherwise; every
 * block must fit a slot, QG_E_CAPACITY otherwise), allocates the ring and
 * builds the graph.  Device pointers of the steps and windows are captured:
 * they must stay valid for the plan's life. */
int qgemv_stream_plan_create(int64_t slot_bytes, int32_t lookahead, const qg_plan_step *steps,
                             int32_t n_steps, const qg_window *win, int32_t n_win,
                             qg_stream_plan **out);

/* Moves streamed window w to rows [row_start, row_start + its length) of the
 * same host matrix (for example the next token's selected expert); runs
 * enqueued before the call keep the rows they were enqueued with.
 * QG_E_RANGE past the matrix's rows; QG_E_ARG for a window no GEMV step
 * streams. */
int qgemv_stream_plan_set_rows(qg_stream_plan *p, int32_t w, int64_t row_start);

/* Device bytes of the plan's ring: (lookahead + 1) * slot_bytes. */
int64_t qgemv_stream_plan_ring_bytes(const qg_stream_plan *p);

/* Enqueues one run of the plan on `stream` (its device must be current).
 * Runs of one plan share its ring: they must not overlap, so enqueue them
 * on one stream. */
int qgemv_stream_plan_run(qg_stream_plan *p, qg_stream_t stream);

/* Waits for the device, frees the plan.  NULL is a no-op. */
int qgemv_stream_plan_destroy(qg_stream_plan *p);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): qgemv_stream_rows with no
 * streamer and no allocation of any kind.  The ring is a device array of
 * QG_NOALLOC_RING_BYTES inside the library (one per GPU, held until the
 * process ends), used as two slots of half that size: block j of the window
 * is copied into slot j mod 2 with hipMemcpyAsync on `stream` and multiplied
 * there by the same kernel as qgemv_rows, so y has qgemv_rows's bits.  Copies
 * and kernels share `stream`: they run one after the other, with no
 * copy/compute overlap.  A block of more than QG_NOALLOC_RING_BYTES / 2
 * bytes gives QG_E_CAPACITY, pageable or device weights QG_E_NOT_PINNED.
 * Every call on a GPU uses that GPU's one ring: calls that overlap on one GPU
 * (on different streams, or from several threads) race and must not be
 * made. */
#define QG_NOALLOC_RING_BYTES (32ll << 20)
int qgemv_stream_rows_noalloc(const qg_matrix *w, int64_t row_start, int64_t row_end,
                              int64_t block_rows, const float *x, float *y, qg_stream_t stream);

/* Waits for the streamer's work, frees it.  NULL is a no-op. */
int qgemv_stream_destroy(qg_streamer *st);

/* ---- host-mapped weights (zero copy) ----
 * The weights stay in page-locked host memory (hipHostMalloc, mapped into the
 * device's address space) and the same kernels read them in place over the
 * host link: no device copy, no ring, no copy stream (hipfire PR, "Design
 * notes": host memory from hipHostMalloc with hipHostMallocMapped, kernels
 * unchanged, dereferencing the host-mapped alias; its "pcie" execution arm).
 * Every other argument, the validation and the result are those of
 * qgemv_rows / qgemv_windows, so a row gives the same bits resident, streamed
 * or mapped.  Weights not in page-locked host memory (pageable or device
 * memory) give QG_E_NOT_PINNED before anything is enqueued.  The host memory
 * must stay allocated and unmodified until the work on `stream` has finished. */
int qgemv_mapped_rows(const qg_matrix *w, int64_t row_start, int64_t row_end, const float *x, float *y,
                      int64_t block_rows, qg_stream_t stream);
int qgemv_mapped_windows(int32_t fmt, int64_t k, const qg_window *win, int32_t n_win,
                         int64_t block_rows, qg_stream_t stream);

/* ---- chains: dependent GEMVs in one persistent grid ----
 * A decode pass is a sequence of GEMVs, each taking the previous one's output
 * through a small transform.  Launched one by one, every GEMV ends with a
 * drain: the last rows finish while HBM idles, and the next launch ramps up
 * from nothing.  A chain runs the whole sequence as ONE launch that spans it
 * (neurostream README, "What the numbers taught us": one pipeline per
 * projection drained once per projection; a plan spanning the layer removed
 * those drains).  Workgroups stay resident, wait at a device-wide barrier
 * between steps, and fetch the weights of their next step before waiting,
 * since weights do not depend on the input.
 *
 * Step s computes, for each of its windows, y = W[row_start:row_end] . op(x),
 * with op applied as the kernel loads x:
 *   QG_IN_X         x
 *   QG_IN_RMS       rms(x), as qgemv_rms_carry(gelu = 0)
 *   QG_IN_GELU_RMS  rms(gelu(x)), as qgemv_rms_carry(gelu = 1)
 *   QG_IN_SILU_MUL  silu(x) * x2, as qgemv_silu_mul
 * Steps run in order and see everything earlier steps wrote.  Each row is
 * computed in qgemv_rows' per-row order and each transform in the order of
 * the call named beside it, so a chain gives the same bits as the equivalent
 * sequence of separate calls. */
/* (enum qg_in_op is declared with qgemv_rows_op above.) */

typedef struct qg_chain_window {
  const void *data;  /* the matrix's row 0, device, 16-byte aligned */
  int64_t n_rows;    /* rows of that matrix, for range checks */
  int64_t row_start; /* first row of the window */
  int64_t row_end;   /* one past the last row */
  const float *x;    /* device, k values: the transform's input */
  const float *x2;   /* device, k values: the multiplier of QG_IN_SILU_MUL, else unused */
  float *y;          /* device, row_end - row_start values */
} qg_chain_window;

typedef struct qg_chain_step {
  int64_t k;         /* inputs per row: a multiple of 32, at most QG_CHAIN_MAX_K */
  int32_t first_win; /* the step's windows: win[first_win .. first_win + n_win) */
  int32_t n_win;     /* >= 1 (windows may be empty) */
  int32_t in_op;     /* enum qg_in_op; the RMS ops need one x shared by all windows */
  float eps;         /* >= 0, for the RMS ops */
} qg_chain_step;

typedef struct qg_chain qg_chain;

/* Validates and uploads a chain of n_steps steps over the host arrays steps
 * and win (all windows of one fmt: Q8_0, Q4_0 or MXFP4; a K-quant format
 * returns QG_E_FMT), sized for the current device.  The chain
 * keeps the pointers, not the data: every buffer must outlive its runs.
 * Within a step, a window's y must not overlap any x, x2 or other y of that
 * step, and no step may write weights.  Synchronising. */
int qgemv_chain_create(int32_t fmt, const qg_chain_step *steps, int32_t n_steps,
                       const qg_chain_window *win, int32_t n_win, qg_chain **out);

/* Enqueues one run of every step on `stream` (one launch on the chain's
 * device, which must be current), of one workgroup per compute unit: all of
 * them must be resident together, so nothing else may occupy compute units
 * while it runs.  Runs of one chain must not overlap: they share its barrier
 * state.  A barrier that waits longer than its spin limit (a few seconds by
 * default) gives up, marks the chain failed and lets the run finish with
 * undefined outputs.  Once a failure is visible to the host (a page-locked
 * word the failing barrier writes; no waiting is involved), qgemv_chain_run
 * enqueues nothing and returns QG_E_BARRIER until qgemv_chain_check has
 * reset the state (a failure of a run still in flight is seen by the next
 * call to qgemv_chain_check). */
int qgemv_chain_run(qg_chain *c, qg_stream_t stream);

/* Waits for the device, then QG_OK, or QG_E_BARRIER if a run's barrier gave
 * up since the last check (workgroups not all resident; those outputs are
 * undefined), after resetting the state for the next run. */
int qgemv_chain_check(qg_chain *c);

/* Polls (>= 1) a barrier waits before it gives up; the default is 2^22.
 * Waits for the device.  QG_E_ARG for 0 or on another device. */
int qgemv_chain_set_spin_limit(qg_chain *c, uint32_t polls);

/* Workgroups a run launches (one per compute unit), or a negative status. */
int64_t qgemv_chain_grid(const qg_chain *c);

/* Waits for the device, frees the chain.  NULL is a no-op. */
int qgemv_chain_destroy(qg_chain *c);

/* Static text for a status. */
const char *qgemv_strerror(int status);

/* Text of the last QG_E_HIP on this thread ("" if none). */
const char *qgemv_last_hip_error(void);

/* Library version, e.g. "0.1.0". */
const char *qgemv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
