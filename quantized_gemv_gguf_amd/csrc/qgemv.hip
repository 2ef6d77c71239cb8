// qgemv.hip -- the C ABI of libqgemv.so (see include/qgemv.h), its host side,
// the chain kernel and the small elementwise kernels.  The GEMV kernel itself
// (block formats, fused row dot, LDS-DMA weight ring) lives in qgemv_impl.h,
// instantiated per fused-transform variant in gemv_op*.hip.
//
// Batch-1 dequant-GEMV over GGUF blocks (Q8_0, Q4_0, MXFP4, Q4_K, Q6_K): every output row
// is a dot product of its dequantized weights with an fp32 activation vector,
// accumulated in fp32, the weights decoded in registers and never written out
// (neurostream README, "How it works", step 5: the fused decode-path GEMV).
// Single-batch decode reads every active weight once per token, so the
// kernels are bound by weight bytes moved (neurostream README, "The idea":
// tokens/sec = effective bandwidth / active bytes per token).  No MFMA: a
// matrix-vector product has no operand reuse to feed a matrix core.
//
// Work decomposition
//   A "team" is one workgroup of WT wavefronts (T = 64 * WT lanes).  Team lane
//   t owns the block columns j = t + T*c (c < C) of every row it touches, and
//   keeps the 32 activations of each such column in registers, loaded once per
//   window (a "column" is 32 weights: a block, or a K-quant sub-block).  A row
//   is one pass: each lane dots its C columns,
//   the 64 lanes of a wave are combined by fixed DPP shifts, and for
//   WT > 1 the per-wave sums go through LDS and are added in wave order.
//   (WT, C) is a function of (format, k) only, and so is the whole per-row
//   operation order: a row gives the same bits whichever window, row block,
//   tile, team, launch or stream computes it, resident, streamed or mapped.
//
//   Rows are cut into tiles that never straddle a row block (block_rows), the
//   tiles of all windows are numbered in window order, and team b takes tiles
//   b, b + T, b + 2T, ... (T teams in the grid).
//
// Matrix layout: row-major [n_rows][k/QK blocks], y[o] = sum_i W[o, i] x[i]
// (RAMforge README, "Milestone 6", matrix layout).  Each row is a whole number
// of blocks, so a row window is one contiguous byte range (neurostream README,
// "The idea").
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "qgemv.h"

#include "qgemv_impl.h"

using namespace qgemv_detail;

// Kernel variants instantiated in gemv_op*.hip.
namespace qgemv_detail {
extern template GemvFn pick_op<kOpNone>(int32_t, Shape);
extern template GemvFn pick_op<kOpRms>(int32_t, Shape);
extern template GemvFn pick_op<kOpRmsGelu>(int32_t, Shape);
extern template GemvFn pick_op<kOpSilu>(int32_t, Shape);
extern template GemvFn pick_op<kOpGelu>(int32_t, Shape);
extern template GemvFn pick_op<kOpSwiglu>(int32_t, Shape);
extern template GemvFn pick_op<kOpRmsSwiglu>(int32_t, Shape);
extern template GemvFn pick_batch<2>(int32_t, Shape);
extern template GemvFn pick_batch<4>(int32_t, Shape);
}  // namespace qgemv_detail

namespace {

// ---------------------------------------------------------------------------
// Dequant (test aid), SiLU*up, RMS carry
// ---------------------------------------------------------------------------

// One thread per 32 weights (nb of them per row).
template <int FMT>
__global__ void dequant_kernel(const uint8_t *base, int64_t row_start, int64_t n_rows, int nb,
                               int64_t row_bytes, float *out) {
  using F = Fmt<FMT>;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= n_rows * nb) return;
  const int64_t r = id / nb;
  const int j = (int)(id - r * nb);
  if constexpr (F::kUnits > 1) {
    const uint8_t *blk = base + (row_start + r) * row_bytes + (int64_t)F::kBytes * (j / F::kUnits);
    float w[32];
    F::dequant(blk, j % F::kUnits, w);
    float *o = out + r * (int64_t)nb * 32 + 32 * j;
#pragma unroll
    for (int e = 0; e < 32; ++e) o[e] = w[e];
    return;
  } else if constexpr (F::kDot) {
    float w[32];
    F::dequant(base + (row_start + r) * row_bytes + (int64_t)F::kBytes * j, w);
    float *o = out + r * (int64_t)nb * 32 + 32 * j;
#pragma unroll
    for (int e = 0; e < 32; ++e) o[e] = w[e];
    return;
  } else {
  const uint8_t *p = base + (row_start + r) * row_bytes + (int64_t)F::kBytes * j;
  uint32_t sbits = 0, q[F::kWords];
  __builtin_memcpy(&sbits, p, F::kScaleBytes);
  __builtin_memcpy(q, p + F::kScaleBytes, 4 * F::kWords);
  float u[32];
  F::decode(q, u);
  const auto s = F::scale(sbits);
  float *o = out + r * (int64_t)nb * 32 + 32 * j;
#pragma unroll
  for (int e = 0; e < 32; ++e) o[e] = F::apply(s, u[e]);
  }
}

__global__ void silu_mul_kernel(const float *g, const float *u, float *h, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float v = g[i];
    h[i] = silu_times(v, u[i]);
  }
}

// out[i] = sum over s < n_sel of w[s] y[s y_stride + i], one fma per term in
// s order (a fixed order: the same bits whichever grid computes it).
__global__ void combine_kernel(const float *y, int64_t y_stride, int n_sel, const float *w, int64_t n,
                               float *out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float acc = 0.0f;
    for (int s = 0; s < n_sel; ++s) acc = fmaf(w[s], y[s * y_stride + i], acc);
    out[i] = acc;
  }
}

// Plain streaming read of n16 16-byte granules: every lane reads one granule
// per iteration, grid-stride, with the weights' non-temporal hint, and folds
// it into an xor so the loads are live; each wave adds one atomic xor to
// *sink.  The bandwidth a kernel that only reads reaches on this device: the
// ceiling the GEMV's weight stream is compared with.
constexpr int kReadGroups = 2048, kReadThreads = 256;
__global__ void __launch_bounds__(kReadThreads) read_kernel(const u32x4 *p, int64_t n16, uint32_t *sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, acc);
}

constexpr int kCarryThreads = 1024;
constexpr int kMaxRmsK = 32 * kCarryThreads;  // largest k whose fused RMS matches qgemv_rms_carry's order


// One workgroup, 16 waves.  For n a multiple of 32 up to 32768 (every k a
// GEMV takes in one pass), thread t owns elements [32t, 32t + 32): it loads
// them once, sums their squares in element order, the lanes of a wave are
// combined by wave_sum63 and the 16 wave sums added in wave order.  The chain
// kernel forms the same sum in the same order from the same lanes, so both
// give identical bits.  Other n: a strided loop, same reduction tree.
__global__ void __launch_bounds__(kCarryThreads)
rms_carry_kernel(const float *v, float *out, int64_t n, float eps, int gelu) {
  __shared__ float part[kCarryThreads / 64];
  const int tid = threadIdx.x;
  float ss = 0.0f;
  if (n % 32 == 0 && n <= 32 * kCarryThreads) {
    const int nb = (int)(n / 32);
    const bool ok = tid < nb;
    const float *p = v + 32 * min(tid, nb - 1);
    float t[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float4 w;
      __builtin_memcpy(&w, p + 4 * q, 16);
      t[4 * q + 0] = ok ? w.x : 0.0f;
      t[4 * q + 1] = ok ? w.y : 0.0f;
      t[4 * q + 2] = ok ? w.z : 0.0f;
      t[4 * q + 3] = ok ? w.w : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      if (gelu) t[e] = gelu_erf(t[e]);
      ss = fmaf(t[e], t[e], ss);
    }
    ss = wave_sum63(ss);
    if ((tid & 63) == 63) part[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int i = 0; i < kCarryThreads / 64; ++i) tot += part[i];
    const float inv = 1.0f / sqrtf(tot / (float)n + eps);
    if (ok) {
      float *o = out + 32 * tid;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 w = make_float4(t[4 * q] * inv, t[4 * q + 1] * inv, t[4 * q + 2] * inv, t[4 * q + 3] * inv);
        __builtin_memcpy(o + 4 * q, &w, 16);
      }
    }
    return;
  }
  for (int64_t i = tid; i < n; i += kCarryThreads) {
    float t = v[i];
    if (gelu) t = gelu_erf(t);
    ss = fmaf(t, t, ss);
  }
  ss = wave_sum63(ss);
  if ((tid & 63) == 63) part[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kCarryThreads / 64; ++i) tot += part[i];
  const float inv = 1.0f / sqrtf(tot / (float)n + eps);
  for (int64_t i = tid; i < n; i += kCarryThreads) {
    float t = v[i];
    if (gelu) t = gelu_erf(t);
    out[i] = t * inv;
  }
}

// ---------------------------------------------------------------------------
// Chain: dependent GEMV steps in one persistent grid
// ---------------------------------------------------------------------------
//
// One workgroup of kChainWaves waves per CU stays resident for the whole
// chain.  In each step a team is ceil(nb/64C) of those waves with the lane
// to block map of gemv_kernel at the same (format, k): C = 1 block column per
// lane for Q8_0, 2 for Q4_0 and MXFP4.  A workgroup holds 12 / WT teams,
// and team tau of the grid takes tiles tau, tau + T, tau + 2T, ...  Between
// steps every workgroup waits at a device-wide barrier, because the next
// step's input is the previous step's output.  Weights never depend on it:
// during its last tile of a step a wave already fetches the rows of its next
// tile, in whichever later step that is, so those loads are in flight while
// the barrier completes (wave 0, which runs the barrier, fetches right after
// arriving instead).  The input transform (RMS, GELU + RMS,
// SiLU * up) is applied as x is loaded into registers; the sum of squares of
// the RMS is formed in the order qgemv_rms_carry uses (32 consecutive
// elements per lane, the lanes of a wave by wave_sum63, the waves in order),
// so a chain reproduces the separate calls bit for bit.

constexpr int kChainWaves = 12;

// Rows per chain tile: the tile cap of gemv_kernel, one row less at two
// columns per lane (the chain keeps more state in registers).
template <int FMT, int C> struct ChainRows { static constexpr int value = TileCap<FMT, C>::value - (C == 2 ? 1 : 0); };
constexpr unsigned kSpinLimit = 1u << 22;  // default barrier polls before giving up (seconds)

struct ChainWinDev {
  const uint8_t *base;
  const float *x, *x2;
  float *y;
  float *act;  // if set, also receives gelu(y) (the next step's GELU, done once per row)
  int64_t row_start, row_end;
};

// Everything a step needs is in its record, its first window included, so a
// single-window step reads no table after the record.
struct ChainStepDev {
  ChainWinDev w0;   // the step's first window
  const float *xs;  // the RMS ops' shared x (first non-empty window's)
  int64_t row_bytes;
  uint64_t team_of_wave;  // 4 bits per wave: its team in the workgroup, 15 = none
  int32_t win0, n_win, pre0;  // windows [win0, win0 + n_win); their tile prefix at pre0
  int32_t in_op, nb, wt, tpw, tile_rows, n_tiles;
  int32_t teams;           // teams in the grid (workgroups * tpw)
  int32_t iters_q, iters_r;  // n_tiles = iters_q * teams + iters_r
  float eps;
};

// Barrier state, one 256-byte line per word.  `count` returns to 0 after every
// barrier; each workgroup polls a generation of its own line (spreading the
// polls over as many lines), which only grows (wrapping): barrier b of a launch
// is complete once it reaches base + b, base being the generation at the
// launch's start, which the host tracks from run to run.
constexpr int kMaxChainGroups = 1024;

struct ChainSync {
  unsigned count, pad0[63];
  unsigned fail, pad1[63];
  // Set by the host: a page-locked host word that a failing barrier also
  // marks (the host reads it without waiting for the device), and the polls
  // a barrier waits before it gives up.
  unsigned *host_fail;
  unsigned spin_limit, pad2[61];
  struct { unsigned gen, pad[63]; } flag[kMaxChainGroups];  // one line per workgroup
};

constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0), expcnt and lgkmcnt unconstrained

// Split-phase device-wide barrier, run by wave 0 of each workgroup as a whole
// wave (every branch uniform).  Every release step below waits for all of
// the wave's outstanding memory operations, so all of them happen before the
// wave fetches the next step's weights: only the wait for the barrier itself
// overlaps that fetch.
//   arrive: release fence (L2 write-back of the workgroup's stores; the
//     compiler's own wait after it can be dropped when nothing else is
//     outstanding, so an explicit one follows), then add 1 to `count`.  The
//     last arrival acquires, resets `count`, releases, and writes `target`
//     to every workgroup's line.
//   wait: unless last, poll the own line until it reaches `target`, then
//     acquire.
// A barrier still incomplete after spin_limit polls marks `fail` (and the
// host's word) and lets the workgroup through, so the kernel always ends; the
// host reports it.
__device__ __forceinline__ bool chain_arrive(ChainSync *sy, unsigned n_groups, unsigned target, int wid) {
  __syncthreads();
  bool last = false;
  if (wid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    const unsigned arrived = __builtin_amdgcn_readfirstlane(
        __hip_atomic_fetch_add(&sy->count, threadIdx.x == 0 ? 1u : 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    last = arrived == n_groups - 1;
    if (last) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(&sy->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      for (unsigned g = threadIdx.x & 63; g < n_groups; g += 64)
        __hip_atomic_store(&sy->flag[g].gen, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  return last;
}

__device__ __forceinline__ void chain_wait(ChainSync *sy, unsigned target, bool last, int wid) {
  if (wid == 0 && !last) {
    const unsigned limit = sy->spin_limit;
    for (unsigned spins = 1;; ++spins) {
      const unsigned g = __builtin_amdgcn_readfirstlane(
          __hip_atomic_load(&sy->flag[blockIdx.x].gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if ((int)(g - target) >= 0) break;
      bool give_up = spins >= limit;
      if ((spins & 63) == 0)
        give_up |= __builtin_amdgcn_readfirstlane(
                        __hip_atomic_load(&sy->fail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0;
      if (give_up) {
        __hip_atomic_store(&sy->fail, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(sy->host_fail, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}


// Pointers read from the chain's device tables lose their address space; the
// kernel marks them global so that loads and stores are global_* (flat ones
// would also count against the LDS counter and stall every LDS wait on the
// weight prefetch).
#define QG_GLOBAL __attribute__((address_space(1)))
// The step, window and tile tables never change during a launch: read through
// the constant address space they become scalar loads, which neither wait on
// nor hold up the vector loads of the weights (as plain global loads after the
// barrier's fences they would be vector loads, each draining the prefetch).
#define QG_CONST __attribute__((address_space(4)))
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));


__device__ __forceinline__ ChainWinDev load_win(const QG_CONST ChainWinDev *p) {
  ChainWinDev d;
  d.base = p->base;
  d.x = p->x;
  d.x2 = p->x2;
  d.y = p->y;
  d.act = p->act;
  d.row_start = p->row_start;
  d.row_end = p->row_end;
  return d;
}

__device__ __forceinline__ ChainStepDev load_step(const QG_CONST ChainStepDev *p) {
  ChainStepDev d;
  d.w0 = load_win(&p->w0);
  d.xs = p->xs;
  d.row_bytes = p->row_bytes;
  d.team_of_wave = p->team_of_wave;
  d.win0 = p->win0;
  d.n_win = p->n_win;
  d.pre0 = p->pre0;
  d.in_op = p->in_op;
  d.nb = p->nb;
  d.wt = p->wt;
  d.tpw = p->tpw;
  d.tile_rows = p->tile_rows;
  d.n_tiles = p->n_tiles;
  d.teams = p->teams;
  d.iters_q = p->iters_q;
  d.iters_r = p->iters_r;
  d.eps = p->eps;
  return d;
}

template <int FMT, int C>
__global__ void __launch_bounds__(64 * kChainWaves) __attribute__((amdgpu_waves_per_eu(3)))
chain_kernel(const ChainStepDev *steps_g, int n_steps, const ChainWinDev *wins_g, const int32_t *prefix_g,
             ChainSync *sync, unsigned base) {
  const QG_CONST ChainStepDev *steps = (const QG_CONST ChainStepDev *)steps_g;
  const QG_CONST ChainWinDev *wins = (const QG_CONST ChainWinDev *)wins_g;
  const QG_CONST int32_t *prefix = (const QG_CONST int32_t *)prefix_g;
  using F = Fmt<FMT>;
  constexpr int BB = F::kBytes;
  constexpr int R = ChainRows<FMT, C>::value;
  constexpr int SB = 64 * C;                   // blocks per wave slice
  constexpr int CH = (SB * BB + 15) / 16 + 1;  // 16-byte chunks a slice can touch
  constexpr int V = (CH + 63) / 64;
  constexpr int ROWB = 64 * V * 16 + 16;
  __shared__ __attribute__((aligned(16))) uint8_t stage[kChainWaves][2][ROWB];
  // Team reduction ring (several teams per workgroup): a wave writes its row
  // sums for tile j into slot j % kRing and counts itself in; the last of the
  // team to arrive adds them in wave order, stores y and marks the slot
  // consumed.  No workgroup-wide sync per tile, so the teams of a workgroup
  // do not wait for each other.  A team that is the whole workgroup uses the
  // workgroup barrier and two of the slots instead.
  constexpr int kRing = 4;
  __shared__ float red[kRing][kChainWaves][R];
  __shared__ unsigned arrived[kChainWaves][kRing], consumed[kChainWaves][kRing];
  __shared__ float ssq[kChainWaves * C];
  // x of an RMS step with k <= kSharedX, read once by the whole workgroup.
  constexpr int kSharedX = 8192;
  constexpr int kSharedIt = (kSharedX / 4 + 64 * kChainWaves - 1) / (64 * kChainWaves);
  __shared__ __attribute__((aligned(16))) float xsh[kSharedX];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lane16 = 16u * lane;
  const int G = gridDim.x;
  const int wg = blockIdx.x;

  // The wave's place in one step.
  struct Role {
    int team0;     // first wave of its team in the workgroup
    int wit;       // its index in the team (its slice: block columns [64 wit, 64 wit + 64))
    int tau, T;    // its team in the grid, teams in the grid
    int my_iters;  // tiles of its team
  };
  // Team tau takes tiles tau, tau + T, ...: iters_q of them, one more if
  // tau < iters_r.
  auto role_of = [&](const ChainStepDev &S, Role &ro) {
    const int tiw = (int)((S.team_of_wave >> (4 * wid)) & 15);
    const bool member = tiw != 15;
    ro.team0 = member ? tiw * S.wt : wid;
    ro.wit = wid - ro.team0;
    ro.T = S.teams;
    const int first = wg * S.tpw;
    ro.tau = first + (member ? tiw : 0);
    ro.my_iters = member ? S.iters_q + (ro.tau < S.iters_r ? 1 : 0) : 0;
  };

  // A tile, kept small (scalar registers are scarce in this kernel).
  struct Tile {
    int s, w, j;                    // step, window within the step, iteration within the step
    int nrows;                      // rows of the tile (at least 1)
    uint32_t rb;                    // row bytes
    uint32_t slice_len;             // bytes of the wave's slice of a row
    int slice_n;                    // blocks of the wave's slice of a row
    const QG_GLOBAL uint8_t *row0;  // the tile's first row advanced to the wave's slice
    QG_GLOBAL float *y;             // y of the tile's first row
    QG_GLOBAL float *act;           // act of the tile's first row, or null
  };
  auto locate = [&](const ChainStepDev &S, int s, int j, int t, int w_from, int wit, Tile &T) {
    int w = 0, tt = t;
    ChainWinDev W = S.w0;
    if (S.n_win > 1) {
      w = w_from;
      while (t >= prefix[S.pre0 + w + 1]) ++w;
      tt = t - prefix[S.pre0 + w];
      W = load_win(wins + S.win0 + w);
    }
    const int64_t off = (int64_t)tt * S.tile_rows;  // first row, from the window's start
    T.s = s;
    T.w = w;
    T.j = j;
    T.nrows = (int)min((int64_t)S.tile_rows, W.row_end - W.row_start - off);
    T.rb = (uint32_t)S.row_bytes;
    T.slice_n = min(SB, S.nb - SB * wit);
    T.slice_len = (uint32_t)(T.slice_n * BB);
    T.row0 = (const QG_GLOBAL uint8_t *)W.base + (W.row_start + off) * S.row_bytes + (int64_t)(SB * wit) * BB;
    T.y = (QG_GLOBAL float *)W.y + off;
    T.act = W.act ? (QG_GLOBAL float *)W.act + off : nullptr;
  };
  // The tile after `cur`: the next one of its step, else the first tile of the
  // next step in which the wave's team has work.
  auto next_tile = [&](const Tile &cur, const Role &ro, const ChainStepDev &S, Tile &nx) -> bool {
    if (cur.j + 1 < ro.my_iters) {
      locate(S, cur.s, cur.j + 1, ro.tau + (cur.j + 1) * ro.T, cur.w, ro.wit, nx);
      return true;
    }
    for (int s2 = cur.s + 1; s2 < n_steps; ++s2) {
      const ChainStepDev S2 = load_step(steps + s2);
      Role r2;
      role_of(S2, r2);
      if (r2.my_iters > 0) {
        locate(S2, s2, 0, r2.tau, 0, r2.wit, nx);
        return true;
      }
    }
    return false;
  };

  u32x4 buf[R][V];
  auto fetch_row = [&](int i, const Tile &T) {
    const QG_GLOBAL uint8_t *p = T.row0 + (uint32_t)min(i, T.nrows - 1) * T.rb;
    const uint32_t ph = (uint32_t)((uintptr_t)p & 15);
    const uint32_t last16 = ((ph + T.slice_len - 1) >> 4) << 4;
    const QG_GLOBAL uint8_t *pa = p - ph;
#pragma unroll
    for (int v = 0; v < V; ++v)  // read once per pass: non-temporal, as the GEMV's copies
      buf[i][v] = __builtin_nontemporal_load((const QG_GLOBAL u32x4 *)(pa + min(lane16 + 1024u * v, last16)));
  };

  // The 32 inputs of each block column SB wit + 64 c + lane, zero past the
  // row.  Once per step (the RMS steps' shared x), each 2048-float run of the
  // wave's slice is read with contiguous 1 KB loads (lane l takes floats
  // 4(l + 64q) .. + 4, q < 8) and turned around in the wave's staging buffer,
  // in two halves of 4 KB: a lane's own 128 contiguous bytes read directly
  // make every load touch 64 cache lines, and when every workgroup reads x at
  // once right after the barrier those requests queue for microseconds.
  float xr[C][32];
  float xs[C][2] = {};  // unit_sums(xr) for the formats whose dot takes them
  auto gather_x = [&](const float *xg, int b0, int nb, float (&out)[32]) {
    const QG_GLOBAL float *x = (const QG_GLOBAL float *)xg + 32 * min(b0, nb - 1);
    const int nbr = min(64, nb - b0);                  // blocks of the run (<= 0: none)
    const uint32_t last = (uint32_t)max(32 * nbr, 4) - 4;  // last float quad inside x
    // Unsigned offsets from a wave-uniform base (one offset register per
    // load), and no per-load zeroing: a lane's block is past the row as a
    // whole, so its inputs are zeroed after the turn-around instead.
    f32x4u t[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) t[q] = *(const QG_GLOBAL f32x4u *)(x + min(4u * (lane + 64 * q), last));
    uint8_t *sb = stage[wid][0];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int q = 0; q < 4; ++q) *(f32x4u *)(sb + 16 * (lane + 64 * q)) = t[4 * half + q];
      __builtin_amdgcn_wave_barrier();
      if ((lane >> 5) == half) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const f32x4u v = *(const f32x4u *)(sb + 128 * (lane & 31) + 16 * e);
          out[4 * e + 0] = v.x;
          out[4 * e + 1] = v.y;
          out[4 * e + 2] = v.z;
          out[4 * e + 3] = v.w;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    if (lane >= nbr) {
#pragma unroll
      for (int e = 0; e < 32; ++e) out[e] = 0.0f;
    }
  };
  // Per window (inside the tile loop, where the current tile's weights are
  // live in registers): each lane loads its own inputs directly.
  auto load_x = [&](const float *xg, const float *x2g, bool silu, int nb, int wit) {
    const QG_GLOBAL float *x = (const QG_GLOBAL float *)xg;
    const QG_GLOBAL float *x2 = (const QG_GLOBAL float *)x2g;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = SB * wit + 64 * c + lane;
      const int jj = min(j, nb - 1);
      const bool ok = j < nb;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        f32x4u v = *(const QG_GLOBAL f32x4u *)(x + 32 * jj + 4 * q);
        if (silu) {
          const f32x4u u = *(const QG_GLOBAL f32x4u *)(x2 + 32 * jj + 4 * q);
          v.x = silu_times(v.x, u.x);
          v.y = silu_times(v.y, u.y);
          v.z = silu_times(v.z, u.z);
          v.w = silu_times(v.w, u.w);
        }
        xr[c][4 * q + 0] = ok ? v.x : 0.0f;
        xr[c][4 * q + 1] = ok ? v.y : 0.0f;
        xr[c][4 * q + 2] = ok ? v.z : 0.0f;
        xr[c][4 * q + 3] = ok ? v.w : 0.0f;
      }
    }
    if constexpr (Fmt<FMT>::kSums) unit_sums<C>(xr, xs);
  };

  // Wave 0 runs the barrier, whose release steps wait for all of the wave's
  // outstanding loads: it fetches a tile of a later step only after arriving
  // at that step's barrier (`deferred`).  The other waves fetch it during
  // their last tile of the current step.
  Tile cur{};
  bool deferred = false;
  for (int s2 = 0; s2 < n_steps; ++s2) {
    const ChainStepDev S2 = load_step(steps + s2);
    Role r2;
    role_of(S2, r2);
    if (r2.my_iters > 0) {
      locate(S2, s2, 0, r2.tau, 0, r2.wit, cur);
#pragma unroll
      for (int i = 0; i < R; ++i) fetch_row(i, cur);
      break;
    }
  }
  // Ring counters restart with every step (its teams differ); every wave is
  // past the previous step's tile loop here (the barrier's workgroup sync),
  // and none enters the next before the sync that ends the barrier.
  auto reset_ring = [&]() {
    if (threadIdx.x < kChainWaves * kRing) {
      (&arrived[0][0])[threadIdx.x] = 0;
      (&consumed[0][0])[threadIdx.x] = 0;
    }
  };
  reset_ring();
  __syncthreads();
  for (int s = 0; s < n_steps; ++s) {
    const ChainStepDev S = load_step(steps + s);
    Role ro;
    role_of(S, ro);
    const bool busy = ro.my_iters > 0;
    if (s > 0) {
      const unsigned target = base + (unsigned)s;
      const bool last = chain_arrive(sync, (unsigned)G, target, wid);
      reset_ring();
      if (deferred && cur.s == s) {
#pragma unroll
        for (int i = 0; i < R; ++i) fetch_row(i, cur);
        deferred = false;
      }
      chain_wait(sync, target, last, wid);
    }
    const bool rms = S.in_op == QG_IN_RMS || S.in_op == QG_IN_GELU_RMS;
    int xw = -1;
    const float *cxp = nullptr, *cx2p = nullptr;  // inputs of the registered x
    if (rms) {
      // Every window of an RMS step shares x: normalise it once for the step.
      // Column c of a lane's blocks is its own 64-block run, summed like one
      // wave of qgemv_rms_carry; the runs are then added in column order.
      const bool gelu = S.in_op == QG_IN_GELU_RMS;
      const bool shared = 32 * S.nb <= kSharedX;
      if (shared) {
        // Small x: the workgroup reads it once with contiguous loads (GELU
        // applied on the way) instead of once per team, right after the
        // barrier when every workgroup wants it.
        const QG_GLOBAL f32x4u *xg = (const QG_GLOBAL f32x4u *)S.xs;
        f32x4u v[kSharedIt];
#pragma unroll
        for (int it = 0; it < kSharedIt; ++it) {
          const int f = (int)threadIdx.x + 64 * kChainWaves * it;
          v[it] = xg[min(f, 8 * S.nb - 1)];
        }
#pragma unroll
        for (int it = 0; it < kSharedIt; ++it) {
          const int f = (int)threadIdx.x + 64 * kChainWaves * it;
          if (f < 8 * S.nb) {
            if (gelu) {
              v[it].x = gelu_erf(v[it].x);
              v[it].y = gelu_erf(v[it].y);
              v[it].z = gelu_erf(v[it].z);
              v[it].w = gelu_erf(v[it].w);
            }
            *(f32x4u *)&xsh[4 * f] = v[it];
          }
        }
        __syncthreads();
      }
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float ss = 0.0f;
        if (busy) {
          if (shared) {
            const int b = SB * ro.wit + 64 * c + lane;
            const float *src = &xsh[32 * min(b, S.nb - 1)];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const f32x4u t = *(const f32x4u *)(src + 4 * e);
              xr[c][4 * e + 0] = b < S.nb ? t.x : 0.0f;
              xr[c][4 * e + 1] = b < S.nb ? t.y : 0.0f;
              xr[c][4 * e + 2] = b < S.nb ? t.z : 0.0f;
              xr[c][4 * e + 3] = b < S.nb ? t.w : 0.0f;
            }
          } else {
            gather_x(S.xs, SB * ro.wit + 64 * c, S.nb, xr[c]);
            if (gelu) {
#pragma unroll
              for (int e = 0; e < 32; ++e) xr[c][e] = gelu_erf(xr[c][e]);
            }
          }
#pragma unroll
          for (int e = 0; e < 32; ++e) ss = fmaf(xr[c][e], xr[c][e], ss);
        }
        ss = wave_sum63(ss);
        if (lane == 63) ssq[C * wid + c] = ss;
      }
      __syncthreads();
      if (busy) {
        float tot = 0.0f;
        for (int v = 0; v < C * S.wt; ++v) tot += ssq[C * ro.team0 + v];
        const float inv = 1.0f / sqrtf(tot / (float)(32 * S.nb) + S.eps);
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
          for (int e = 0; e < 32; ++e) xr[c][e] *= inv;
        if constexpr (Fmt<FMT>::kSums) unit_sums<C>(xr, xs);
      }
      xw = INT32_MAX;
    }
    const int tiw = ro.team0 / max(S.wt, 1);
    for (int j = 0; j < ro.my_iters; ++j) {
      float acc[R];
#pragma unroll
      for (int i = 0; i < R; ++i) acc[i] = 0.0f;
      const Tile done = cur;
      Tile nx = cur;
      const bool more = next_tile(cur, ro, S, nx);
      const bool now = more && (wid != 0 || nx.s == s);
      deferred = more && !now;
      if (xw != INT32_MAX && cur.w != xw) {
        // (a window with the inputs already in registers keeps them: a reload
        // would also wait for the weight prefetch, the load counter being in
        // order)
        const ChainWinDev W = S.n_win > 1 ? load_win(wins + S.win0 + cur.w) : S.w0;
        if (xw < 0 || W.x != cxp || (S.in_op == QG_IN_SILU_MUL && W.x2 != cx2p)) {
          load_x(W.x, W.x2, S.in_op == QG_IN_SILU_MUL, S.nb, ro.wit);
          cxp = W.x;
          cx2p = W.x2;
        }
        xw = cur.w;
      }
      const int nrows = cur.nrows;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        uint8_t *sb = stage[wid][i & 1];
#pragma unroll
        for (int v = 0; v < V; ++v) *(u32x4 *)(sb + lane16 + 1024 * v) = buf[i][v];
        if (now) fetch_row(i, nx);
        if (i < nrows) {
          __builtin_amdgcn_wave_barrier();
          const int ph = (int)((uintptr_t)(done.row0 + (uint32_t)i * done.rb) & 15);
          const float sp = row_partial<FMT, C>(sb, ph, lane, done.slice_n, xr, xs);
          acc[i] = wave_sum63(sp);
          __builtin_amdgcn_wave_barrier();
        }
      }
      cur = nx;
      if (S.wt == 1) {
        if (lane == 63) {
#pragma unroll
          for (int i = 0; i < R; ++i)
            if (i < nrows) {
              done.y[i] = acc[i];
              if (done.act) done.act[i] = gelu_erf(acc[i]);
            }
        }
      } else if (S.wt == kChainWaves) {
        // The team is the whole workgroup: the hardware barrier is cheaper than
        // the ring.  (Not with idle waves: they would not take these barriers.)
        if (lane == 63) {
#pragma unroll
          for (int i = 0; i < R; ++i) red[j & 1][wid][i] = acc[i];
        }
        __syncthreads();
        if (wid == 0 && lane < nrows) {
          float sum = red[j & 1][0][lane];
          for (int v = 1; v < S.wt; ++v) sum += red[j & 1][v][lane];
          done.y[lane] = sum;
          if (done.act) done.act[lane] = gelu_erf(sum);
        }
      } else {
        const int slot = j & (kRing - 1);
        const unsigned use = (unsigned)(j / kRing);
        // The slot's previous use must have been read (waits only when this
        // wave runs kRing tiles ahead of its team's slowest).
        while (__builtin_amdgcn_readfirstlane(
                   __hip_atomic_load(&consumed[tiw][slot], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) < use)
          __builtin_amdgcn_s_sleep(1);
        unsigned before = 0;
        if (lane == 63) {
#pragma unroll
          for (int i = 0; i < R; ++i) red[slot][wid][i] = acc[i];
          before = __hip_atomic_fetch_add(&arrived[tiw][slot], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        before = __builtin_amdgcn_readlane(before, 63);
        if (before == (use + 1) * (unsigned)S.wt - 1) {
          // Last of the team: every partial of this tile is in the slot.
          if (lane < nrows) {
            float sum = red[slot][ro.team0][lane];
            for (int v = 1; v < S.wt; ++v) sum += red[slot][ro.team0 + v][lane];
            done.y[lane] = sum;
            if (done.act) done.act[lane] = gelu_erf(sum);
          }
          __builtin_amdgcn_wave_barrier();
          if (lane == 0) __hip_atomic_store(&consumed[tiw][slot], use + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

thread_local std::string g_last_hip;

int hip_fail(hipError_t e, const char *what) {
  g_last_hip = std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
  return QG_E_HIP;
}

#define QG_HIP(call)                                    \
  do {                                                  \
    hipError_t e_ = (call);                             \
    if (e_ != hipSuccess) return hip_fail(e_, #call);   \
  } while (0)

int block_bytes(int32_t fmt) {
  switch (fmt) {
    case QG_Q8_0: return Fmt<QG_Q8_0>::kBytes;
    case QG_Q4_0: return Fmt<QG_Q4_0>::kBytes;
    case QG_MXFP4: return Fmt<QG_MXFP4>::kBytes;
    case QG_Q4_K: return Fmt<QG_Q4_K>::kBytes;
    case QG_Q6_K: return Fmt<QG_Q6_K>::kBytes;
    default: return QG_E_FMT;
  }
}

bool kquant(int32_t fmt) { return fmt == QG_Q4_K || fmt == QG_Q6_K; }

// Weights per block.
int block_weights(int32_t fmt) { return block_bytes(fmt) < 0 ? QG_E_FMT : kquant(fmt) ? 256 : 32; }

// Bytes of one row of k inputs (fmt and k already checked).
int64_t row_bytes_of(int32_t fmt, int64_t k) { return k / block_weights(fmt) * block_bytes(fmt); }

int check_fmt_k(int32_t fmt, int64_t k) {
  if (block_bytes(fmt) < 0) return QG_E_FMT;
  if (k <= 0 || k % block_weights(fmt) != 0) return QG_E_SHAPE;
  return QG_OK;
}

// Team shape, a function of (format, k) only.  Q8_0 and the K-quants: one
// column per lane while a row fits 12 waves (k <= 24576), else two.  Q4_0 and
// MXFP4: two columns per lane: their decode is VALU-bound, and a lane's second
// block shares the row's staging, reduction and addressing work.  The team
// has one wave per 64*C columns, so every wave owns at least one column (and,
// for the K-quants, whole super-blocks: k is a multiple of 256).
int first_c(int32_t fmt) { return fmt == QG_Q8_0 || kquant(fmt) ? 1 : 2; }

int team_shape(int32_t fmt, int64_t k, Shape *s) {
  const int64_t nb = k / 32;
  for (int c = first_c(fmt); c <= kMaxC; ++c) {
    const int64_t wt = (nb + 64 * c - 1) / (64 * c);
    if (wt <= kMaxWT) { s->wt = (int)wt; s->c = c; return QG_OK; }
  }
  return QG_E_SHAPE;  // k above 32 * 64 * kMaxWT * kMaxC = 49152
}

int tile_cap(int32_t fmt, int c) {
  switch (fmt) {
    case QG_Q8_0: return c == 1 ? TileCap<QG_Q8_0, 1>::value : TileCap<QG_Q8_0, 2>::value;
    case QG_Q4_0: return c == 1 ? TileCap<QG_Q4_0, 1>::value : TileCap<QG_Q4_0, 2>::value;
    default: return c == 1 ? TileCap<QG_MXFP4, 1>::value : TileCap<QG_MXFP4, 2>::value;
  }
}

int check_matrix(const qg_matrix *w) {
  if (!w) return QG_E_NULL;
  int rc = check_fmt_k(w->fmt, w->k);
  if (rc) return rc;
  if (w->n_rows < 0 || w->reserved != 0) return w->n_rows < 0 ? QG_E_SHAPE : QG_E_ARG;
  Shape s;
  if ((rc = team_shape(w->fmt, w->k, &s))) return rc;
  if (w->n_bytes != w->n_rows * row_bytes_of(w->fmt, w->k)) return QG_E_SIZE;
  if (!w->data && w->n_bytes > 0) return QG_E_NULL;
  if ((uintptr_t)w->data & 15) return QG_E_ARG;
  return QG_OK;
}

int check_range(int64_t n_rows, int64_t r0, int64_t r1) {
  if (r0 < 0 || r0 > r1 || r1 > n_rows) return QG_E_RANGE;
  return QG_OK;
}

int device_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// The kernel for (format, team shape, transforms); null for a combination
// that has no kernel (SiLU input with GELU output).
GemvFn pick(int32_t fmt, Shape s, int32_t in_op, int32_t out_op) {
  const bool gelu = out_op == QG_OUT_GELU;
  if (in_op == QG_IN_X) return gelu ? pick_op<kOpGelu>(fmt, s) : pick_op<kOpNone>(fmt, s);
  if (in_op == QG_IN_RMS) return gelu ? pick_op<kOpRmsGelu>(fmt, s) : pick_op<kOpRms>(fmt, s);
  if (in_op == QG_IN_SILU_MUL && !gelu) return pick_op<kOpSilu>(fmt, s);
  return nullptr;
}

// in_op / out_op / eps: the fused transforms (QG_IN_X, QG_OUT_Y: none); x2[i]
// is window i's SiLU multiplier (x2 may be null when in_op is not
// QG_IN_SILU_MUL).  nt > 1: nt tokens (2 or 4, no transform), token t's x at
// win.x + t x_stride and its y at win.y + t y_stride.  up: SwiGLU pairs,
// up[i] the row 0 of window i's up matrix (win.data the gate's; same shape),
// y[j] = silu(gate_j . x) * (up_j . x); the kernel walks virtual rows, two
// per output row.
// A GEMV launch, prepared: kernel, grid, block and arguments (fn is null for
// a launch with no rows).
struct GemvLaunch {
  GemvFn fn;
  unsigned grid, block;
  GemvArgs a;
};

int prepare_gemv(GemvLaunch *L, int32_t fmt, int64_t k, const qg_window *win_in, int n_in, int64_t block_rows,
                 int32_t in_op = QG_IN_X, float eps = 0.0f, int32_t out_op = QG_OUT_Y,
                 const float *const *x2 = nullptr, int nt = 1, int64_t x_stride = 0, int64_t y_stride = 0,
                 const void *const *up = nullptr) {
  L->fn = nullptr;
  Shape s;
  int rc = team_shape(fmt, k, &s);
  if (rc) return rc;
  const int64_t pm = up ? 2 : 1;  // virtual rows per output row
  qg_window win[kMaxWindows];
  const float *wx2[kMaxWindows];
  const void *wup[kMaxWindows];
  int n = 0;
  int64_t maxlen = 1, total = 0;
  for (int i = 0; i < n_in; ++i) {
    if (win_in[i].row_end == win_in[i].row_start) continue;
    wx2[n] = x2 ? x2[i] : nullptr;
    wup[n] = up ? up[i] : nullptr;
    win[n] = win_in[i];
    win[n].row_start *= pm;
    win[n].row_end *= pm;
    maxlen = std::max<int64_t>(maxlen, win[n].row_end - win[n].row_start);
    total += win[n].row_end - win[n].row_start;
    ++n;
  }
  if (n == 0) return QG_OK;  // (L->fn stays null: nothing to launch)
  const int64_t B = block_rows > 0 ? std::min<int64_t>(pm * block_rows, maxlen) : maxlen;
  const int64_t teams_max = std::max<int64_t>(1, (int64_t)device_cus() * gemv_teams_per_cu(fmt, s.wt));
  int tile_rows =
      (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)kGemvTileRows, B, (total + teams_max - 1) / teams_max}));
  if (up) tile_rows = std::max(2, tile_rows & ~1);  // whole pairs (B and every window are even)
  GemvArgs a;
  memset(&a, 0, sizeof(a));
  int64_t tiles = 0;
  const int64_t tpb = (B + tile_rows - 1) / tile_rows;
  for (int i = 0; i < n; ++i) {
    const int64_t len = win[i].row_end - win[i].row_start;
    const int64_t full = len / B, rem = len - full * B;
    a.win[i].base = (const uint8_t *)win[i].data;
    a.win[i].base2 = (const uint8_t *)wup[i];
    a.win[i].x = win[i].x;
    a.win[i].x2 = wx2[i];
    a.win[i].y = win[i].y;
    a.win[i].row_start = win[i].row_start;
    a.win[i].row_end = win[i].row_end;
    a.tile_prefix[i] = (int32_t)tiles;
    tiles += full * tpb + (rem + tile_rows - 1) / tile_rows;
    if (tiles > INT32_MAX / 2) return QG_E_SHAPE;
  }
  for (int i = n; i <= kMaxWindows; ++i) a.tile_prefix[i] = (int32_t)tiles;
  a.n_win = n;
  a.nb = (int32_t)(k / 32);
  a.row_bytes = row_bytes_of(fmt, k);
  a.block_rows = B;
  a.tile_rows = tile_rows;
  a.n_tiles = (int32_t)tiles;
  a.tiles_per_block = (int32_t)tpb;
  a.in_op = in_op;
  a.out_op = out_op;
  a.eps = eps;
  a.x_stride = x_stride;
  a.y_stride = y_stride;
  const int64_t teams = std::min<int64_t>(teams_max, tiles);
  const GemvFn fn = up ? (in_op == QG_IN_RMS ? pick_op<kOpRmsSwiglu>(fmt, s)
                          : in_op == QG_IN_X  ? pick_op<kOpSwiglu>(fmt, s)
                                              : nullptr)
                    : nt == 1 ? pick(fmt, s, in_op, out_op)
                    : nt == 2 && in_op == QG_IN_X && out_op == QG_OUT_Y ? pick_batch<2>(fmt, s)
                    : nt == 4 && in_op == QG_IN_X && out_op == QG_OUT_Y ? pick_batch<4>(fmt, s)
                                                                        : nullptr;
  if (!fn) return QG_E_ARG;
  L->fn = fn;
  L->grid = (unsigned)teams;
  L->block = 64u * (unsigned)s.wt;
  L->a = a;
  return QG_OK;
}

int launch_gemv(int32_t fmt, int64_t k, const qg_window *win_in, int n_in, int64_t block_rows,
                hipStream_t stream, int32_t in_op = QG_IN_X, float eps = 0.0f, int32_t out_op = QG_OUT_Y,
                const float *const *x2 = nullptr, int nt = 1, int64_t x_stride = 0, int64_t y_stride = 0,
                const void *const *up = nullptr) {
  static thread_local GemvLaunch L;  // (4 KB of arguments: kept off the stack)
  int rc = prepare_gemv(&L, fmt, k, win_in, n_in, block_rows, in_op, eps, out_op, x2, nt, x_stride, y_stride, up);
  if (rc || !L.fn) return rc;
  hipLaunchKernelGGL(L.fn, dim3(L.grid), dim3(L.block), 0, stream, L.a.win[0].x, L.a.nb, L.a.n_tiles, L.a);
  QG_HIP(hipGetLastError());
  return QG_OK;
}

int validate_windows(int32_t fmt, int64_t k, const qg_window *win, int32_t n_win, int64_t block_rows) {
  int rc = check_fmt_k(fmt, k);
  if (rc) return rc;
  Shape s;
  if ((rc = team_shape(fmt, k, &s))) return rc;
  if (n_win < 0 || n_win > kMaxWindows || block_rows < 0) return QG_E_ARG;
  if (n_win > 0 && !win) return QG_E_NULL;
  for (int i = 0; i < n_win; ++i) {
    if (win[i].n_rows < 0) return QG_E_SHAPE;
    if ((rc = check_range(win[i].n_rows, win[i].row_start, win[i].row_end))) return rc;
    if (win[i].row_end > win[i].row_start && (!win[i].data || !win[i].x || !win[i].y)) return QG_E_NULL;
    if ((uintptr_t)win[i].data & 15) return QG_E_ARG;
  }
  return QG_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

namespace {
// The streamers' copy streams: kCopyStreams non-blocking streams per device,
// created on first use and kept until the process ends.
constexpr int kCopyStreams = 2;

hipError_t copy_pool(int device, hipStream_t **out) {
  static std::mutex mu;
  static hipStream_t pool[64][kCopyStreams] = {};
  if (device < 0 || device >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  for (int i = 0; i < kCopyStreams; ++i)
    if (!pool[device][i]) {
      hipError_t e = hipStreamCreateWithFlags(&pool[device][i], hipStreamNonBlocking);
      if (e != hipSuccess) {
        pool[device][i] = nullptr;
        return e;
      }
    }
  *out = pool[device];
  return hipSuccess;
}
}  // namespace

struct qg_streamer {
  int device;
  int64_t slot_bytes;
  int64_t slot_stride;  // slot_bytes rounded up to 256 (slots stay 16-byte aligned)
  int lookahead;
  uint8_t *ring;
  // Copy streams, used in turn by consecutive blocks (slot s takes stream
  // s mod their count), so that two host->device copies can run at once.
  // They come from a per-device pool created once per process: the runtime
  // spreads streams over a few hardware queues as they are created, and
  // streams made and dropped per streamer ended up sharing the caller's
  // queue now and then, which serialised copies with kernels.
  std::vector<hipStream_t> copies;
  std::vector<hipEvent_t> ready, freed;
  std::vector<char> freed_valid;
  uint64_t next;
};

extern "C" {

const char *qgemv_version(void) { return "0.1.0"; }

const char *qgemv_strerror(int status) {
  switch (status) {
    case QG_OK: return "ok";
    case QG_E_NULL: return "a required pointer is NULL";
    case QG_E_FMT: return "unknown quantization format";
    case QG_E_SHAPE: return "bad shape (k must be a positive multiple of 32 (256 for K-quants), at most 49152; n_rows >= 0)";
    case QG_E_RANGE: return "row range or expert id out of range";
    case QG_E_SIZE: return "n_bytes does not match n_rows * (k/QK) * block bytes";
    case QG_E_ARG: return "bad argument (block_rows, lookahead, window count, n, eps, stride, or weights not 16-byte aligned)";
    case QG_E_NOT_PINNED: return "streamed weights are not in page-locked host memory";
    case QG_E_CAPACITY: return "a row block is larger than a ring slot";
    case QG_E_BARRIER: return "a chain's device-wide barrier gave up waiting (workgroups not co-resident)";
    case QG_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *qgemv_last_hip_error(void) { return g_last_hip.c_str(); }

int64_t qgemv_block_bytes(int32_t fmt) { return block_bytes(fmt); }

int64_t qgemv_block_weights(int32_t fmt) { return block_weights(fmt); }

int64_t qgemv_weight_bytes(int32_t fmt, int64_t n_rows, int64_t k) {
  int rc = check_fmt_k(fmt, k);
  if (rc) return rc;
  if (n_rows < 0) return QG_E_SHAPE;
  return n_rows * row_bytes_of(fmt, k);
}

int qgemv_rows(const qg_matrix *w, int64_t row_start, int64_t row_end, const float *x, float *y,
               int64_t block_rows, qg_stream_t stream) {
  int rc = check_matrix(w);
  if (rc) return rc;
  if ((rc = check_range(w->n_rows, row_start, row_end))) return rc;
  if (block_rows < 0) return QG_E_ARG;
  if (row_end == row_start) return QG_OK;
  if (!x || !y) return QG_E_NULL;
  qg_window win = {w->data, w->n_rows, row_start, row_end, x, y};
  return launch_gemv(w->fmt, w->k, &win, 1, block_rows, stream);
}

int qgemv_rows_batch(const qg_matrix *w, int64_t row_start, int64_t row_end, const float *x, int64_t x_stride,
                     int32_t n_tok, float *y, int64_t y_stride, int64_t block_rows, qg_stream_t stream) {
  int rc = check_matrix(w);
  if (rc) return rc;
  if ((rc = check_range(w->n_rows, row_start, row_end))) return rc;
  const int64_t n = row_end - row_start;
  if (block_rows < 0 || n_tok < 0 || x_stride < 0 || (n_tok > 1 && y_stride < n)) return QG_E_ARG;
  if (n == 0 || n_tok == 0) return QG_OK;
  if (!x || !y) return QG_E_NULL;
  Shape s;
  if ((rc = team_shape(w->fmt, w->k, &s))) return rc;
  qg_window win = {w->data, w->n_rows, row_start, row_end, nullptr, nullptr};
  // passes of four tokens (two, one) while the team shape allows
  for (int32_t t = 0; t < n_tok;) {
    const int32_t left = n_tok - t;
    const int nt = left >= 4 && s.wt <= batch_max_wt(4, s.c) ? 4 : left >= 2 && s.wt <= batch_max_wt(2, s.c) ? 2 : 1;
    win.x = x + (int64_t)t * x_stride;
    win.y = y + (int64_t)t * y_stride;
    if ((rc = launch_gemv(w->fmt, w->k, &win, 1, block_rows, stream, QG_IN_X, 0.0f, QG_OUT_Y, nullptr, nt,
                          x_stride, y_stride)))
      return rc;
    t += nt;
  }
  return QG_OK;
}

int qgemv_rows_mfma(const qg_matrix *w, int64_t row_start, int64_t row_end, const float *x, int64_t x_stride,
                    int32_t n_tok, float *y, int64_t y_stride, qg_stream_t stream) {
  int rc = check_matrix(w);
  if (rc) return rc;
  if ((rc = check_range(w->n_rows, row_start, row_end))) return rc;
  const int64_t n = row_end - row_start;
  if (n_tok < 0 || x_stride < 0 || (n_tok > 1 && y_stride < n)) return QG_E_ARG;
  if (n == 0 || n_tok == 0) return QG_OK;
  if (!x || !y) return QG_E_NULL;
  const int64_t rb = row_bytes_of(w->fmt, w->k);
  MfmaArgs a;
  a.w = (const uint8_t *)w->data + row_start * rb;
  a.row_bytes = rb;
  a.n_rows = n;
  a.x_stride = x_stride;
  a.y_stride = y_stride;
  a.nb = (int32_t)(w->k / 32);  // 32-weight units (a K-quant super-block is 8)
  // passes of 16 tokens, each reading the weights once
  for (int32_t t = 0; t < n_tok; t += 16) {
    a.x = x + (int64_t)t * x_stride;
    a.y = y + (int64_t)t * y_stride;
    a.n_tok = std::min<int32_t>(16, n_tok - t);
    if ((rc = launch_gemv_mfma(w->fmt, a, (hipStream_t)stream))) return rc;
    QG_HIP(hipGetLastError());
  }
  return QG_OK;
}

int qgemv_rows_op(const qg_matrix *w, int64_t row_start, int64_t row_end, const float *x, const float *x2,
                  int32_t in_op, float eps, int32_t out_op, float *y, int64_t block_rows, qg_stream_t stream) {
  int rc = check_matrix(w);
  if (rc) return rc;
  if ((rc = check_range(w->n_rows, row_start, row_end))) return rc;
  if (block_rows < 0) return QG_E_ARG;
  if (in_op != QG_IN_X && in_op != QG_IN_RMS && in_op != QG_IN_SILU_MUL) return QG_E_ARG;
  if (out_op != QG_OUT_Y && out_op != QG_OUT_GELU) return QG_E_ARG;
  if (in_op == QG_IN_SILU_MUL && out_op == QG_OUT_GELU) return QG_E_ARG;
  if (in_op == QG_IN_RMS && (!(eps >= 0.0f) || eps > 3.0e38f || w->k > kMaxRmsK)) return QG_E_ARG;
  if (row_end == row_start) return QG_OK;
  if (!x || !y || (in_op == QG_IN_SILU_MUL && !x2)) return QG_E_NULL;
  qg_window win = {w->data, w->n_rows, row_start, row_end, x, y};
  return launch_gemv(w->fmt, w->k, &win, 1, block_rows, stream, in_op, eps, out_op, &x2);
}

int qgemv_windows(int32_t fmt, int64_t k, const qg_window *win, int32_t n_win, int64_t block_rows,
                  qg_stream_t stream) {
  int rc = validate_windows(fmt, k, win, n_win, block_rows);
  if (rc) return rc;
  if (n_win == 0) return QG_OK;
  return launch_gemv(fmt, k, win, n_win, block_rows, stream);
}

// The windows of the selected experts, with optional fused transforms: window
// (m, s) reads x + s x_stride (and x2 + s x_stride for QG_IN_SILU_MUL).
int expert_windows(const qg_matrix *mats, int32_t n_mat, int64_t n_expert, const int32_t *ids, int32_t n_sel,
                   const float *x, int64_t x_stride, const float *x2, int32_t in_op, float eps, int32_t out_op,
                   float *y, int64_t block_rows, hipStream_t stream) {
  if (!mats || (n_sel > 0 && !ids)) return QG_E_NULL;
  if (n_mat < 1 || n_sel < 0 || (int64_t)n_mat * n_sel > kMaxWindows || x_stride < 0 || block_rows < 0)
    return QG_E_ARG;
  if (n_expert <= 0) return QG_E_SHAPE;
  int rc;
  for (int m = 0; m < n_mat; ++m) {
    if ((rc = check_matrix(&mats[m]))) return rc;
    if (mats[m].fmt != mats[0].fmt || mats[m].k != mats[0].k || mats[m].n_rows != mats[0].n_rows)
      return QG_E_SHAPE;
  }
  if (mats[0].n_rows % n_expert != 0) return QG_E_SHAPE;
  const int64_t out = mats[0].n_rows / n_expert;
  for (int s = 0; s < n_sel; ++s)
    if (ids[s] < 0 || ids[s] >= n_expert) return QG_E_RANGE;
  if (in_op != QG_IN_X && in_op != QG_IN_RMS && in_op != QG_IN_SILU_MUL) return QG_E_ARG;
  if (out_op != QG_OUT_Y && out_op != QG_OUT_GELU) return QG_E_ARG;
  if (in_op == QG_IN_SILU_MUL && out_op == QG_OUT_GELU) return QG_E_ARG;
  if (in_op == QG_IN_RMS && (!(eps >= 0.0f) || eps > 3.0e38f || mats[0].k > kMaxRmsK)) return QG_E_ARG;
  if (n_sel == 0 || out == 0) return QG_OK;
  if (!x || !y || (in_op == QG_IN_SILU_MUL && !x2)) return QG_E_NULL;
  qg_window win[kMaxWindows];
  const float *wx2[kMaxWindows];
  int n = 0;
  for (int m = 0; m < n_mat; ++m)
    for (int s = 0; s < n_sel; ++s) {
      win[n].data = mats[m].data;
      win[n].n_rows = mats[m].n_rows;
      win[n].row_start = (int64_t)ids[s] * out;
      win[n].row_end = (int64_t)(ids[s] + 1) * out;
      win[n].x = x + (int64_t)s * x_stride;
      win[n].y = y + ((int64_t)m * n_sel + s) * out;
      wx2[n] = x2 ? x2 + (int64_t)s * x_stride : nullptr;
      ++n;
    }
  return launch_gemv(mats[0].fmt, mats[0].k, win, n, block_rows, stream, in_op, eps, out_op, wx2);
}

int qgemv_expert_windows(const qg_matrix *mats, int32_t n_mat, int64_t n_expert, const int32_t *ids,
                         int32_t n_sel, const float *x, int64_t x_stride, float *y, int64_t block_rows,
                         qg_stream_t stream) {
  return expert_windows(mats, n_mat, n_expert, ids, n_sel, x, x_stride, nullptr, QG_IN_X, 0.0f, QG_OUT_Y, y,
                        block_rows, stream);
}

int qgemv_expert_windows_op(const qg_matrix *mats, int32_t n_mat, int64_t n_expert, const int32_t *ids,
                            int32_t n_sel, const float *x, const float *x2, int64_t x_stride, int32_t in_op,
                            float eps, int32_t out_op, float *y, int64_t block_rows, qg_stream_t stream) {
  return expert_windows(mats, n_mat, n_expert, ids, n_sel, x, x_stride, x2, in_op, eps, out_op, y, block_rows,
                        stream);
}

namespace {
// Checks shared by the SwiGLU-pair entry points: gate and up are twins.
int check_pair(const qg_matrix *gate, const qg_matrix *up, int32_t in_op, float eps) {
  int rc = check_matrix(gate);
  if (rc) return rc;
  if ((rc = check_matrix(up))) return rc;
  if (up->fmt != gate->fmt || up->k != gate->k || up->n_rows != gate->n_rows) return QG_E_SHAPE;
  if (in_op != QG_IN_X && in_op != QG_IN_RMS) return QG_E_ARG;
  if (in_op == QG_IN_RMS && (!(eps >= 0.0f) || eps > 3.0e38f || gate->k > kMaxRmsK)) return QG_E_ARG;
  return QG_OK;
}
}  // namespace

int qgemv_rows_swiglu(const qg_matrix *gate, const qg_matrix *up, int64_t row_start, int64_t row_end,
                      const float *x, int32_t in_op, float eps, float *h, int64_t block_rows, qg_stream_t stream) {
  if (!gate || !up) return QG_E_NULL;
  int rc = check_pair(gate, up, in_op, eps);
  if (rc) return rc;
  if ((rc = check_range(gate->n_rows, row_start, row_end))) return rc;
  if (block_rows < 0) return QG_E_ARG;
  if (row_end == row_start) return QG_OK;
  if (!x || !h) return QG_E_NULL;
  qg_window win = {gate->data, gate->n_rows, row_start, row_end, x, h};
  const void *upd = up->data;
  return launch_gemv(gate->fmt, gate->k, &win, 1, block_rows, stream, in_op, eps, QG_OUT_Y, nullptr, 1, 0, 0, &upd);
}

int qgemv_expert_swiglu(const qg_matrix *gate, const qg_matrix *up, int64_t n_expert, const int32_t *ids,
                        int32_t n_sel, const float *x, int64_t x_stride, int32_t in_op, float eps, float *h,
                        int64_t block_rows, qg_stream_t stream) {
  if (!gate || !up || (n_sel > 0 && !ids)) return QG_E_NULL;
  int rc = check_pair(gate, up, in_op, eps);
  if (rc) return rc;
  if (n_sel < 0 || n_sel > kMaxWindows || x_stride < 0 || block_rows < 0) return QG_E_ARG;
  if (n_expert <= 0 || gate->n_rows % n_expert != 0) return QG_E_SHAPE;
  const int64_t out = gate->n_rows / n_expert;
  for (int s = 0; s < n_sel; ++s)
    if (ids[s] < 0 || ids[s] >= n_expert) return QG_E_RANGE;
  if (n_sel == 0 || out == 0) return QG_OK;
  if (!x || !h) return QG_E_NULL;
  qg_window win[kMaxWindows];
  const void *upd[kMaxWindows];
  for (int s = 0; s < n_sel; ++s) {
    win[s] = {gate->data, gate->n_rows, (int64_t)ids[s] * out, (int64_t)(ids[s] + 1) * out,
              x + (int64_t)s * x_stride, h + (int64_t)s * out};
    upd[s] = up->data;
  }
  return launch_gemv(gate->fmt, gate->k, win, n_sel, block_rows, stream, in_op, eps, QG_OUT_Y, nullptr, 1, 0, 0,
                     upd);
}

int qgemv_combine(const float *y, int64_t y_stride, int32_t n_sel, const float *w, int64_t n, float *out,
                  qg_stream_t stream) {
  if (n < 0 || n_sel < 0 || (n_sel > 1 && y_stride < n)) return QG_E_ARG;
  if (n == 0) return QG_OK;
  if (!out || (n_sel > 0 && (!y || !w))) return QG_E_NULL;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, y, y_stride, n_sel, w, n, out);
  QG_HIP(hipGetLastError());
  return QG_OK;
}

int qgemv_read_ceiling(const void *data, int64_t n_bytes, uint32_t *sink, qg_stream_t stream) {
  if (!data || !sink) return QG_E_NULL;
  if (n_bytes <= 0 || n_bytes % 16 != 0 || ((uintptr_t)data & 15)) return QG_E_ARG;
  hipLaunchKernelGGL(read_kernel, dim3(kReadGroups), dim3(kReadThreads), 0, stream, (const u32x4 *)data,
                     n_bytes / 16, sink);
  QG_HIP(hipGetLastError());
  return QG_OK;
}

int qgemv_silu_mul(const float *g, const float *u, float *h, int64_t n, qg_stream_t stream) {
  if (n < 0) return QG_E_ARG;
  if (n == 0) return QG_OK;
  if (!g || !u || !h) return QG_E_NULL;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, g, u, h, n);
  QG_HIP(hipGetLastError());
  return QG_OK;
}

int qgemv_rms_carry(const float *v, float *out, int64_t n, float eps, int32_t gelu, qg_stream_t stream) {
  if (n < 1 || !(eps >= 0.0f) || (gelu != 0 && gelu != 1)) return QG_E_ARG;
  if (!v || !out) return QG_E_NULL;
  hipLaunchKernelGGL(rms_carry_kernel, dim3(1), dim3(kCarryThreads), 0, stream, v, out, n, eps, (int)gelu);
  QG_HIP(hipGetLastError());
  return QG_OK;
}

int qgemv_dequant_rows(const qg_matrix *w, int64_t row_start, int64_t row_end, float *out,
                       qg_stream_t stream) {
  int rc = check_matrix(w);
  if (rc) return rc;
  if ((rc = check_range(w->n_rows, row_start, row_end))) return rc;
  if (row_end == row_start) return QG_OK;
  if (!out) return QG_E_NULL;
  const int nb = (int)(w->k / 32);
  const int64_t rb = row_bytes_of(w->fmt, w->k);
  const int64_t n = (row_end - row_start) * nb;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  const uint8_t *base = (const uint8_t *)w->data;
  switch (w->fmt) {
    case QG_Q8_0:
      hipLaunchKernelGGL(dequant_kernel<QG_Q8_0>, dim3(blocks), dim3(256), 0, stream, base, row_start,
                         row_end - row_start, nb, rb, out);
      break;
    case QG_Q4_0:
      hipLaunchKernelGGL(dequant_kernel<QG_Q4_0>, dim3(blocks), dim3(256), 0, stream, base, row_start,
                         row_end - row_start, nb, rb, out);
      break;
    case QG_Q4_K:
      hipLaunchKernelGGL(dequant_kernel<QG_Q4_K>, dim3(blocks), dim3(256), 0, stream, base, row_start,
                         row_end - row_start, nb, rb, out);
      break;
    case QG_Q6_K:
      hipLaunchKernelGGL(dequant_kernel<QG_Q6_K>, dim3(blocks), dim3(256), 0, stream, base, row_start,
                         row_end - row_start, nb, rb, out);
      break;
    default:
      hipLaunchKernelGGL(dequant_kernel<QG_MXFP4>, dim3(blocks), dim3(256), 0, stream, base, row_start,
                         row_end - row_start, nb, rb, out);
  }
  QG_HIP(hipGetLastError());
  return QG_OK;
}

// ---- streamer ---------------------------------------------------------------

int qgemv_stream_create(int64_t slot_bytes, int32_t lookahead, qg_streamer **out) {
  if (!out) return QG_E_NULL;
  if (slot_bytes < 1 || lookahead < 1 || lookahead > 64) return QG_E_ARG;
  *out = nullptr;
  qg_streamer *st = new qg_streamer();
  st->slot_bytes = slot_bytes;
  st->slot_stride = (slot_bytes + 255) / 256 * 256;
  st->lookahead = lookahead;
  st->ring = nullptr;
  st->next = 0;
  const int n = lookahead + 1;
  auto fail = [&](hipError_t e, const char *what) {
    int rc = hip_fail(e, what);
    qgemv_stream_destroy(st);
    return rc;
  };
  hipError_t e;
  if ((e = hipGetDevice(&st->device)) != hipSuccess) return fail(e, "hipGetDevice");
  if ((e = hipMalloc((void **)&st->ring, (size_t)st->slot_stride * n)) != hipSuccess) return fail(e, "hipMalloc(ring)");
  hipStream_t *pool = nullptr;
  if ((e = copy_pool(st->device, &pool)) != hipSuccess) return fail(e, "hipStreamCreateWithFlags");
  st->copies.assign(pool, pool + std::min(lookahead, kCopyStreams));
  st->ready.assign(n, nullptr);
  st->freed.assign(n, nullptr);
  st->freed_valid.assign(n, 0);
  for (int i = 0; i < n; ++i) {
    if ((e = hipEventCreateWithFlags(&st->ready[i], hipEventDisableTiming)) != hipSuccess)
      return fail(e, "hipEventCreateWithFlags");
    if ((e = hipEventCreateWithFlags(&st->freed[i], hipEventDisableTiming)) != hipSuccess)
      return fail(e, "hipEventCreateWithFlags");
  }
  if ((e = hipDeviceSynchronize()) != hipSuccess) return fail(e, "hipDeviceSynchronize");
  *out = st;
  return QG_OK;
}

int64_t qgemv_stream_ring_bytes(const qg_streamer *st) {
  if (!st) return QG_E_NULL;
  return st->slot_bytes * (st->lookahead + 1);
}

int qgemv_stream_destroy(qg_streamer *st) {
  if (!st) return QG_OK;
  int rc = QG_OK;
  hipError_t e;
  for (auto cs : st->copies)
    if (cs && (e = hipStreamSynchronize(cs)) != hipSuccess && rc == QG_OK) rc = hip_fail(e, "hipStreamSynchronize");
  for (auto ev : st->freed)
    if (ev) {
      if ((e = hipEventSynchronize(ev)) != hipSuccess && rc == QG_OK) rc = hip_fail(e, "hipEventSynchronize");
      (void)hipEventDestroy(ev);
    }
  for (auto ev : st->ready)
    if (ev) (void)hipEventDestroy(ev);
  // (the copy streams belong to the per-device pool and stay)
  if (st->ring) (void)hipFree(st->ring);
  delete st;
  return rc;
}

namespace {

int check_pinned(const void *p) {
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof(attr));
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return QG_E_NOT_PINNED;
  }
  if (attr.type != hipMemoryTypeHost) return QG_E_NOT_PINNED;
  return QG_OK;
}

// The device address of page-locked host memory (hipHostMalloc; mapped into
// every device's address space), or QG_E_NOT_PINNED for pageable or device
// memory.  Checked before anything is enqueued.
int mapped_alias(const void *host, const void **dev) {
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof(attr));
  hipError_t e = hipPointerGetAttributes(&attr, host);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return QG_E_NOT_PINNED;
  }
  if (attr.type != hipMemoryTypeHost || !attr.devicePointer) return QG_E_NOT_PINNED;
  if ((uintptr_t)attr.devicePointer & 15) return QG_E_ARG;
  *dev = attr.devicePointer;
  return QG_OK;
}

// Stream the row blocks of validated windows through the ring.
int stream_windows(qg_streamer *st, int32_t fmt, int64_t k, const qg_window *win, int n_win,
                   int64_t block_rows, hipStream_t stream) {
  const int64_t rb = row_bytes_of(fmt, k);
  const int nslot = st->lookahead + 1;
  // every block must fit a slot; check all before enqueueing anything
  for (int i = 0; i < n_win; ++i) {
    const int64_t len = win[i].row_end - win[i].row_start;
    if (len == 0) continue;
    const int64_t B = block_rows > 0 ? std::min(block_rows, len) : len;
    if (B * rb > st->slot_bytes) return QG_E_CAPACITY;
    int rc = check_pinned(win[i].data);
    if (rc) return rc;
  }
  for (int i = 0; i < n_win; ++i) {
    const int64_t len = win[i].row_end - win[i].row_start;
    const int64_t B = block_rows > 0 ? block_rows : len;
    for (int64_t r = win[i].row_start; r < win[i].row_end; r += B) {
      const int64_t n = std::min(B, win[i].row_end - r);
      const int slot = (int)(st->next++ % (uint64_t)nslot);
      uint8_t *dst = st->ring + (int64_t)slot * st->slot_stride;
      hipStream_t cs = st->copies[slot % st->copies.size()];
      if (st->freed_valid[slot]) QG_HIP(hipStreamWaitEvent(cs, st->freed[slot], 0));
      QG_HIP(hipMemcpyAsync(dst, (const uint8_t *)win[i].data + r * rb, (size_t)(n * rb),
                            hipMemcpyHostToDevice, cs));
      QG_HIP(hipEventRecord(st->ready[slot], cs));
      QG_HIP(hipStreamWaitEvent(stream, st->ready[slot], 0));
      qg_window blk = {dst, n, 0, n, win[i].x, win[i].y + (r - win[i].row_start)};
      int rc = launch_gemv(fmt, k, &blk, 1, 0, stream);
      if (rc) return rc;
      QG_HIP(hipEventRecord(st->freed[slot], stream));
      st->freed_valid[slot] = 1;
    }
  }
  return QG_OK;
}

}  // namespace

int qgemv_stream_rows(qg_streamer *st, const qg_matrix *w, int64_t row_start, int64_t row_end,
                      int64_t block_rows, const float *x, float *y, qg_stream_t stream) {
  if (!st) return QG_E_NULL;
  int rc = check_matrix(w);
  if (rc) return rc;
  if ((rc = check_range(w->n_rows, row_start, row_end))) return rc;
  if (block_rows < 0) return QG_E_ARG;
  if (row_end == row_start) return QG_OK;
  if (!x || !y) return QG_E_NULL;
  qg_window win = {w->data, w->n_rows, row_start, row_end, x, y};
  return stream_windows(st, w->fmt, w->k, &win, 1, block_rows, stream);
}

int qgemv_stream_windows(qg_streamer *st, int32_t fmt, int64_t k, const qg_window *win, int32_t n_win,
                         int64_t block_rows, qg_stream_t stream) {
  if (!st) return QG_E_NULL;
  int rc = validate_windows(fmt, k, win, n_win, block_rows);
  if (rc) return rc;
  if (n_win == 0) return QG_OK;
  return stream_windows(st, fmt, k, win, n_win, block_rows, stream);
}

// ---- streamed plans: a layer's streamed steps as one replayed graph ---------------

}  // extern "C"

struct qg_stream_plan {
  int device;
  uint8_t *ring;
  int64_t slot_bytes, slot_stride;
  int lookahead;
  hipGraph_t graph;
  hipGraphExec_t exec;
  // Per plan window: its pinned host matrix, row bytes, rows, current first
  // row and length; and its copy nodes (node, first row of the block within
  // the window, bytes, ring destination) for re-pointing.
  struct Copy {
    hipGraphNode_t node;
    int64_t off, bytes;
    void *dst;
  };
  struct Win {
    const uint8_t *host;
    int64_t rb, n_rows, row_start, len;
    bool streamed;
    std::vector<Copy> copies;
  };
  std::vector<Win> wins;
};

namespace {

int plan_destroy(qg_stream_plan *p) {
  if (!p) return QG_OK;
  hipError_t e = hipDeviceSynchronize();
  if (p->exec) (void)hipGraphExecDestroy(p->exec);
  if (p->graph) (void)hipGraphDestroy(p->graph);
  if (p->ring) (void)hipFree(p->ring);
  delete p;
  return e == hipSuccess ? QG_OK : hip_fail(e, "hipDeviceSynchronize");
}

int validate_plan(int64_t slot_bytes, int32_t lookahead, const qg_plan_step *steps, int32_t n_steps,
                  const qg_window *win, int32_t n_win) {
  if (!steps || (n_win > 0 && !win)) return QG_E_NULL;
  if (slot_bytes < 1 || lookahead < 1 || lookahead > 64 || n_steps < 1 || n_win < 0) return QG_E_ARG;
  std::vector<char> used(n_win, 0);
  for (int i = 0; i < n_steps; ++i) {
    const qg_plan_step &S = steps[i];
    int rc;
    if (S.op == QG_PLAN_GEMV) {
      if (S.n_win < 1 || S.first_win < 0 || S.first_win > n_win - S.n_win) return QG_E_ARG;
      if ((rc = validate_windows(S.fmt, S.k, win + S.first_win, S.n_win, S.block_rows))) return rc;
      const int64_t rb = row_bytes_of(S.fmt, S.k);
      for (int w = S.first_win; w < S.first_win + S.n_win; ++w) {
        if (used[w]) return QG_E_ARG;  // a window belongs to one step
        used[w] = 1;
        const int64_t len = win[w].row_end - win[w].row_start;
        if (len == 0) continue;
        const int64_t B = S.block_rows > 0 ? std::min(S.block_rows, len) : len;
        if (B * rb > slot_bytes) return QG_E_CAPACITY;
        if ((rc = check_pinned(win[w].data))) return rc;
      }
    } else if (S.op == QG_PLAN_SILU_MUL) {
      if (S.n < 0) return QG_E_ARG;
      if (S.n > 0 && (!S.a || !S.b || !S.out)) return QG_E_NULL;
    } else if (S.op == QG_PLAN_COMBINE) {
      if (S.n < 0 || S.n_sel < 0 || (S.n_sel > 1 && S.stride < S.n)) return QG_E_ARG;
      if (S.n > 0 && (!S.out || (S.n_sel > 0 && (!S.a || !S.b)))) return QG_E_NULL;
    } else {
      return QG_E_ARG;
    }
  }
  return QG_OK;
}

}  // namespace

extern "C" {

int qgemv_stream_plan_create(int64_t slot_bytes, int32_t lookahead, const qg_plan_step *steps, int32_t n_steps,
                             const qg_window *win, int32_t n_win, qg_stream_plan **out) {
  if (!out) return QG_E_NULL;
  *out = nullptr;
  int rc = validate_plan(slot_bytes, lookahead, steps, n_steps, win, n_win);
  if (rc) return rc;
  qg_stream_plan *p = new qg_stream_plan();
  p->slot_bytes = slot_bytes;
  p->slot_stride = (slot_bytes + 255) / 256 * 256;
  p->lookahead = lookahead;
  auto fail = [&](int code) {
    plan_destroy(p);
    return code;
  };
  auto hfail = [&](hipError_t e, const char *what) {
    int code = hip_fail(e, what);
    plan_destroy(p);
    return code;
  };
  hipError_t e;
  if ((e = hipGetDevice(&p->device)) != hipSuccess) return hfail(e, "hipGetDevice");
  const int nslot = lookahead + 1;
  if ((e = hipMalloc((void **)&p->ring, (size_t)p->slot_stride * nslot)) != hipSuccess) return hfail(e, "hipMalloc(ring)");
  if ((e = hipGraphCreate(&p->graph, 0)) != hipSuccess) return hfail(e, "hipGraphCreate");
  p->wins.resize(n_win);
  for (int w = 0; w < n_win; ++w) {
    p->wins[w].host = (const uint8_t *)win[w].data;
    p->wins[w].n_rows = win[w].n_rows;
    p->wins[w].row_start = win[w].row_start;
    p->wins[w].len = win[w].row_end - win[w].row_start;
    p->wins[w].streamed = false;
  }
  // Compute nodes (GEMV blocks, elementwise steps) run in program order, one
  // after the other; block b's copy waits only for the kernel that last read
  // its ring slot (block b - lookahead - 1), so copies run ahead across steps.
  std::vector<hipGraphNode_t> kern;  // kernel node of every streamed block, in order
  hipGraphNode_t prev = nullptr;     // the last compute node
  static thread_local GemvLaunch L;
  for (int i = 0; i < n_steps; ++i) {
    const qg_plan_step &S = steps[i];
    if (S.op == QG_PLAN_GEMV) {
      const int64_t rb = row_bytes_of(S.fmt, S.k);
      for (int w = S.first_win; w < S.first_win + S.n_win; ++w) {
        qg_stream_plan::Win &W = p->wins[w];
        W.rb = rb;
        W.streamed = true;
        if (W.len == 0) continue;
        const int64_t B = S.block_rows > 0 ? std::min(S.block_rows, W.len) : W.len;
        for (int64_t off = 0; off < W.len; off += B) {
          const int64_t n = std::min(B, W.len - off);
          const size_t b = kern.size();
          uint8_t *dst = p->ring + (int64_t)(b % (size_t)nslot) * p->slot_stride;
          hipGraphNode_t cn;
          hipGraphNode_t cdep = b >= (size_t)nslot ? kern[b - nslot] : nullptr;
          if ((e = hipGraphAddMemcpyNode1D(&cn, p->graph, cdep ? &cdep : nullptr, cdep ? 1 : 0, dst,
                                           W.host + (W.row_start + off) * rb, (size_t)(n * rb),
                                           hipMemcpyHostToDevice)) != hipSuccess)
            return hfail(e, "hipGraphAddMemcpyNode1D");
          W.copies.push_back({cn, off, n * rb, dst});
          qg_window blk = {dst, n, 0, n, win[w].x, win[w].y + off};
          if ((rc = prepare_gemv(&L, S.fmt, S.k, &blk, 1, 0))) return fail(rc);
          const float *x_first = L.a.win[0].x;
          int32_t nb_first = L.a.nb, tiles_first = L.a.n_tiles;
          void *args[] = {&x_first, &nb_first, &tiles_first, &L.a};
          hipKernelNodeParams kp = {};
          kp.func = (void *)L.fn;
          kp.gridDim = dim3(L.grid);
          kp.blockDim = dim3(L.block);
          kp.sharedMemBytes = 0;
          kp.kernelParams = args;
          kp.extra = nullptr;
          hipGraphNode_t deps[2] = {cn, prev};
          hipGraphNode_t kn;
          if ((e = hipGraphAddKernelNode(&kn, p->graph, deps, prev ? 2 : 1, &kp)) != hipSuccess)
            return hfail(e, "hipGraphAddKernelNode");
          kern.push_back(kn);
          prev = kn;
        }
      }
    } else if (S.n > 0 && (S.op == QG_PLAN_SILU_MUL || S.n_sel >= 0)) {
      const unsigned blocks = (unsigned)std::min<int64_t>((S.n + 255) / 256, 4096);
      hipKernelNodeParams kp = {};
      kp.gridDim = dim3(blocks);
      kp.blockDim = dim3(256);
      kp.extra = nullptr;
      const float *a = S.a, *b = S.b;
      float *o = S.out;
      int64_t n = S.n, stride = S.stride;
      int n_sel = S.n_sel;
      void *sargs[] = {&a, &b, &o, &n};
      void *cargs[] = {&a, &stride, &n_sel, &b, &n, &o};
      if (S.op == QG_PLAN_SILU_MUL) {
        kp.func = (void *)silu_mul_kernel;
        kp.kernelParams = sargs;
      } else {
        kp.func = (void *)combine_kernel;
        kp.kernelParams = cargs;
      }
      hipGraphNode_t kn;
      if ((e = hipGraphAddKernelNode(&kn, p->graph, prev ? &prev : nullptr, prev ? 1 : 0, &kp)) != hipSuccess)
        return hfail(e, "hipGraphAddKernelNode");
      prev = kn;
    }
  }
  if ((e = hipGraphInstantiate(&p->exec, p->graph, nullptr, nullptr, 0)) != hipSuccess)
    return hfail(e, "hipGraphInstantiate");
  *out = p;
  return QG_OK;
}

int qgemv_stream_plan_set_rows(qg_stream_plan *p, int32_t w, int64_t row_start) {
  if (!p) return QG_E_NULL;
  if (w < 0 || w >= (int32_t)p->wins.size() || !p->wins[w].streamed) return QG_E_ARG;
  qg_stream_plan::Win &W = p->wins[w];
  if (row_start < 0 || row_start + W.len > W.n_rows) return QG_E_RANGE;
  int dev = 0;
  QG_HIP(hipGetDevice(&dev));
  if (dev != p->device) return QG_E_ARG;
  for (const auto &c : W.copies)
    QG_HIP(hipGraphExecMemcpyNodeSetParams1D(p->exec, c.node, c.dst, W.host + (row_start + c.off) * W.rb,
                                             (size_t)c.bytes, hipMemcpyHostToDevice));
  W.row_start = row_start;
  return QG_OK;
}

int64_t qgemv_stream_plan_ring_bytes(const qg_stream_plan *p) {
  if (!p) return QG_E_NULL;
  return p->slot_bytes * (p->lookahead + 1);
}

int qgemv_stream_plan_run(qg_stream_plan *p, qg_stream_t stream) {
  if (!p) return QG_E_NULL;
  int dev = 0;
  QG_HIP(hipGetDevice(&dev));
  if (dev != p->device) return QG_E_ARG;
  QG_HIP(hipGraphLaunch(p->exec, (hipStream_t)stream));
  return QG_OK;
}

int qgemv_stream_plan_destroy(qg_stream_plan *p) { return plan_destroy(p); }

// ---- streaming without allocation -----------------------------------------------
//
// The ring of qgemv_stream_rows_noalloc: a file-scope device array, one per
// GPU the library runs on, held until the process ends.  In host code its
// name is only a stand-in; the device address comes from hipGetSymbolAddress,
// once per device, and only that address is ever passed on.
static __device__ __align__(256) uint8_t scratch[QG_NOALLOC_RING_BYTES];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {};

// The current device's copy of `scratch`.
int scratch_of_device(uint8_t **out) {
  int dev = 0;
  QG_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return QG_E_ARG;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    QG_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return hip_fail(hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = (uint8_t *)g_scratch_ptr[dev];
  return QG_OK;
}

}  // namespace

int qgemv_stream_rows_noalloc(const qg_matrix *w, int64_t row_start, int64_t row_end, int64_t block_rows,
                              const float *x, float *y, qg_stream_t stream) {
  int rc = check_matrix(w);
  if (rc) return rc;
  if ((rc = check_range(w->n_rows, row_start, row_end))) return rc;
  if (block_rows < 0) return QG_E_ARG;
  if (row_end == row_start) return QG_OK;
  if (!x || !y) return QG_E_NULL;
  const int64_t rb = row_bytes_of(w->fmt, w->k);
  const int64_t len = row_end - row_start;
  const int64_t B = block_rows > 0 ? std::min(block_rows, len) : len;
  constexpr int64_t kSlot = QG_NOALLOC_RING_BYTES / 2;
  if (B * rb > kSlot) return QG_E_CAPACITY;
  if ((rc = check_pinned(w->data))) return rc;
  uint8_t *ring = nullptr;
  if ((rc = scratch_of_device(&ring))) return rc;
  // Block j goes to slot j mod 2; its copy and its kernel are both on
  // `stream`, so the copy into a slot always follows the kernel that last
  // read it.
  int j = 0;
  for (int64_t r = row_start; r < row_end; r += B, ++j) {
    const int64_t n = std::min(B, row_end - r);
    uint8_t *dst = ring + (j & 1) * kSlot;
    QG_HIP(hipMemcpyAsync(dst, (const uint8_t *)w->data + r * rb, (size_t)(n * rb), hipMemcpyHostToDevice,
                          (hipStream_t)stream));
    qg_window blk = {dst, n, 0, n, x, y + (r - row_start)};
    if ((rc = launch_gemv(w->fmt, w->k, &blk, 1, 0, (hipStream_t)stream))) return rc;
  }
  return QG_OK;
}

// ---- host-mapped weights: the kernels read page-locked host memory in place ----

int qgemv_mapped_rows(const qg_matrix *w, int64_t row_start, int64_t row_end, const float *x, float *y,
                      int64_t block_rows, qg_stream_t stream) {
  int rc = check_matrix(w);
  if (rc) return rc;
  if ((rc = check_range(w->n_rows, row_start, row_end))) return rc;
  if (block_rows < 0) return QG_E_ARG;
  if (row_end == row_start) return QG_OK;
  if (!x || !y) return QG_E_NULL;
  const void *dev = nullptr;
  if ((rc = mapped_alias(w->data, &dev))) return rc;
  qg_window win = {dev, w->n_rows, row_start, row_end, x, y};
  return launch_gemv(w->fmt, w->k, &win, 1, block_rows, stream);
}

int qgemv_mapped_windows(int32_t fmt, int64_t k, const qg_window *win, int32_t n_win, int64_t block_rows,
                         qg_stream_t stream) {
  int rc = validate_windows(fmt, k, win, n_win, block_rows);
  if (rc) return rc;
  if (n_win == 0) return QG_OK;
  qg_window dw[kMaxWindows];
  for (int i = 0; i < n_win; ++i) {
    dw[i] = win[i];
    if (win[i].row_end == win[i].row_start) continue;
    if ((rc = mapped_alias(win[i].data, &dw[i].data))) return rc;
  }
  return launch_gemv(fmt, k, dw, n_win, block_rows, stream);
}

}  // extern "C"

// ---- chain --------------------------------------------------------------------

struct qg_chain {
  int device;
  int32_t fmt;
  int32_t n_steps;
  int grid;
  unsigned gen;  // barrier generation at the start of the next run
  void *mem;  // one device allocation: steps, windows, tile prefixes, barrier state
  unsigned *host_fail;  // page-locked, mapped: a failed barrier's mark, read without waiting
  unsigned spin_limit;
  ChainStepDev *steps;
  ChainWinDev *wins;
  int32_t *prefix;
  ChainSync *sync;
};

namespace {

typedef void (*ChainFn)(const ChainStepDev *, int, const ChainWinDev *, const int32_t *, ChainSync *, unsigned);

// The chain uses the team shape of qgemv_rows at the same k (one column per
// lane for Q8_0, two for Q4_0 and MXFP4), so its rows give the same bits.
ChainFn chain_fn(int32_t fmt) {
  switch (fmt) {
    case QG_Q8_0: return chain_kernel<QG_Q8_0, 1>;
    case QG_Q4_0: return chain_kernel<QG_Q4_0, 2>;
    default: return chain_kernel<QG_MXFP4, 2>;
  }
}

bool rms_op(int32_t op) { return op == QG_IN_RMS || op == QG_IN_GELU_RMS; }

// Writes the host-set fields of a chain's barrier state (after it was zeroed).
hipError_t sync_host_fields(ChainSync *sy, unsigned *host_fail, unsigned spin_limit) {
  void *dev = nullptr;
  hipError_t e = hipHostGetDevicePointer(&dev, host_fail, 0);
  if (e != hipSuccess) return e;
  if ((e = hipMemcpy(&sy->host_fail, &dev, sizeof(dev), hipMemcpyHostToDevice)) != hipSuccess) return e;
  return hipMemcpy(&sy->spin_limit, &spin_limit, sizeof(spin_limit), hipMemcpyHostToDevice);
}

int validate_chain(int32_t fmt, const qg_chain_step *steps, int32_t n_steps, const qg_chain_window *win,
                   int32_t n_win) {
  if (!steps || !win) return QG_E_NULL;
  if (block_bytes(fmt) < 0 || kquant(fmt)) return QG_E_FMT;  // no K-quant chain kernel
  if (n_steps < 1 || n_win < 1) return QG_E_ARG;
  for (int i = 0; i < n_win; ++i) {
    if (win[i].n_rows < 0) return QG_E_SHAPE;
    int rc = check_range(win[i].n_rows, win[i].row_start, win[i].row_end);
    if (rc) return rc;
    if ((uintptr_t)win[i].data & 15) return QG_E_ARG;
  }
  for (int s = 0; s < n_steps; ++s) {
    const qg_chain_step &S = steps[s];
    if (S.k <= 0 || S.k % 32 != 0 || S.k > QG_CHAIN_MAX_K) return QG_E_SHAPE;
    if (S.in_op < QG_IN_X || S.in_op > QG_IN_SILU_MUL) return QG_E_ARG;
    if (S.n_win < 1 || S.first_win < 0 || S.first_win > n_win - S.n_win) return QG_E_ARG;
    if (rms_op(S.in_op) && !(S.eps >= 0.0f)) return QG_E_ARG;
    const float *xs = nullptr;
    for (int w = S.first_win; w < S.first_win + S.n_win; ++w) {
      const qg_chain_window &W = win[w];
      if (W.row_end == W.row_start) continue;
      if (!W.data || !W.x || !W.y || (S.in_op == QG_IN_SILU_MUL && !W.x2)) return QG_E_NULL;
      if (rms_op(S.in_op)) {
        if (xs && W.x != xs) return QG_E_ARG;
        xs = W.x;
      }
    }
  }
  return QG_OK;
}

}  // namespace

extern "C" {

int qgemv_chain_create(int32_t fmt, const qg_chain_step *steps, int32_t n_steps, const qg_chain_window *win,
                       int32_t n_win, qg_chain **out) {
  if (!out) return QG_E_NULL;
  int rc = validate_chain(fmt, steps, n_steps, win, n_win);
  if (rc) return rc;
  int dev = 0, per_cu = 0;
  QG_HIP(hipGetDevice(&dev));
  const ChainFn fn = chain_fn(fmt);
  QG_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)fn, 64 * kChainWaves, 0));
  if (per_cu < 1) return hip_fail(hipErrorInvalidConfiguration, "chain workgroup does not fit a compute unit");
  const int grid = std::min(device_cus() * per_cu, kMaxChainGroups);
  const int bb = block_bytes(fmt);
  const int cc = first_c(fmt);  // block columns per lane (the chain takes k <= 24576: always this one)
  const int cap = tile_cap(fmt, cc) - (cc == 2 ? 1 : 0);  // ChainRows

  std::vector<ChainWinDev> hw(n_win);
  for (int i = 0; i < n_win; ++i)
    hw[i] = {(const uint8_t *)win[i].data, win[i].x, win[i].x2, win[i].y, nullptr, win[i].row_start, win[i].row_end};
  std::vector<ChainStepDev> hs(n_steps);
  std::vector<int32_t> hp;
  for (int s = 0; s < n_steps; ++s) {
    const qg_chain_step &S = steps[s];
    const int nb = (int)(S.k / 32);
    const int wt = (nb + 64 * cc - 1) / (64 * cc);
    const int tpw = kChainWaves / wt;
    const int64_t teams = (int64_t)grid * tpw;
    // Rows per tile: the fewest rows for the busiest team, with a small
    // charge per tile (the split never changes a row's result).
    int tr_best = 1;
    double best = 1e300;
    for (int tr = 1; tr <= cap; ++tr) {
      int64_t tiles = 0;
      for (int w = S.first_win; w < S.first_win + S.n_win; ++w)
        tiles += (win[w].row_end - win[w].row_start + tr - 1) / tr;
      const int64_t tpt = (tiles + teams - 1) / teams;
      const double cost = (double)tpt * tr + 0.5 * (double)tpt;
      if (cost < best - 1e-9) { best = cost; tr_best = tr; }
    }
    ChainStepDev d;
    memset(&d, 0, sizeof(d));
    d.pre0 = (int32_t)hp.size();
    int64_t tiles = 0;
    hp.push_back(0);
    for (int w = S.first_win; w < S.first_win + S.n_win; ++w) {
      tiles += (win[w].row_end - win[w].row_start + tr_best - 1) / tr_best;
      if (tiles > INT32_MAX / 2) return QG_E_SHAPE;
      hp.push_back((int32_t)tiles);
      if (rms_op(S.in_op) && !d.xs && win[w].row_end > win[w].row_start) d.xs = win[w].x;
    }
    d.w0 = hw[S.first_win];
    d.row_bytes = (int64_t)nb * bb;
    d.team_of_wave = 0;
    for (int v = 0; v < kChainWaves; ++v)
      d.team_of_wave |= (uint64_t)(v / wt < tpw ? v / wt : 15) << (4 * v);
    d.teams = (int32_t)teams;
    d.win0 = S.first_win;
    d.n_win = S.n_win;
    d.in_op = S.in_op;
    d.nb = nb;
    d.wt = wt;
    d.tpw = tpw;
    d.tile_rows = tr_best;
    d.n_tiles = (int32_t)tiles;
    d.iters_q = (int32_t)(tiles / teams);
    d.iters_r = (int32_t)(tiles % teams);
    d.eps = S.eps;
    hs[s] = d;
  }
  if (hp.size() > (size_t)INT32_MAX / 2) return QG_E_SHAPE;
  // A GELU + RMS step whose x is the whole output of one window of the step
  // before it gets gelu(x) from that window's stores (computed once per row
  // instead of once per team), into a buffer of the chain, and normalises it.
  std::vector<std::pair<int, int>> gelu_feed;  // (producing window, consuming step)
  for (int s = 1; s < n_steps; ++s) {
    if (hs[s].in_op != QG_IN_GELU_RMS || !hs[s].xs) continue;
    const qg_chain_step &P = steps[s - 1];
    for (int w = P.first_win; w < P.first_win + P.n_win; ++w)
      if (win[w].y == hs[s].xs && win[w].row_end - win[w].row_start == steps[s].k) {
        gelu_feed.push_back({w, s});
        break;
      }
  }

  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  const size_t o_steps = 0, o_wins = up(sizeof(ChainStepDev) * hs.size());
  const size_t o_pre = o_wins + up(sizeof(ChainWinDev) * hw.size());
  const size_t o_sync = o_pre + up(sizeof(int32_t) * hp.size());
  size_t o_act = o_sync + up(sizeof(ChainSync));
  std::vector<size_t> act_off(n_win, 0);  // offset of a window's gelu buffer, 0 = none
  for (auto &f : gelu_feed)
    if (!act_off[f.first]) {
      act_off[f.first] = o_act;
      o_act += up(sizeof(float) * steps[f.second].k);
    }
  const size_t total = o_act;
  uint8_t *mem = nullptr;
  QG_HIP(hipMalloc((void **)&mem, total));
  for (auto &f : gelu_feed) {
    hw[f.first].act = (float *)(mem + act_off[f.first]);
    hs[f.second].in_op = QG_IN_RMS;
    hs[f.second].xs = hw[f.first].act;
  }
  for (int s = 0; s < n_steps; ++s) hs[s].w0 = hw[steps[s].first_win];
  auto fail = [&](hipError_t e, const char *what) {
    (void)hipFree(mem);
    return hip_fail(e, what);
  };
  hipError_t e;
  if ((e = hipMemcpy(mem + o_steps, hs.data(), sizeof(ChainStepDev) * hs.size(), hipMemcpyHostToDevice)))
    return fail(e, "hipMemcpy(steps)");
  if ((e = hipMemcpy(mem + o_wins, hw.data(), sizeof(ChainWinDev) * hw.size(), hipMemcpyHostToDevice)))
    return fail(e, "hipMemcpy(windows)");
  if ((e = hipMemcpy(mem + o_pre, hp.data(), sizeof(int32_t) * hp.size(), hipMemcpyHostToDevice)))
    return fail(e, "hipMemcpy(prefix)");
  if ((e = hipMemset(mem + o_sync, 0, sizeof(ChainSync)))) return fail(e, "hipMemset(sync)");
  unsigned *hf = nullptr;
  if ((e = hipHostMalloc((void **)&hf, sizeof(unsigned), hipHostMallocMapped))) return fail(e, "hipHostMalloc(fail)");
  *hf = 0;
  if ((e = sync_host_fields((ChainSync *)(mem + o_sync), hf, kSpinLimit))) {
    (void)hipHostFree(hf);
    return fail(e, "hipMemcpy(sync fields)");
  }
  if ((e = hipDeviceSynchronize())) {
    (void)hipHostFree(hf);
    return fail(e, "hipDeviceSynchronize");
  }
  qg_chain *c = new qg_chain;
  c->host_fail = hf;
  c->spin_limit = kSpinLimit;
  c->device = dev;
  c->fmt = fmt;
  c->n_steps = n_steps;
  c->grid = grid;
  c->gen = 0;
  c->mem = mem;
  c->steps = (ChainStepDev *)(mem + o_steps);
  c->wins = (ChainWinDev *)(mem + o_wins);
  c->prefix = (int32_t *)(mem + o_pre);
  c->sync = (ChainSync *)(mem + o_sync);
  *out = c;
  return QG_OK;
}

int qgemv_chain_run(qg_chain *c, qg_stream_t stream) {
  if (!c) return QG_E_NULL;
  int dev = 0;
  QG_HIP(hipGetDevice(&dev));
  if (dev != c->device) return QG_E_ARG;
  // An earlier run's barrier gave up (as far as the host can see without
  // waiting): the barrier state is stale until qgemv_chain_check resets it.
  if (__atomic_load_n(c->host_fail, __ATOMIC_ACQUIRE)) return QG_E_BARRIER;
  // An ordinary launch of exactly as many workgroups as the device holds at
  // once, so on a device running nothing else every workgroup is resident.
  // (Should one not be, the barrier gives up after a bounded wait instead of
  // hanging, and qgemv_chain_check reports it.)
  hipLaunchKernelGGL(chain_fn(c->fmt), dim3((unsigned)c->grid), dim3(64 * kChainWaves), 0, stream, c->steps,
                     c->n_steps, c->wins, c->prefix, c->sync, c->gen);
  QG_HIP(hipGetLastError());
  c->gen += (unsigned)(c->n_steps - 1);
  return QG_OK;
}

int qgemv_chain_check(qg_chain *c) {
  if (!c) return QG_E_NULL;
  int dev = 0;
  QG_HIP(hipGetDevice(&dev));
  if (dev != c->device) return QG_E_ARG;
  QG_HIP(hipDeviceSynchronize());
  unsigned fail = 0;
  QG_HIP(hipMemcpy(&fail, &c->sync->fail, sizeof(fail), hipMemcpyDeviceToHost));
  if (!fail && !__atomic_load_n(c->host_fail, __ATOMIC_ACQUIRE)) return QG_OK;
  QG_HIP(hipMemset(c->sync, 0, sizeof(ChainSync)));
  QG_HIP(sync_host_fields(c->sync, c->host_fail, c->spin_limit));
  QG_HIP(hipDeviceSynchronize());
  __atomic_store_n(c->host_fail, 0u, __ATOMIC_RELEASE);
  c->gen = 0;
  return QG_E_BARRIER;
}

int qgemv_chain_set_spin_limit(qg_chain *c, uint32_t polls) {
  if (!c) return QG_E_NULL;
  if (polls < 1) return QG_E_ARG;
  int dev = 0;
  QG_HIP(hipGetDevice(&dev));
  if (dev != c->device) return QG_E_ARG;
  QG_HIP(hipDeviceSynchronize());
  QG_HIP(hipMemcpy(&c->sync->spin_limit, &polls, sizeof(polls), hipMemcpyHostToDevice));
  c->spin_limit = polls;
  return QG_OK;
}

int64_t qgemv_chain_grid(const qg_chain *c) { return c ? (int64_t)c->grid : (int64_t)QG_E_NULL; }

int qgemv_chain_destroy(qg_chain *c) {
  if (!c) return QG_OK;
  hipError_t e = hipDeviceSynchronize();
  hipError_t f = hipFree(c->mem);
  hipError_t h = hipHostFree(c->host_fail);
  delete c;
  if (f == hipSuccess) f = h;
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  if (f != hipSuccess) return hip_fail(f, "hipFree");
  return QG_OK;
}

}  // extern "C"
