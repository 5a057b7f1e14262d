// Weight-streaming factor GEMV for decode-sized M (M <= 64), bf16 MFMA.
//
// One factor of a decomposed projection (W ~ A B, DeInfer section 2.1,
// Eq. (1)) applied to a few token rows reads every weight once and does M
// multiply-adds per weight: 16 flop/byte at M = 16, above the float32 VALU
// ridge of MI355X and far below the bf16 MFMA ridge. So the product runs on
// MFMA with the token rows padded to 16, organised to keep HBM streaming:
//
//  * Weights are stored transposed, Wt[N, K], in 16 x 32 operand tiles
//    (1 KB each, MFMA lane order). A work item is 16 output columns -- one
//    row of tiles, a contiguous 16 * K * 2-byte block -- times a K split.
//    Output tiles this narrow give enough work items to fill the chip
//    without splitting K for most factor shapes.
//  * Per 32-wide reduction step a wave reads one weight tile (lane l: bytes
//    16 l .. 16 l + 15, one contiguous 1 KB per instruction): that is the
//    MFMA A operand, rows n0 + l % 16. The token rows are the B operand,
//    x[m][k0 + 8 (l / 16) ..]: from an operand-tiled activation (one
//    contiguous 1 KB again) or from a plain row-major one. The accumulator
//    lane (j, g) holds y[m = j][n0 + 4g + r], so the epilogue stores four
//    consecutive outputs per lane, row-major or straight into the operand
//    tiles of the next GEMV.
//  * RMSNorm stays out of the weight stream: its row scale commutes with
//    the product, W (g * x / rms(x)) = (W (g * x)) / rms(x). The residual
//    epilogue that produces x also stores g * x as bf16 operand tiles and
//    each tile's row sums of squares; the consuming GEMV streams g * x and
//    multiplies its rows by 1 / rms(x), formed from those sums, at the end.
//  * The waves of a workgroup take interleaved steps of the item's K range
//    and keep four steps (4 KB of weights) in flight each; their sums
//    meet in LDS and are added in wave order.
//  * With more than one K split, each workgroup writes its partial sums
//    through to the device-coherent level (relaxed agent-scope atomic
//    stores), waits for them to complete and bumps a per-tile counter; the
//    last workgroup to arrive reads the partials back with device-coherent
//    loads, sums them in split order (deterministic) and runs the epilogue.
//    One atomic per workgroup, and no L2 writeback or invalidate (an
//    agent-scope fence would cost both on every workgroup).
//  * Epilogues: bf16 / f32 store, scatter into the latent KV cache (operand
//    tiles, key cache position-major, value cache rank-major), residual
//    add, and SwiGLU for paired (gate, up) launches whose two halves share
//    the output columns.
//  * Fused chains (the factor pair of Eq. (1) and the consecutive pairs of a
//    decode step in one launch): a persistent grid takes work items from an
//    atomic ticket counter in stage order -- every item of stage s before
//    any item of stage s + 1. An item first issues its first weight steps
//    (weights never depend on an earlier stage), then waits until every item
//    of the previous stage has counted itself done, then loads its
//    activations and finishes; so the next stage's weight stream starts
//    while the previous stage's last items and merges drain, with no launch
//    in between, and the rank-k intermediate passes from one stage to the
//    next through the device-coherent level (it is a few tens of KB at
//    decode sizes) without a kernel boundary. A waiting item only ever waits
//    for items with smaller tickets, which were handed to workgroups already
//    running and which never wait for a larger ticket, so every wait ends
//    whatever the number of resident workgroups; the wait is bounded anyway
//    (a time-out poisons the item's outputs with NaN instead of hanging).
//    Data that a later stage of the same launch reads is written with
//    agent-scope atomic stores (written through to the device-coherent
//    level, like the split-K partials) and published with the same store /
//    wait / counter sequence. It is read with plain, cacheable loads: each
//    such buffer is written by exactly one stage of a launch and no
//    workgroup touches it before observing that stage complete, so no cache
//    of any XCD can hold an older copy from this launch (kernel boundaries
//    invalidate copies from earlier ones), and its reads -- as many bytes as
//    the weights for one-tile items -- stay in L2 instead of each going to
//    the memory side.
#include <stdlib.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace dl {

namespace {
constexpr int kRows = 16;   // output columns per tile (rows of Wt)

// Device-coherent 8-byte accesses for the split-K partial sums: relaxed
// agent-scope atomics compile to plain loads/stores with the system-coherent
// cache policy (written through to, and read from, the level shared by all
// XCDs), without the L2 writeback/invalidate of an agent-scope fence.
__device__ __forceinline__ void store_coherent(float *p, float a, float b) {
  const uint64_t v = static_cast<uint64_t>(__float_as_uint(a)) |
                     (static_cast<uint64_t>(__float_as_uint(b)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void load_coherent(const float *p, float &a, float &b) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  a = __uint_as_float(static_cast<uint32_t>(v));
  b = __uint_as_float(static_cast<uint32_t>(v >> 32));
}
// Wait until every memory access this wave issued has completed; the
// "memory" clobber keeps the compiler from moving accesses across it.
__device__ __forceinline__ void wait_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Accesses of data that another workgroup of the same launch produces or
// consumes (COH = 1: agent-scope relaxed atomics, compiled to plain accesses
// with the device-coherence bit; COH = 0: plain accesses).
template <int COH>
__device__ __forceinline__ u32x4 ld16c(const uint16_t *p) {
  if constexpr (COH) {
    const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
    const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32), static_cast<uint32_t>(b),
                 static_cast<uint32_t>(b >> 32)};
  } else {
    return *reinterpret_cast<const u32x4 *>(p);
  }
}
template <int COH>
__device__ __forceinline__ u32x2 ld8c(const uint16_t *p) {
  if constexpr (COH) {
    const uint64_t a = __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return u32x2{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32)};
  } else {
    return *reinterpret_cast<const u32x2 *>(p);
  }
}
template <int COH>
__device__ __forceinline__ f32x4 ld16fc(const float *p) {
  const u32x4 v = ld16c<COH>(reinterpret_cast<const uint16_t *>(p));
  return f32x4{__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
}
template <int COH>
__device__ __forceinline__ float ldfc(const float *p) {
  if constexpr (COH)
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}
template <int COH>
__device__ __forceinline__ void st8c(uint16_t *p, u32x2 v) {
  if constexpr (COH)
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), static_cast<uint64_t>(v.x) | (static_cast<uint64_t>(v.y) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *reinterpret_cast<u32x2 *>(p) = v;
}
template <int COH>
__device__ __forceinline__ void st16fc(float *p, f32x4 v) {
  if constexpr (COH) {
    store_coherent(p, v[0], v[1]);
    store_coherent(p + 2, v[2], v[3]);
  } else {
    *reinterpret_cast<f32x4 *>(p) = v;
  }
}
template <int COH>
__device__ __forceinline__ void stfc(float *p, float v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// Interleave the 8 XCDs: dispatch hands workgroup b to XCD b % 8; give each
// XCD a contiguous range of items, i.e. neighbouring weight tiles.
__device__ __forceinline__ int xcd_item(int b, int grid) {
  const int per = grid >> 3;  // grid is a multiple of 8
  return (b & 7) * per + (b >> 3);
}

// Activation modes: row-major bf16, operand-tiled bf16.
enum XMode : int { XM_BF16 = 0, XM_TILED = 1 };

// Activation operands are loaded into the prefetch ring with the weights
// (so waiting for a step never waits for later prefetches). Row-major mode
// reads row `row` at column k; tiled mode reads fragment (row block mb,
// column step k / 32) of an [Mpad, cols] operand-tiled matrix.
template <int XM, int COH>
__device__ __forceinline__ u32x4 load_x(const uint16_t *X, int ldx, int row, int mb, int k, int lane) {
  if constexpr (XM == XM_TILED)
    return ld16c<COH>(X + frag_off(mb, k >> 5, ldx, lane));
  else
    return ld16c<COH>(X + static_cast<size_t>(row) * ldx + k);
}

// LDS of one work item: per-wave sums [kWaves][RED], their total [RED],
// the RMSNorm row scales and a broadcast flag.
struct GvLds {
  float *wsum;
  float *red;
  float *rscale;
  int *flag;
};
// Chain hooks of one work item (all null outside a chain): wait until the
// kChainQueues counters at wait_done (kSyncStride apart) sum to wait_need
// after the first weight loads; count the item in *done when finished;
// *err records a wait time-out.
struct GvSync {
  const int *wait_done;
  int wait_need;
  int *done;
  int *err;
};
// Sum of the kChainQueues done counters at d, read by the lanes of one wave
// (one coherent load per lane) and added across the wave.
__device__ __forceinline__ int chain_done_sum(const int *d, int lane) {
  static_assert(kChainQueues <= 64, "one counter per lane");
  int v = lane < kChainQueues
              ? __hip_atomic_load(d + kSyncStride * lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
              : 0;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
// Polls (each one to two microseconds) before a chain wait gives up: far
// beyond any stage's duration; reached only if the launch's ticket and
// counters were not zero at the start.
constexpr int kSpinLimit = 1 << 21;

// One work item of a GEMV launch (or of one chain stage).
template <int MB, int XM, int PAIRED, int RS, int R, int kWaves, int COH>
__device__ __forceinline__ void gemv_item(const GvArgs &a, const int item, const GvLds &L,
                                          const GvSync &sy) {
  constexpr bool XT = XM == XM_TILED;
  constexpr int kThreads = kWaves * 64;
  constexpr int HALVES = PAIRED ? 2 : 1;
  constexpr int NACC = HALVES * R * MB;      // f32x4 accumulators per lane
  constexpr int RED = NACC * 4 * 64;         // floats of one wave's sums
  constexpr int PART = RED;                  // floats of one split's partial sums
  float *const red = L.red;
  float *const rscale = L.rscale;
  int &last_flag = *L.flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, grp = lane >> 4;
  // work item = (K split, group of R consecutive 16-row tiles of one
  // segment); `tile` numbers the groups
  const int split = item / a.ntiles;
  const int tile = item - split * a.ntiles;
  int si = 0;
  if (a.nseg > 1 && tile >= a.seg[1].tile_begin) si = 1;
  if (a.nseg > 2 && tile >= a.seg[2].tile_begin) si = 2;
  const GvSeg sg = a.seg[si];
  const int n0 = (tile - sg.tile_begin) * R * kRows;
  const int seg_tiles = (sg.N + kRows - 1) / kRows;

  const int ksteps = (a.K + a.K2) >> 5;
  const int s_begin = split * a.split_steps;
  const int s_end = min(s_begin + a.split_steps, ksteps);

  f32x4 acc[HALVES][R][MB];
#pragma unroll
  for (int h = 0; h < HALVES; ++h)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[h][r][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // 32-wide steps (weights + activations) in flight per wave
  // 32-wide steps (weights + activations) in flight per wave (a ring twice
  // or four times as deep measured the same)
  constexpr int kDepth = MB <= 2 ? 4 : 2;
  struct Stage {
    u32x4 w[R];    // one weight tile per row tile, sharing ...
    u32x4 x[MB];   // ... the activation fragment
  };
  // every load below is unconditional (rows clamped, pointers selected), so
  // the compiler's wait counts stay exact across the prefetch ring
  // this item's rows of weight tiles (16 rows x K each), lane offset
  // included; tiles past the segment's last repeat it and are not stored
  const uint16_t *w1[R];
  const uint16_t *w2[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int tr = min((n0 >> 4) + r, seg_tiles - 1);
    w1[r] = sg.W + frag_off(tr, 0, a.K, lane);
    w2[r] = PAIRED ? sg.W2 + frag_off(tr, 0, a.K2, lane) : w1[r];
  }
  auto load_w = [&](Stage &sb, int st) {
    int k = st * 32;
    const bool second = PAIRED && k >= a.K;
    k -= second ? a.K : 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
      sb.w[r] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4 *>((second ? w2[r] : w1[r]) + static_cast<size_t>(k >> 5) * 512));
  };
  auto load_xs = [&](Stage &sb, int st) {
    int k = st * 32;
    const bool second = PAIRED && k >= a.K;
    const uint16_t *X = static_cast<const uint16_t *>(second ? sg.X2 : sg.X);
    const int ldx = second ? sg.ldx2 : sg.ldx;
    k -= second ? a.K : 0;
    if (!XT) k += 8 * grp;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      sb.x[mb] = load_x<XM, 0>(X, ldx, min(mb * 16 + j, a.M - 1), mb, k, lane);
  };
  auto load_stage = [&](Stage &sb, int st) {
    load_w(sb, st);
    load_xs(sb, st);
  };
  // `valid` is false for the padding steps at the end of the ring: their
  // activation operand is zeroed (a select, not a branch), so the loop body
  // stays branch-free and the compiler's wait counts stay exact. Padding
  // rows (>= M) of the activation are zeroed the same way.
  auto compute = [&](const Stage &sb, int st, bool valid) {
    const int h = PAIRED && st * 32 >= a.K ? HALVES - 1 : 0;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      u32x4 x = sb.x[mb];
      if (!valid || mb * 16 + j >= a.M) x = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (h == 0)
          acc[0][r][mb] = mfma_bf16(sb.w[r], x, acc[0][r][mb]);
        else
          acc[HALVES - 1][r][mb] = mfma_bf16(sb.w[r], x, acc[HALVES - 1][r][mb]);
      }
    }
  };

  // this wave's steps: s_begin + wave + kWaves * i, i < nst; kDepth in flight.
  // Ring slots past the last step reload the last step (cache hits) and
  // compute with a zero operand, so the loop body has no branches.
  const int st0 = s_begin + wave;
  const int nst = st0 < s_end ? (s_end - st0 + kWaves - 1) / kWaves : 0;
  const int st_last = st0 + kWaves * (nst - 1);
  // RMSNorm row scale (RS): this wave's rows (wave, wave + kWaves, ...) of
  // the producer's per-tile sums of squares, columns lane + 64 c, requested
  // before the weight stream with a fixed count (rows and columns clamped,
  // out-of-range terms dropped by a select), so they arrive while the first
  // weights do; summed in a fixed order after the main loop.
  constexpr int RSR = RS ? (MB * 16 + kWaves - 1) / kWaves : 1;
  constexpr int RSC = MB <= 2 ? 8 : 4;   // columns per lane read up front
  float rs_acc[RSR][RSC];
  // the ring's first weights, then (in a chain) the wait for the producing
  // stage, then everything that stage wrote: row sums and activations
  Stage ring[kDepth];
  if (nst > 0) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      load_w(ring[d], min(st0 + kWaves * d, st_last));
      __builtin_amdgcn_sched_barrier(0);   // stages issue in ring order
    }
  }
  bool poison = false;
  if (sy.wait_done) {
    if (wave == 0) {   // the whole wave polls (the loop condition is wave-uniform)
      int spins = 0;
      while (chain_done_sum(sy.wait_done, lane) < sy.wait_need) {
        __builtin_amdgcn_s_sleep(8);
        if (++spins == kSpinLimit) {
          if (lane == 0) __hip_atomic_store(sy.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
      if (lane == 0) last_flag = spins == kSpinLimit;
    }
    __syncthreads();
    poison = last_flag;
    __syncthreads();   // last_flag is reused by the split merge
  }
  if constexpr (RS) {
#pragma unroll
    for (int i = 0; i < RSR; ++i)
#pragma unroll
      for (int c = 0; c < RSC; ++c)
        rs_acc[i][c] = ldfc<0>(a.rs_part + static_cast<size_t>(min(wave + kWaves * i, a.M - 1)) * a.rs_cols +
                                 min(lane + 64 * c, a.rs_cols - 1));
  }
  if (nst > 0) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      load_xs(ring[d], min(st0 + kWaves * d, st_last));
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int i = 0; i < nst; i += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        compute(ring[d], min(st0 + kWaves * (i + d), st_last), i + d < nst);
        // keep the ring order: the scheduler must not sink this reload
        // next to its use or hoist it above the compute of an older stage
        __builtin_amdgcn_sched_barrier(0);
        load_stage(ring[d], min(st0 + kWaves * (i + d + kDepth), st_last));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if constexpr (RS) {
#pragma unroll
    for (int i = 0; i < RSR; ++i) {
      const int m = wave + kWaves * i;
      float sq = 0.f;
#pragma unroll
      for (int c = 0; c < RSC; ++c) sq += lane + 64 * c < a.rs_cols ? rs_acc[i][c] : 0.f;
      for (int c = lane + 64 * RSC; c < a.rs_cols; c += 64)   // wider rows
        sq += ldfc<0>(a.rs_part + static_cast<size_t>(min(m, a.M - 1)) * a.rs_cols + c);
      sq = wave_sum(sq);
      if (lane == 0 && m < a.M) rscale[m] = rsqrtf(sq / static_cast<float>(a.K) + a.eps);
    }
  }
  // per-wave sums -> LDS, then a fixed-order sum over the waves:
  // red[((((h * R + r) * MB + mb) * 4 + e) * 64 + lane]
#pragma unroll
  for (int h = 0; h < HALVES; ++h)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          L.wsum[wave * RED + (((h * R + r) * MB + mb) * 4 + e) * 64 + lane] = acc[h][r][mb][e];
  __syncthreads();
  for (int idx = tid; idx < RED; idx += kThreads) {
    float v = L.wsum[idx];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += L.wsum[w * RED + idx];
    red[idx] = v;
  }
  __syncthreads();

  if (a.ksplit > 1) {
    float *mine = a.part + (static_cast<size_t>(tile) * a.ksplit + split) * PART;
    for (int i = tid; i < PART / 2; i += kThreads) store_coherent(mine + 2 * i, red[2 * i], red[2 * i + 1]);
    wait_memory();
    __syncthreads();
    if (tid == 0)
      last_flag = __hip_atomic_fetch_add(&a.counters[tile], 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == a.ksplit - 1;
    __syncthreads();
    if (!last_flag) {
      // this item is done: its partials are published
      if (sy.done && tid == 0) __hip_atomic_fetch_add(sy.done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    // eight partials in flight per thread (indices clamped, loads
    // unconditional), summed in split order
    const float *base = a.part + static_cast<size_t>(tile) * a.ksplit * PART;
    const int ks = a.ksplit;
    for (int i = tid; i < PART / 2; i += kThreads) {
      float v0 = 0.f, v1 = 0.f;
      for (int sp0 = 0; sp0 < ks; sp0 += 8) {
        float x0[8], x1[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          load_coherent(base + static_cast<size_t>(min(sp0 + u, ks - 1)) * PART + 2 * i, x0[u], x1[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (sp0 + u < ks) {
            v0 += x0[u];
            v1 += x1[u];
          }
        }
      }
      red[2 * i] = v0;
      red[2 * i + 1] = v1;
    }
    if (tid == 0) __hip_atomic_store(&a.counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }

  // epilogue: unit u = (m * R + rt) * 4 + q writes y[m][n0 + 16 rt + 4q ..
  // + 3] (four consecutive units share a row and a tile: lanes 4k .. 4k + 3);
  // the accumulator lane of (column 16 rt + 4q + e, row m) is 16q + m % 16,
  // register e
  for (int u = tid; u < a.M * R * 4; u += kThreads) {
  const int m = u / (R * 4), rt = (u >> 2) % R, q = u & 3;
  const int n = n0 + 16 * rt + 4 * q;
  if (n >= sg.N) continue;
  const int mb = m >> 4, ln = 16 * q + (m & 15);
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = red[(((0 * R + rt) * MB + mb) * 4 + r) * 64 + ln];
  if constexpr (RS) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] *= rscale[m];
  }
  if (poison) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = __builtin_nanf("");
  }
  const size_t oi = static_cast<size_t>(m) * sg.ldo + n;
  switch (sg.omode) {
    case GV_OUT_BF16:
      st8c<COH>(static_cast<uint16_t *>(sg.out) + oi, u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])});
      break;
    case GV_OUT_F32:
      st16fc<COH>(static_cast<float *>(sg.out) + oi, f32x4{v[0], v[1], v[2], v[3]});
      break;
    case GV_OUT_TILED:
      st8c<COH>(static_cast<uint16_t *>(sg.out) + tile_off(m, n, sg.N),
                u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])});
      break;
    case GV_OUT_RELU_TILED:
      st8c<COH>(static_cast<uint16_t *>(sg.out) + tile_off(m, n, sg.N),
                u32x2{pack2(fmaxf(v[0], 0.f), fmaxf(v[1], 0.f)), pack2(fmaxf(v[2], 0.f), fmaxf(v[3], 0.f))});
      break;
    case GV_OUT_CACHE: {   // key cache page: [kPage, N] operand tiles
      const int b = m / a.T, pos = a.past[b] + m - b * a.T;
      const int pg = cache_page(a.block_table, a.page_stride, b, pos / kPage);
      *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(sg.out) + key_off(pg, pos, n, sg.N)) =
          u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
      break;
    }
    case GV_OUT_CACHE_T: {   // value cache page: [N, kPage] operand tiles
      const int b = m / a.T, pos = a.past[b] + m - b * a.T;
      const int pg = cache_page(a.block_table, a.page_stride, b, pos / kPage);
      uint16_t *pool = static_cast<uint16_t *>(sg.out);
#pragma unroll
      for (int r = 0; r < 4; ++r) pool[val_off(pg, pos, n + r, sg.N)] = f2bf(v[r]);
      break;
    }
    case GV_OUT_RES_F32: {
      const size_t ri = static_cast<size_t>(m) * sg.ldr + n;
      if (sg.res_f32) {
        const f32x4 rr = ld16fc<0>(static_cast<const float *>(sg.R) + ri);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += rr[r];
      } else {
        const u32x2 rr = ld8c<0>(static_cast<const uint16_t *>(sg.R) + ri);
        v[0] += bflo(rr.x);
        v[1] += bfhi(rr.x);
        v[2] += bflo(rr.y);
        v[3] += bfhi(rr.y);
      }
      const f32x4 o = f32x4{v[0], v[1], v[2], v[3]};
      st16fc<COH>(static_cast<float *>(sg.out) + oi, o);
      if (sg.out2) *reinterpret_cast<f32x4 *>(sg.out2 + oi) = o;   // read after the launch only
      if (sg.out_nt) {
        // next RMSNorm's input: g * o as bf16 operand tiles, and the sum of
        // squares of o over this tile's 16 columns of row m (the four
        // threads of the row are lanes 4m .. 4m + 3; N % 16 == 0)
        float gn[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          gn[r] = sg.gamma ? (sg.gamma_f32 ? static_cast<const float *>(sg.gamma)[n + r]
                                           : bf2f(static_cast<const uint16_t *>(sg.gamma)[n + r]))
                           : 1.f;
        st8c<COH>(sg.out_nt + tile_off(m, n, sg.N),
                  u32x2{pack2(o[0] * gn[0], o[1] * gn[1]), pack2(o[2] * gn[2], o[3] * gn[3])});
        float sq = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
        sq += __shfl_xor(sq, 1, 64);
        sq += __shfl_xor(sq, 2, 64);
        if (q == 0) stfc<COH>(sg.ssq_out + static_cast<size_t>(m) * (sg.N >> 4) + (n >> 4), sq);
      }
      break;
    }
    case GV_OUT_RES_BF16: {
      const f32x4 rr = ld16fc<0>(static_cast<const float *>(sg.R) + static_cast<size_t>(m) * sg.ldr + n);
      st8c<COH>(static_cast<uint16_t *>(sg.out) + oi,
                u32x2{pack2(v[0] + rr[0], v[1] + rr[1]), pack2(v[2] + rr[2], v[3] + rr[3])});
      break;
    }
    default: {  // GV_OUT_SWIGLU, GV_OUT_SWIGLU_TILED
      float g2[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) g2[r] = silu(v[r]) * red[(((1 * R + rt) * MB + mb) * 4 + r) * 64 + ln];
      const size_t o = sg.omode == GV_OUT_SWIGLU_TILED ? tile_off(m, n, sg.N) : oi;
      st8c<COH>(static_cast<uint16_t *>(sg.out) + o, u32x2{pack2(g2[0], g2[1]), pack2(g2[2], g2[3])});
      break;
    }
  }
  }
  if (sy.done) {
    // every output of this item is stored (and device-visible: its stores
    // are coherent ones and have completed) before the item counts as done
    wait_memory();
    __syncthreads();
    if (tid == 0) __hip_atomic_fetch_add(sy.done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int MB, int XM, int PAIRED, int RS, int R, int kWaves>
__global__ __launch_bounds__(kWaves * 64) void gemv_kernel(GvArgs a) {
  constexpr int RED = (PAIRED ? 2 : 1) * R * MB * 4 * 64;
  __shared__ __attribute__((aligned(16))) float wsum[kWaves * RED];
  __shared__ __attribute__((aligned(16))) float red[RED];
  __shared__ float rscale[MB * 16];
  __shared__ int flag;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  if (item >= a.ntiles * a.ksplit) return;
  gemv_item<MB, XM, PAIRED, RS, R, kWaves, 0>(a, item, GvLds{wsum, red, rscale, &flag},
                                              GvSync{nullptr, 0, nullptr, nullptr});
}

// Persistent chain: stage s's items i with i % kChainQueues == q form queue
// q's share of the stage; workgroup b takes tickets of queue b %
// kChainQueues, whose items run stage by stage. An item of stage s > 0
// waits for all of stage s - 1 (and so, transitively, for every earlier
// stage). Each wait is for items that precede it in every queue: in its own
// queue they were handed out before it to running workgroups, and in any
// other queue they are reached before that queue's stage-s items, by
// workgroups that only ever wait for still earlier stages, so by induction
// on the stage every wait ends. Dynamic LDS: per-wave sums and their total
// for the largest stage, (4 + 1) * red_max floats.
template <int MB>
__global__ __launch_bounds__(256) void gemv_chain_kernel(GvChain c) {
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  __shared__ float rscale[MB * 16];
  __shared__ int flag, ticket;
  int red_max = 0;
  for (int s = 0; s < c.nst; ++s)
    red_max = max(red_max, (c.st[s].K2 > 0 ? 2 : 1) * c.st[s].rtiles * MB * 4 * 64);
  const GvLds L{dyn, dyn + 4 * red_max, rscale, &flag};
  const int queue = blockIdx.x % kChainQueues;
  for (;;) {
    if (threadIdx.x == 0)
      ticket = __hip_atomic_fetch_add(c.sync + kSyncStride * queue, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int t = ticket;
    __syncthreads();   // the ticket is read before the next one is taken
    // queue ticket -> (stage, item): the queue's share of stage s is items
    // queue, queue + kChainQueues, ...
    int s = 0;
    for (; s < c.nst; ++s) {
      const int n = c.st[s].ntiles * c.st[s].ksplit;
      const int share = n > queue ? (n - queue + kChainQueues - 1) / kChainQueues : 0;
      if (t < share) break;
      t -= share;
    }
    if (s == c.nst) return;   // every item of this queue is taken
    s = __builtin_amdgcn_readfirstlane(s);
    t = queue + kChainQueues * t;
    const GvArgs &a = c.st[s];
    const GvSync sy{s > 0 ? c.sync + kSyncStride * (kChainQueues * s) : nullptr,
                    s > 0 ? c.st[s - 1].ntiles * c.st[s - 1].ksplit : 0,
                    c.sync + kSyncStride * (kChainQueues * (1 + s) + queue),
                    c.sync + kSyncStride * (kChainQueues * (1 + kMaxChain))};
    const int R = a.rtiles;
    if (!a.x_tiled) {   // first stage only: row-major activations from outside the chain
      if (R == 1) gemv_item<MB, XM_BF16, 0, 0, 1, 4, 1>(a, t, L, sy);
      else if (R == 2) gemv_item<MB, XM_BF16, 0, 0, 2, 4, 1>(a, t, L, sy);
      else if constexpr (MB <= 2) gemv_item<MB, XM_BF16, 0, 0, 4, 4, 1>(a, t, L, sy);
    } else if (a.K2 > 0) {
      if (R == 1) gemv_item<MB, XM_TILED, 1, 0, 1, 4, 1>(a, t, L, sy);
      else if (R == 2) gemv_item<MB, XM_TILED, 1, 0, 2, 4, 1>(a, t, L, sy);
      else if constexpr (MB <= 2) gemv_item<MB, XM_TILED, 1, 0, 4, 4, 1>(a, t, L, sy);
    } else if (a.rs_part) {
      if (R == 1) gemv_item<MB, XM_TILED, 0, 1, 1, 4, 1>(a, t, L, sy);
      else if (R == 2) gemv_item<MB, XM_TILED, 0, 1, 2, 4, 1>(a, t, L, sy);
      else if constexpr (MB <= 2) gemv_item<MB, XM_TILED, 0, 1, 4, 4, 1>(a, t, L, sy);
    } else {
      if (R == 1) gemv_item<MB, XM_TILED, 0, 0, 1, 4, 1>(a, t, L, sy);
      else if (R == 2) gemv_item<MB, XM_TILED, 0, 0, 2, 4, 1>(a, t, L, sy);
      else if constexpr (MB <= 2) gemv_item<MB, XM_TILED, 0, 0, 4, 4, 1>(a, t, L, sy);
    }
    __syncthreads();   // LDS is reused by the next item
  }
}

template <int MB>
hipError_t launch_chain_mb(const GvChain &c, int grid, hipStream_t s) {
  int red_max = 0;
  for (int i = 0; i < c.nst; ++i)
    red_max = std::max(red_max, (c.st[i].K2 > 0 ? 2 : 1) * c.st[i].rtiles * MB * 4 * 64);
  const int dyn = 5 * red_max * static_cast<int>(sizeof(float));
  const void *fn = reinterpret_cast<const void *>(&gemv_chain_kernel<MB>);
  static int dyn_set = 0;   // largest dynamic LDS allowed so far for this instantiation
  if (dyn > dyn_set && dyn > 65536) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
    if (e != hipSuccess) return e;
    dyn_set = dyn;
  }
  gemv_chain_kernel<MB><<<grid, 256, dyn, s>>>(c);
  return hipGetLastError();
}

template <int MB, int XM, int PAIRED, int RS>
hipError_t launch_t(const GvArgs &a, int grid, hipStream_t s) {
  if (MB <= 2 && a.rtiles == 4)   // (four tiles of four row blocks would overflow LDS)
    gemv_kernel<MB, XM, PAIRED, RS, MB <= 2 ? 4 : 2, 4><<<grid, 4 * 64, 0, s>>>(a);
  else if (a.rtiles == 2)
    gemv_kernel<MB, XM, PAIRED, RS, 2, 4><<<grid, 4 * 64, 0, s>>>(a);
  else if (a.waves == 4)
    gemv_kernel<MB, XM, PAIRED, RS, 1, 4><<<grid, 4 * 64, 0, s>>>(a);
  else
    gemv_kernel<MB, XM, PAIRED, RS, 1, 8><<<grid, 8 * 64, 0, s>>>(a);
  return hipGetLastError();
}

template <int MB>
hipError_t launch_mb(const GvArgs &a, int grid, hipStream_t s) {
  if (a.K2 > 0)
    return a.x_tiled ? launch_t<MB, XM_TILED, 1, 0>(a, grid, s) : launch_t<MB, XM_BF16, 1, 0>(a, grid, s);
  if (a.rs_part)
    return a.x_tiled ? launch_t<MB, XM_TILED, 0, 1>(a, grid, s) : launch_t<MB, XM_BF16, 0, 1>(a, grid, s);
  return a.x_tiled ? launch_t<MB, XM_TILED, 0, 0>(a, grid, s) : launch_t<MB, XM_BF16, 0, 0>(a, grid, s);
}

int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}
}  // namespace

// Compute units of the current device (256 on MI355X).
int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    cus = hipGetDevice(&dev) == hipSuccess &&
                  hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0
              ? v
              : 256;
  }
  return cus;
}

size_t gemv_plan(GvArgs &a) {
  int tiles = 0;
  for (int i = 0; i < a.nseg; ++i) tiles += (a.seg[i].N + kRows - 1) / kRows;
  a.waves = env_int("DL_GEMV_WAVES", 4) == 8 ? 8 : 4;
  const int ksteps = (a.K + a.K2) / 32;
  const int cus = std::max(1, env_int("DL_GEMV_CUS", device_cus()));
  const int min_steps = std::max(1, env_int("DL_GEMV_MIN_STEPS", 4));
  // K split: the largest that keeps the grid within one workgroup per
  // compute unit (ks = CUs / items), never more. Measured per launch on
  // 256 CUs: grids a little over the CU count (264, 304 or 352 workgroups)
  // are as slow as a whole extra round on the CUs that take two items, and
  // each split adds a merge; a one-round grid with some CUs idle is faster
  // (e.g. 136 unsplit tiles of a 4096-wide K, or 116 tiles split in two).
  const int ks_max = std::max(1, std::min(64, ksteps / (min_steps * a.waves)));
  auto splits = [&](int items) { return std::max(1, std::min(ks_max, cus / std::max(1, items))); };
  // Two or four row tiles per item share each activation fragment (halving
  // or quartering the activation reads, which otherwise cost twice the
  // weight bytes per step at 32 rows). Four tiles only up to 32 token rows
  // (LDS).
  int R = 1;
  if (a.waves == 4) {
    const int forced = env_int("DL_GEMV_R", 0);
    // the widest item (four tiles up to 32 token rows, else two) whose K
    // stream, after the one-round split, still has at least 64 steps:
    // long-K factors gain (54 -> 37 us for the 70B A_down at 32 rows), while
    // short-K ones lose to the shorter streams and larger merges
    R = forced == 1 || forced == 2 || forced == 4 ? forced : 1;
    for (int r = 4; r >= 2 && forced == 0; r /= 2) {
      if ((r == 4 && a.M > 32) || tiles < r) continue;
      const int ks_r = splits((tiles + r - 1) / r);
      if ((ksteps + ks_r - 1) / ks_r >= 64) {
        R = r;
        break;
      }
    }
    if (R == 4 && a.M > 32) R = 2;
  }
  a.rtiles = R;
  int items = 0;
  for (int i = 0; i < a.nseg; ++i) {
    a.seg[i].tile_begin = items;
    items += ((a.seg[i].N + kRows - 1) / kRows + R - 1) / R;
  }
  a.ntiles = items;
  const int ks_forced = env_int("DL_GEMV_KS", 0);
  const int ks = ks_forced > 0 ? std::min(ks_forced, ks_max) : splits(items);
  const int sps = (ksteps + ks - 1) / ks;
  a.split_steps = sps;
  a.ksplit = (ksteps + sps - 1) / sps;
  const int MB = (a.M + 15) / 16;
  const int halves = a.K2 > 0 ? 2 : 1;
  const size_t part = static_cast<size_t>(halves) * R * MB * 4 * 64;
  return a.ksplit > 1 ? part * a.ntiles * a.ksplit : 0;
}

// the chain's stage table travels as the kernel argument (4 KB at most)
static_assert(sizeof(GvChain) <= 4096, "chain stage table exceeds the kernel-argument limit");

hipError_t launch_gemv_chain(const GvChain &c, hipStream_t s) {
  TraceGuard trace_guard(K_GEMV_CHAIN, s);
  if (c.nst < 1 || c.nst > kMaxChain) return hipErrorInvalidValue;
  int total = 0;
  for (int i = 0; i < c.nst; ++i) {
    const GvArgs &a = c.st[i];
    // the chain runs four waves per item, stages of one M, tiled inputs after
    // the first, and at most four row tiles per item for two row blocks
    if (a.waves != 4 || a.M != c.st[0].M || (i > 0 && !a.x_tiled) || (a.rtiles == 4 && a.M > 32))
      return hipErrorInvalidValue;
    total += a.ntiles * a.ksplit;
  }
  // one persistent workgroup per compute unit: measured fastest (a second,
  // waiting workgroup per unit slowed the running stage down)
  const int per_cu = std::max(1, std::min(8, env_int("DL_CHAIN_WGS_PER_CU", 1)));
  // at least one workgroup per queue
  const int grid = std::max(kChainQueues, std::min(total, per_cu * device_cus()));
  switch ((c.st[0].M + 15) / 16) {
    case 1: return launch_chain_mb<1>(c, grid, s);
    case 2: return launch_chain_mb<2>(c, grid, s);
    case 3: return launch_chain_mb<3>(c, grid, s);
    default: return launch_chain_mb<4>(c, grid, s);
  }
}

hipError_t launch_gemv(const GvArgs &a, hipStream_t s) {
  TraceGuard trace_guard(K_GEMV_BF16, s);
  const int items = a.ntiles * a.ksplit;
  const int grid = (items + 7) / 8 * 8;
  const int mb = (a.M + 15) / 16;
  switch (mb) {
    case 1: return launch_mb<1>(a, grid, s);
    case 2: return launch_mb<2>(a, grid, s);
    case 3: return launch_mb<3>(a, grid, s);
    default: return launch_mb<4>(a, grid, s);
  }
}

}  // namespace dl
