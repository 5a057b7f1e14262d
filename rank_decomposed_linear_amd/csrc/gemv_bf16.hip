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
template <int XM>
__device__ __forceinline__ u32x4 load_x(const uint16_t *X, int ldx, int row, int mb, int k, int lane) {
  if constexpr (XM == XM_TILED)
    return *reinterpret_cast<const u32x4 *>(X + frag_off(mb, k >> 5, ldx, lane));
  else
    return *reinterpret_cast<const u32x4 *>(X + static_cast<size_t>(row) * ldx + k);
}

template <int MB, int XM, int PAIRED, int RS, int R, int kWaves>
__global__ __launch_bounds__(kWaves * 64) void gemv_kernel(GvArgs a) {
  constexpr bool XT = XM == XM_TILED;
  constexpr int kThreads = kWaves * 64;
  constexpr int HALVES = PAIRED ? 2 : 1;
  constexpr int NACC = HALVES * R * MB;      // f32x4 accumulators per lane
  constexpr int RED = NACC * 4 * 64;         // floats of one wave's sums
  constexpr int PART = RED;                  // floats of one split's partial sums
  __shared__ __attribute__((aligned(16))) float wsum[kWaves][RED];
  __shared__ __attribute__((aligned(16))) float red[PART];
  __shared__ float rscale[MB * 16];
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, grp = lane >> 4;
  // work item = (K split, group of R consecutive 16-row tiles of one
  // segment); `tile` numbers the groups
  const int item = xcd_item(blockIdx.x, gridDim.x);
  if (item >= a.ntiles * a.ksplit) return;
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
  auto load_stage = [&](Stage &sb, int st) {
    int k = st * 32;
    const bool second = PAIRED && k >= a.K;
    const uint16_t *X = static_cast<const uint16_t *>(second ? sg.X2 : sg.X);
    const int ldx = second ? sg.ldx2 : sg.ldx;
    k -= second ? a.K : 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
      sb.w[r] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4 *>((second ? w2[r] : w1[r]) + static_cast<size_t>(k >> 5) * 512));
    if (!XT) k += 8 * grp;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) sb.x[mb] = load_x<XM>(X, ldx, min(mb * 16 + j, a.M - 1), mb, k, lane);
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
  if constexpr (RS) {
#pragma unroll
    for (int i = 0; i < RSR; ++i)
#pragma unroll
      for (int c = 0; c < RSC; ++c)
        rs_acc[i][c] = a.rs_part[static_cast<size_t>(min(wave + kWaves * i, a.M - 1)) * a.rs_cols +
                                 min(lane + 64 * c, a.rs_cols - 1)];
  }
  if (nst > 0) {
    Stage ring[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      load_stage(ring[d], min(st0 + kWaves * d, st_last));
      __builtin_amdgcn_sched_barrier(0);   // stages issue in ring order
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
        sq += a.rs_part[static_cast<size_t>(min(m, a.M - 1)) * a.rs_cols + c];
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
          wsum[wave][(((h * R + r) * MB + mb) * 4 + e) * 64 + lane] = acc[h][r][mb][e];
  __syncthreads();
  for (int idx = tid; idx < RED; idx += kThreads) {
    float v = wsum[0][idx];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += wsum[w][idx];
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
    if (!last_flag) return;
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
  const size_t oi = static_cast<size_t>(m) * sg.ldo + n;
  switch (sg.omode) {
    case GV_OUT_BF16:
      *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(sg.out) + oi) =
          u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
      break;
    case GV_OUT_F32:
      *reinterpret_cast<f32x4 *>(static_cast<float *>(sg.out) + oi) = f32x4{v[0], v[1], v[2], v[3]};
      break;
    case GV_OUT_TILED:
      *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(sg.out) + tile_off(m, n, sg.N)) =
          u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
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
        const f32x4 rr = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(sg.R) + ri);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += rr[r];
      } else {
        const u32x2 rr = *reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(sg.R) + ri);
        v[0] += bflo(rr.x);
        v[1] += bfhi(rr.x);
        v[2] += bflo(rr.y);
        v[3] += bfhi(rr.y);
      }
      const f32x4 o = f32x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4 *>(static_cast<float *>(sg.out) + oi) = o;
      if (sg.out2) *reinterpret_cast<f32x4 *>(sg.out2 + oi) = o;
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
        *reinterpret_cast<u32x2 *>(sg.out_nt + tile_off(m, n, sg.N)) =
            u32x2{pack2(o[0] * gn[0], o[1] * gn[1]), pack2(o[2] * gn[2], o[3] * gn[3])};
        float sq = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
        sq += __shfl_xor(sq, 1, 64);
        sq += __shfl_xor(sq, 2, 64);
        if (q == 0) sg.ssq_out[static_cast<size_t>(m) * (sg.N >> 4) + (n >> 4)] = sq;
      }
      break;
    }
    case GV_OUT_RES_BF16: {
      const f32x4 rr = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(sg.R) +
                                                         static_cast<size_t>(m) * sg.ldr + n);
      *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(sg.out) + oi) =
          u32x2{pack2(v[0] + rr[0], v[1] + rr[1]), pack2(v[2] + rr[2], v[3] + rr[3])};
      break;
    }
    default: {  // GV_OUT_SWIGLU, GV_OUT_SWIGLU_TILED
      float g2[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) g2[r] = silu(v[r]) * red[(((1 * R + rt) * MB + mb) * 4 + r) * 64 + ln];
      const size_t o = sg.omode == GV_OUT_SWIGLU_TILED ? tile_off(m, n, sg.N) : oi;
      *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(sg.out) + o) = u32x2{pack2(g2[0], g2[1]), pack2(g2[2], g2[3])};
      break;
    }
  }
  }
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
  // or quartering the activation reads): the widest item whose count still
  // fills 7/8 of the compute units in one unsplit round. (Pairing tiles of a
  // split launch by raising its split measured slower: shorter streams per
  // wave, larger merges.) Four tiles only up to 32 token rows (LDS).
  int R = 1;
  if (a.waves == 4) {
    const int forced = env_int("DL_GEMV_R", 0);
    const int fill = (7 * cus + 7) / 8;
    R = forced == 1 || forced == 2 || forced == 4 ? forced
        : tiles >= 4 * fill && a.M <= 32        ? 4
        : tiles >= 2 * fill                     ? 2
                                                : 1;
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
