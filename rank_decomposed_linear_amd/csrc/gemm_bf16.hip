// bf16 MFMA GEMM for prefill-sized M: one factor of a decomposed projection
// (W ~ A B, DeInfer section 2.1, Eq. (1)), C = X W with f32 accumulation.
//
// Tile 256 x 256 x 32, 8 waves (two per SIMD, so one wave's LDS traffic and
// barrier wait hide under the other's MFMAs). Each wave owns a 128 x 64
// block of C: 8 x 4 accumulator blocks of v_mfma_f32_16x16x32_bf16.
//
// Both operands sit in LDS in MFMA operand-tile order (16 rows x 32 k per
// 1 KB, lane l at byte 16 l), so every operand read is one conflict-free
// ds_read_b128 of a contiguous 1 KB and every staging write is one too. The
// factors already live in that order in HBM (Wt [N, K] in 16 x 32 tiles): a
// weight tile's k step is 16 contiguous 1 KB fragments. Activations that
// the layer produces itself are stored in the same tiles, so their
// fragments are contiguous too (16 rows x 64 bytes per fragment in
// row-major activations touch half of 16 cache lines, and staging them cost
// about a tenth of the GEMM's rate); row-major activations from the caller
// are read with lane l fetching row (l % 16), k columns 8 (l / 16) .. +7 of
// its fragment. Staging is direct to LDS
// (global_load_lds_dwordx4: lane l of a wave lands at byte 16 l of the
// wave's 1 KB destination), so no registers or LDS store instructions carry
// it. Four separately declared 32 KB stage buffers (the compiler then sees
// that the loads into one do not alias the operand reads from another):
// tile kt + 3 is in flight while tile kt is multiplied, which hides the
// load latency that a two-buffer pipeline leaves exposed at every k step.
//
// Work order: the hardware deals workgroups to the eight XCDs round-robin;
// the linear index is remapped so each XCD runs a contiguous range of tiles,
// taken in groups of kGroupM row tiles, so the CUs sharing an XCD's L2 share
// activation rows and weight columns.
#include <algorithm>
#include <atomic>

#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace dl {

namespace {
constexpr int BM = 256, BN = 256, BK = 32;
constexpr int kThreads = 512;
constexpr int kFrags = (BM / 16) * (BK / 32);  // 1 KB fragments per operand per stage
constexpr int kStage = 2 * kFrags * 64;        // u32x4 per stage (A then B)
constexpr int kXcds = 8;
constexpr int kGroupM = 4;
constexpr int kEpPitch = 256 + 4;  // f32 row pitch of the epilogue's LDS rows
constexpr int kEpRows = 32;        // rows per epilogue pass (one stage buffer)

// Linear tile index of workgroup `bid` among `total`: the XCD x = bid % 8
// runs the contiguous range [start_x, start_x + count_x) (a bijection).
__device__ __forceinline__ int xcd_linear(int bid, int total) {
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int q = total / kXcds, rem = total % kXcds;
  return xcd < rem ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
}

// Linear tile index -> (row tile, column tile), in groups of kGroupM row tiles.
__device__ __forceinline__ void tile_rc(int L, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int per_group = kGroupM * tiles_n;
  const int g = L / per_group, w = L - g * per_group;
  const int gm = min(kGroupM, tiles_m - g * kGroupM);
  tn = w / gm;
  tm = g * kGroupM + (w - tn * gm);
}

__device__ __forceinline__ int seg_of(const GemmArgs &a, int tn) {
  int si = 0;
  if (a.nseg > 1 && tn >= a.seg[1].tile_begin) si = 1;
  if (a.nseg > 2 && tn >= a.seg[2].tile_begin) si = 2;
  return si;
}

// Output modes that read a second operand R at the output positions.
__host__ __device__ constexpr bool reads_r(int om) {
  return om == GEMM_OUT_SWIGLU || om == GEMM_OUT_BF16_RES_F32 || om == GEMM_OUT_F32_RES_BF16;
}

// R at row m, columns n .. n + 7: 16 bytes of bf16 in r[0], or 32 bytes of
// f32 in r[0], r[1].
__device__ __forceinline__ void load_r(const GemmSeg &sg, int om, int m, int n, u32x4 (&r)[2]) {
  if (om == GEMM_OUT_BF16_RES_F32) {
    const u32x4 *rp = reinterpret_cast<const u32x4 *>(static_cast<const float *>(sg.R) +
                                                      static_cast<size_t>(m) * sg.ldr + n);
    r[0] = rp[0];
    r[1] = rp[1];
  } else if (om == GEMM_OUT_SWIGLU || om == GEMM_OUT_F32_RES_BF16) {
    const size_t o = sg.r_tiled ? tile_off(m, n, sg.ldr) : static_cast<size_t>(m) * sg.ldr + n;
    r[0] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(sg.R) + o);
  }
}

// Applies the output mode to the f32 results of row m, columns n .. n + 7
// (r: R there, from load_r, for the modes that read it), and stores them.
// OM >= 0: every segment of the launch has mode OM, so only its code is
// compiled (no other mode's loads whose pending registers would make the
// compiler wait for every earlier store); OM < 0: the segment's own.
// Results that are not read again soon are stored non-temporally (they
// would otherwise evict the operand tiles the CUs of an XCD share from L2).
template <int OM>
__device__ __forceinline__ void epi_store(const GemmArgs &a, const GemmSeg &sg, int m, int n,
                                          float (&v)[8], const u32x4 (&r)[2]) {
  const int om = OM >= 0 ? OM : sg.omode;
  if (om == GEMM_OUT_CACHE || om == GEMM_OUT_CACHE_T) {
    // key cache page [kPage, N] / value cache page [N, kPage], operand tiles
    const int b = m / a.T, pos = a.past_lens[b] + (m - b * a.T);
    const int pg = cache_page(a.block_table, a.page_stride, b, pos / kPage);
    uint16_t *pool = static_cast<uint16_t *>(sg.C);
    if (om == GEMM_OUT_CACHE) {
      *reinterpret_cast<u32x4 *>(pool + key_off(pg, pos, n, sg.N)) =
          u32x4{pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) pool[val_off(pg, pos, n + e, sg.N)] = f2bf(v[e]);
    }
    return;
  }
  const size_t o = static_cast<size_t>(m) * sg.ldc + n;
  if (om == GEMM_OUT_RELU) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = fmaxf(v[e], 0.f);
  } else if (om == GEMM_OUT_SWIGLU) {
    // R (the gate values) may be C itself: each element is read and then
    // overwritten by this thread only
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] *= silu(bflo(r[0][e]));
      v[2 * e + 1] *= silu(bfhi(r[0][e]));
    }
  } else if (om == GEMM_OUT_BF16_RES_F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] += __uint_as_float(r[0][e]);
      v[4 + e] += __uint_as_float(r[1][e]);
    }
    if (sg.C32) {
      __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]},
                                  reinterpret_cast<f32x4 *>(sg.C32 + o));
      __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]},
                                  reinterpret_cast<f32x4 *>(sg.C32 + o + 4));
    }
  } else if (om == GEMM_OUT_F32_RES_BF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] += bflo(r[0][e]);
      v[2 * e + 1] += bfhi(r[0][e]);
    }
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]},
                                reinterpret_cast<f32x4 *>(sg.C32 + o));
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]},
                                reinterpret_cast<f32x4 *>(sg.C32 + o + 4));
    return;
  }
  // bf16 C: the eight columns n .. n + 7 of row m are contiguous in both
  // layouts
  const size_t oc = sg.c_tiled ? tile_off(m, n, sg.ldc) : o;
  __builtin_nontemporal_store(
      u32x4{pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])},
      reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(sg.C) + oc));
}

constexpr int kEpU4 = (kEpRows * kEpPitch + 3) / 4;  // epilogue rows in u32x4 units
template <int OM>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmArgs a) {
  __shared__ u32x4 stage0[kStage > kEpU4 ? kStage : kEpU4];
  __shared__ u32x4 stage1[kStage];
  __shared__ u32x4 stage2[kStage];
  __shared__ u32x4 stage3[kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;

  // Workgroups below a.full run whole tiles; the rest are the split units:
  // unit u takes part u % split of the k tiles of tile a.full + u / split.
  const int ktiles_all = a.K / BK;
  int L, kbeg = 0, ktiles = ktiles_all, unit = -1;
  if (static_cast<int>(blockIdx.x) < a.full) {
    L = xcd_linear(blockIdx.x, a.full);
  } else {
    unit = blockIdx.x - a.full;
    const int part = unit % a.split;
    L = a.full + unit / a.split;
    kbeg = part * ktiles_all / a.split;
    ktiles = (part + 1) * ktiles_all / a.split - kbeg;
  }
  int tm, tn;
  tile_rc(L, a.tiles_m, a.tiles_n, tm, tn);
  const GemmSeg &sg = a.seg[seg_of(a, tn)];
  const int n0 = (tn - sg.tile_begin) * BN;
  const int m0 = tm * BM;
  const int K = a.K;

  // Staging: thread t moves fragment (wave + 8 i), lane `lane`, of both
  // operands, i = 0..1: row block wave + 8 i of the 32-wide k tile.
  // Out-of-range rows and weight rows are clamped (their results are never
  // stored), so every load is issued.
  // Row-major X: lane l fetches row (l % 16), k columns 8 (l / 16) .. +7 of
  // the fragment (16 rows x 64 bytes); tiled X: the fragment is one
  // contiguous 1 KB, lane l its bytes 16 l .. 16 l + 15.
  const uint16_t *xp[2];
  const uint16_t *wp[2];
  const int nblk_last = (sg.N >> 4) - 1;
  const bool xt = a.xmode == GEMM_X_TILED;
  const int xstep = xt ? 512 : BK;   // elements from one k tile to the next
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rb = wave + 8 * i;
    if (xt) {
      const int rbk = min((m0 >> 4) + rb, (a.M - 1) >> 4);
      xp[i] = sg.X + frag_off(rbk, kbeg, sg.ldx, lane);
    } else {
      const int row = min(m0 + 16 * rb + (lane & 15), a.M - 1);
      xp[i] = sg.X + static_cast<size_t>(row) * sg.ldx + 8 * (lane >> 4) + kbeg * BK;
    }
    const int nb = min((n0 >> 4) + rb, nblk_last);
    wp[i] = sg.W + frag_off(nb, kbeg, K, lane);
  }
  // direct-to-LDS staging of k tile kt into `dst`: unit i of this wave fills
  // the 1 KB fragment wave + 8 i of each operand
  typedef const void __attribute__((address_space(1))) *gptr;
  typedef void __attribute__((address_space(3))) *lptr;
  auto dma = [&](u32x4 *dst, int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_global_load_lds((gptr)(xp[i] + static_cast<size_t>(kt) * xstep),
                                       (lptr)(dst + (wave + 8 * i) * 64), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gptr)(wp[i] + static_cast<size_t>(kt) * 512),
                                       (lptr)(dst + kFrags * 64 + (wave + 8 * i) * 64), 16, 0,
                                       0);
    }
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One basic block per k tile, so the scheduling groups below can order
  // it: the loads of tile kt + 3 and this tile's B fragments first, then each
  // A fragment read three fragments ahead of its four MFMAs. The tile ends
  // when this wave's loads of tile kt + 1 have landed (loads complete in
  // issue order, so the 8 loads of tiles kt + 2 and kt + 3 may remain) and a
  // barrier. Near the end, the loads of tiles past the last reload the last
  // tile into a buffer that is not read again. The loop is unrolled by four
  // so every buffer is static.
  // s_waitcnt vmcnt(8) lgkmcnt(0) (gfx9 encoding: vmcnt bits 3:0 and 15:14,
  // expcnt 6:4, lgkmcnt 11:8), then a barrier without a memory fence. The
  // builtin wait is visible to the compiler's own wait insertion.
  auto bar_after_wait = [] {
    __builtin_amdgcn_s_waitcnt(0x0078);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto ktile = [&](const u32x4 *base, u32x4 *next, int kt) {
    dma(next, min(kt + 3, ktiles - 1));
    u32x4 bq[4], ar[8];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) bq[nb] = base[kFrags * 64 + (wn * 4 + nb) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) ar[i] = base[(wm * 8 + i) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[i][nb] = mfma_bf16(ar[i], bq[nb], acc[i][nb]);
    // groups: 0x008 MFMA, 0x020 VMEM read, 0x100 DS read
    __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 7, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i + 3 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    // this wave's tile kt + 1 has landed and its operand reads of tile kt
    // have returned; no memory fence (which would wait for every load)
    bar_after_wait();
  };
  dma(stage0, 0);
  dma(stage1, min(1, ktiles - 1));
  dma(stage2, min(2, ktiles - 1));
  bar_after_wait();
  int kt = 0;
  for (; kt + 3 < ktiles; kt += 4) {
    ktile(stage0, stage3, kt);
    ktile(stage1, stage0, kt + 1);
    ktile(stage2, stage1, kt + 2);
    ktile(stage3, stage2, kt + 3);
  }
  if (kt < ktiles) ktile(stage0, stage3, kt);
  if (kt + 1 < ktiles) ktile(stage1, stage0, kt + 1);
  if (kt + 2 < ktiles) ktile(stage2, stage1, kt + 2);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Epilogue, in eight passes of 32 rows: the waves owning the pass's rows
  // park their f32 accumulators in LDS (row pitch kEpPitch, so the 16-lane
  // column groups of an accumulator row land in distinct banks), then every
  // thread takes 8 consecutive columns of a row and applies the segment's
  // output mode with 16-byte accesses. Lane (j, grp) of block (mb, nb) holds
  // C[128 wm + 16 mb + 4 grp + r][64 wn + 16 nb + j].
  // Pass barriers order LDS accesses only: s_waitcnt lgkmcnt(0), then
  // s_barrier without a fence, so each pass's global stores stay in flight
  // under the next pass (a fenced barrier waits for them).
  auto bar_lds = [] {
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  const int j = lane & 15, grp = lane >> 4;
  float *ep = reinterpret_cast<float *>(stage0);
  const int c8 = 8 * (tid & 31);
  const int n = n0 + c8;
  // R of this thread's two rows of a pass, loaded one pass ahead (before the
  // previous pass's stores, so waiting for it leaves those stores in flight)
  constexpr bool kR = OM >= 0 && reads_r(OM);
  u32x4 rq[2][2][2];
  // (rows and columns clamped into R, so every load is issued and no
  // branch splits the wait counting; clamped values are not used)
  auto fetch_r = [&](int p, u32x4 (&dst)[2][2]) {
#pragma unroll
    for (int it = 0; it < kEpRows / 16; ++it) {
      const int m = min(m0 + kEpRows * p + (tid >> 5) + 16 * it, a.M - 1);
      load_r(sg, OM, m, min(n, sg.N - 8), dst[it]);
    }
  };
  if constexpr (kR) fetch_r(0, rq[0]);
#pragma unroll
  for (int p = 0; p < BM / kEpRows; ++p) {
    if (wm == (p >> 2)) {
#pragma unroll
      for (int mh = 0; mh < 2; ++mh)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            ep[(mh * 16 + 4 * grp + r) * kEpPitch + wn * 64 + nb * 16 + j] = acc[2 * (p & 3) + mh][nb][r];
    }
    bar_lds();
    if constexpr (kR) {
      if (p + 1 < BM / kEpRows) fetch_r(p + 1, rq[(p + 1) & 1]);
    }
    if (n < sg.N) {
#pragma unroll
      for (int it = 0; it < kEpRows / 16; ++it) {
        const int rr = (tid >> 5) + 16 * it;
        const int m = m0 + kEpRows * p + rr;
        if (m >= a.M) continue;
        const f32x4 lo = *reinterpret_cast<const f32x4 *>(ep + rr * kEpPitch + c8);
        const f32x4 hi = *reinterpret_cast<const f32x4 *>(ep + rr * kEpPitch + c8 + 4);
        float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if (unit >= 0) {
          // split unit: the f32 partial tile, row-major [BM, BN]
          float *pp = a.part + (static_cast<size_t>(unit) * BM + kEpRows * p + rr) * BN + c8;
          *reinterpret_cast<f32x4 *>(pp) = lo;
          *reinterpret_cast<f32x4 *>(pp + 4) = hi;
          continue;
        }
        if constexpr (kR) {
          epi_store<OM>(a, sg, m, n, v, rq[p & 1][it]);
        } else {
          u32x4 r[2];
          load_r(sg, OM >= 0 ? OM : sg.omode, m, n, r);
          epi_store<OM>(a, sg, m, n, v, r);
        }
      }
    }
    bar_lds();
  }
}

// Sum of the split tiles' partials and the output mode: workgroup (i, rb)
// takes rows 8 rb .. 8 rb + 7 of split tile i, thread t row t / 32 of them
// and columns 8 (t % 32) .. +7; the parts are added in order.
constexpr int kFixThreads = 256, kFixRows = kFixThreads / 32;
__global__ __launch_bounds__(kFixThreads) void gemm_bf16_fixup_kernel(GemmArgs a) {
  const int i = blockIdx.x / (BM / kFixRows), rb = blockIdx.x % (BM / kFixRows);
  int tm, tn;
  tile_rc(a.full + i, a.tiles_m, a.tiles_n, tm, tn);
  const GemmSeg &sg = a.seg[seg_of(a, tn)];
  const int row = rb * kFixRows + (threadIdx.x >> 5), c8 = 8 * (threadIdx.x & 31);
  const int m = tm * BM + row, n = (tn - sg.tile_begin) * BN + c8;
  if (m >= a.M || n >= sg.N) return;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < a.split; ++q) {
    const float *pp = a.part + (static_cast<size_t>(i * a.split + q) * BM + row) * BN + c8;
    const f32x4 lo = *reinterpret_cast<const f32x4 *>(pp);
    const f32x4 hi = *reinterpret_cast<const f32x4 *>(pp + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] += lo[e];
      v[4 + e] += hi[e];
    }
  }
  u32x4 r[2];
  load_r(sg, sg.omode, m, n, r);
  epi_store<-1>(a, sg, m, n, v, r);
}

// Compute units of the current device (256 when it cannot be asked).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Remainder split. With one workgroup per compute unit (the stage buffers
// fill the LDS), `tiles` tiles run in rounds of C; the last round has only
// r = tiles % C of them. Cutting each of those r tiles into s parts of its k
// range gives r s units that take ceil(r s / C) rounds of 1 / s the length,
// at the price of writing and re-reading an f32 partial tile per unit and a
// fixup launch. Cost model in k steps of a whole tile (about 0.9 us at the
// measured MFMA rate): a partial tile's 512 KB of traffic is about 0.1 of
// one, the fixup launch about 5. The best s in 2..8 (each part at least 16
// k steps) is taken when it saves at least 10 k steps.
constexpr int kMaxSplit = 8, kMinPartK = 16;
constexpr double kPartCost = 0.1, kFixCost = 5.0, kMinGain = 10.0;
struct SplitPlan {
  int full, split;
};
SplitPlan split_plan(int tiles, int ktiles) {
  const int C = device_cus(), r = tiles % C;
  SplitPlan p{tiles, 1};
  if (r == 0) return p;
  double best = kMinGain;
  for (int s = 2; s <= kMaxSplit && ktiles / s >= kMinPartK; ++s) {
    const int units = r * s, rounds = (units + C - 1) / C;
    const double gain = ktiles * (1.0 - static_cast<double>(rounds) / s) - units * kPartCost - kFixCost;
    if (gain > best) {
      best = gain;
      p.full = tiles - r;
      p.split = s;
    }
  }
  return p;
}
}  // namespace

size_t gemm_part_bytes(int M, int ntiles_n, int K) {
  if (M <= 0 || ntiles_n <= 0 || K < BK) return 0;
  const int64_t tiles = static_cast<int64_t>(ntiles_n) * ((M + BM - 1) / BM);
  if (tiles > INT32_MAX) return 0;
  const SplitPlan p = split_plan(static_cast<int>(tiles), K / BK);
  return static_cast<size_t>(tiles - p.full) * p.split * BM * BN * sizeof(float);
}

int gemm_ntiles(int N) { return (N + BN - 1) / BN; }

hipError_t launch_gemm_bf16(GemmArgs &a, hipStream_t s) {
  TraceGuard trace_guard(K_GEMM_BF16, s);
  int tiles = 0;
  for (int i = 0; i < a.nseg; ++i) {
    a.seg[i].tile_begin = tiles;
    tiles += gemm_ntiles(a.seg[i].N);
  }
  a.tiles_n = tiles;
  a.tiles_m = (a.M + BM - 1) / BM;
  const int64_t total = static_cast<int64_t>(a.tiles_n) * a.tiles_m;
  if (total <= 0 || total > INT32_MAX || a.K < BK) return hipErrorInvalidValue;
  a.full = static_cast<int>(total);
  a.split = 1;
  const size_t need = gemm_part_bytes(a.M, a.tiles_n, a.K);
  if (need > 0 && a.part && a.part_bytes >= need) {
    const SplitPlan p = split_plan(static_cast<int>(total), a.K / BK);
    a.full = p.full;
    a.split = p.split;
  }
  const int64_t grid = a.full + static_cast<int64_t>(total - a.full) * a.split;
  int om = a.seg[0].omode;
  for (int i = 1; i < a.nseg; ++i)
    if (a.seg[i].omode != om) om = -1;
  const dim3 g(static_cast<unsigned>(grid));
  switch (om) {
    case GEMM_OUT_BF16: gemm_bf16_kernel<GEMM_OUT_BF16><<<g, kThreads, 0, s>>>(a); break;
    case GEMM_OUT_SWIGLU: gemm_bf16_kernel<GEMM_OUT_SWIGLU><<<g, kThreads, 0, s>>>(a); break;
    case GEMM_OUT_RELU: gemm_bf16_kernel<GEMM_OUT_RELU><<<g, kThreads, 0, s>>>(a); break;
    case GEMM_OUT_BF16_RES_F32: gemm_bf16_kernel<GEMM_OUT_BF16_RES_F32><<<g, kThreads, 0, s>>>(a); break;
    case GEMM_OUT_F32_RES_BF16: gemm_bf16_kernel<GEMM_OUT_F32_RES_BF16><<<g, kThreads, 0, s>>>(a); break;
    default: gemm_bf16_kernel<-1><<<g, kThreads, 0, s>>>(a); break;
  }
  if (a.split > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned fix = static_cast<unsigned>(total - a.full) * (BM / kFixRows);
    gemm_bf16_fixup_kernel<<<dim3(fix), kFixThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace dl
