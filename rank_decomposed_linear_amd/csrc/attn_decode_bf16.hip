// Decode attention over the low-rank KV cache, bf16 MFMA (DeInfer section
// 4.2: rebuild K = C_k B_k and V = C_v B_v from the cached latents, rotate
// the rebuilt keys, attend). One query token per sequence.
//
// The value side is never rebuilt: softmax(s) V = (softmax(s) C_v) B_v
// (associativity of the product; only the rounding order changes), so the
// probabilities are applied to the r_v-wide latents and the result is
// multiplied by B_v once per work item. The keys must be rebuilt per
// position because the rotary embedding acts on them after B_k.
//
// Work item = (sequence b, kv head g, context split), one workgroup of four
// waves (one per SIMD, so each wave has the whole register file for deep
// software pipelining). Per work item:
//  * Factors and caches are stored in 16 x 32 operand tiles (1 KB, MFMA
//    lane order): B_k^T / B_v^T as [n_kv * d, r]; the caches in pages of 64
//    positions, a key page as [64, r_k], a value page as [r_v, 64], reached
//    through the sequence's block table (or contiguously). Every operand
//    fragment below is one contiguous 1 KB read.
//  * The B_k^T tiles of head g are copied once into LDS, fragment (rank
//    step rs, d block x) = dimensions 16x .. 16x+15. The rotary partner of
//    dimension 16x + i is 16(x + d/32) + i: same lane, same register of the
//    rebuilt keys. (For ranks too large for LDS, the leading rank steps
//    stay resident and the rest are restaged per position group through a
//    two-step tail area.)
//  * LDS is sized per launch: the resident factor first, then as long a
//    context chunk as the rest of the 160 KB holds (scores and
//    probabilities need 4 G + 32 bytes per position), so a split is
//    normally walked in one chunk:
//    phase 1: each wave rebuilds K^T for up to 64 positions at a time, an
//      even share of the chunk's 16-position blocks per wave (A = factor
//      fragment from LDS, read one rank step ahead; B = key-cache tile of
//      16 positions, eight rank steps ahead), rotates the pairs in
//      registers and forms S^T = K Q^T straight from the accumulators (the
//      reduction slots of an operand may be any permutation shared by both
//      operands). Scores go to LDS.
//    softmax: chunk max per head, probabilities in bf16 operand order in
//      LDS, running max / sum, rescale factor.
//    phase 2: U^T[r][h] += C_v^T[r][pos] P^T[pos][h]; A = value-cache tile
//      (16 ranks x 32 positions), each wave owns a set of 16-row rank
//      blocks. The loads start before the softmax barrier.
//  * O^T = B_v^T U^T on MFMA (U rounded to bf16), then the split's partial
//    (O, max, sum) is merged by the last workgroup of (b, g) to finish
//    (device-coherent partials, one counter atomic per workgroup).
//  * Rotary angles: the turn fraction pos * w_i / (2 pi) is split into a
//    per-slice base reduced exactly in float64 and a small float32 offset,
//    so float32 sin/cos see an argument in [-pi, pi] at any position.
#include <math.h>
#include <stdlib.h>

#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace dl {

namespace {

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ void store_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ f32x4 load4_coherent(const float *p) {
  return f32x4{load_coherent(p), load_coherent(p + 1), load_coherent(p + 2), load_coherent(p + 3)};
}
__device__ __forceinline__ void store4_coherent(float *p, f32x4 v) {
#pragma unroll
  for (int r = 0; r < 4; ++r) store_coherent(p + r, v[r]);
}

// XCD-aware order: consecutive work items (the kv heads of one context
// split of one sequence, which read the same cache rows) share an XCD.
__device__ __forceinline__ int xcd_item(int b, int grid) {
  const int per = grid >> 3;
  return (b & 7) * per + (b >> 3);
}

// rotary turn fraction of (position, frequency) -> (cos, sin)
__device__ __forceinline__ void turn_cs(float t, float &c, float &s) {
  t -= rintf(t);
  __sincosf(t * 6.283185307179586f, &s, &c);
}

// s_waitcnt immediate that waits until at most n vector loads are in flight
// and leaves the other counters free (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// zero the bf16 elements e >= nv of an 8-element operand
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int nv) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t m = (2 * q < nv ? 0x0000ffffu : 0u) | (2 * q + 1 < nv ? 0xffff0000u : 0u);
    v[q] &= m;
  }
  return v;
}

constexpr int kNW = 4;                  // waves per workgroup
constexpr int kThreads = 64 * kNW;
constexpr int kSlice = 64;              // positions per wave slice in phase 1
constexpr int kNP = kSlice / 16;        // 16-position blocks per slice
constexpr int kMaxPitch = 2048;         // positions per softmax chunk (at most)
constexpr int kCDepth = 8;              // cache-row prefetch depth (rank steps)
constexpr int kVDepth = 4;              // value-row prefetch depth (32-position groups)

template <int D>
struct Tile {
  static constexpr int CPL = D / 32;   // columns per lane per column group
  static constexpr int NE = CPL;       // operands per column group
  static constexpr int NB = 2 * NE;    // 16-wide d blocks
  static constexpr int HALF = D / 2;
  __device__ static constexpr int dim(int blk, int row) { return 16 * blk + row; }
};


// The end of a work item (every thread of the workgroup calls it after a
// barrier): O^T = B_v^T U^T on MFMA by waves 0..3 (U rounded to bf16, read
// from LDS [16][r_v] at the start of dlds, or from this item's rows of the
// workspace when ugi is set), normalised into the output, or stored as the
// split's partial (O, max, sum) with device-coherent stores; then the last
// workgroup of (b, g) to arrive merges the splits.
template <int D, int NT>
__device__ __forceinline__ void finish_item(const AttnDecodeArgs &a, char *dlds, const float *ugi, const float *mfin,
                                            const float *lfin, float *cmb_m, float *cmb_l, int *last_flag, int w,
                                            int b, int g, int split) {
  using T = Tile<D>;
  constexpr int NB = T::NB;
  constexpr int OBW = NB / kNW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, grp = lane >> 4;
  const int G = a.n_q / a.n_kv;
  const float *ulds = reinterpret_cast<const float *>(dlds);
  const int D2 = D + 2;
  float *part = a.part + ((static_cast<size_t>(b) * a.n_q + g * G) * a.nsplit) * D2;
  if (wave < kNW) {
    // wave owns d blocks OBW * wave .. +OBW; A = B_v^T tiles, B = U (bf16)
    f32x4 oacc[OBW];
#pragma unroll
    for (int x = 0; x < OBW; ++x) oacc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float *urow = ulds + j * a.r_v + 8 * grp;
    const float *urow_g = ugi ? ugi + static_cast<size_t>(j) * a.r_v + 8 * grp : nullptr;
    for (int s0 = 0; s0 < a.r_v / 32; s0 += 2) {   // r_v / 32 is even
      u32x4 av[2][OBW];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int x = 0; x < OBW; ++x)
          av[q][x] = ld16(a.bv + frag_off(g * NB + OBW * wave + x, s0 + q, a.r_v, lane));
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        f32x4 u0, u1;
        if (ugi) {   // (rows j >= G hold finite values; their outputs are not stored)
          u0 = load4_coherent(urow_g + 32 * (s0 + q));
          u1 = load4_coherent(urow_g + 32 * (s0 + q) + 4);
        } else {
          u0 = *reinterpret_cast<const f32x4 *>(urow + 32 * (s0 + q));
          u1 = *reinterpret_cast<const f32x4 *>(urow + 32 * (s0 + q) + 4);
        }
        const u32x4 bop = u32x4{pack2(u0[0], u0[1]), pack2(u0[2], u0[3]), pack2(u1[0], u1[1]), pack2(u1[2], u1[3])};
#pragma unroll
        for (int x = 0; x < OBW; ++x) oacc[x] = mfma_bf16(av[q][x], bop, oacc[x]);
      }
    }
    // lane (head j, grp) holds O^T[16 (OBW wave + x) + 4grp + r][j]
    if (j < G) {
#pragma unroll
      for (int x = 0; x < OBW; ++x) {
        const int dd = 16 * (OBW * wave + x) + 4 * grp;
        if (a.nsplit == 1) {
          const float il = 1.f / lfin[j];
          const int col = (g * G + j) * D + dd;
          const size_t oi = a.out_tiled ? tile_off(b, col, a.n_q * D) : static_cast<size_t>(b) * a.n_q * D + col;
          if (a.out_f32)
            *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + oi) = oacc[x] * il;
          else
            *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(a.out) + oi) =
                u32x2{pack2(oacc[x][0] * il, oacc[x][1] * il), pack2(oacc[x][2] * il, oacc[x][3] * il)};
        } else {
          float *dst = part + (static_cast<size_t>(j) * a.nsplit + split) * D2;
#pragma unroll
          for (int r = 0; r < 4; ++r) store_coherent(dst + dd + r, oacc[x][r]);
          if (dd == 0) {
            store_coherent(dst + D, mfin[j]);
            store_coherent(dst + D + 1, lfin[j]);
          }
        }
      }
    }
  }
  if (a.nsplit == 1) return;

  // ---------------- last workgroup of (b, g) merges the splits ----------------
  wait_memory();
  __syncthreads();
  int *counter = a.counters + b * a.n_kv + g;
  if (tid == 0)
    *last_flag = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                a.nsplit - 1;
  __syncthreads();
  if (!*last_flag) return;
  // split statistics -> LDS (reused): sm[h][s], sl[h][s]
  float *sm = reinterpret_cast<float *>(dlds), *sl = sm + 16 * a.nsplit;
  for (int idx = tid; idx < G * a.nsplit; idx += NT) {
    const int h = idx / a.nsplit, sp = idx % a.nsplit;
    const float *src = part + (static_cast<size_t>(h) * a.nsplit + sp) * D2;
    sm[idx] = load_coherent(src + D);
    sl[idx] = load_coherent(src + D + 1);
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int sp = 0; sp < a.nsplit; ++sp) M = fmaxf(M, sm[tid * a.nsplit + sp]);
    float L = 0.f;
    for (int sp = 0; sp < a.nsplit; ++sp) {
      const float m = sm[tid * a.nsplit + sp];
      if (m != -INFINITY) L += exp2f(m - M) * sl[tid * a.nsplit + sp];
    }
    cmb_m[tid] = M;
    cmb_l[tid] = L;
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += NT) {
    const int h = idx / D, dd = idx % D;
    const float M = cmb_m[h];
    float o = 0.f;
    for (int sp0 = 0; sp0 < a.nsplit; sp0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = load_coherent(part + (static_cast<size_t>(h) * a.nsplit + min(sp0 + u, a.nsplit - 1)) * D2 + dd);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int sp = sp0 + u;
        if (sp < a.nsplit) {
          const float m = sm[h * a.nsplit + sp];
          if (m != -INFINITY) o += exp2f(m - M) * v[u];
        }
      }
    }
    const int col = (g * G + h) * D + dd;
    const size_t oi = a.out_tiled ? tile_off(b, col, a.n_q * D) : static_cast<size_t>(b) * a.n_q * D + col;
    if (a.out_f32)
      static_cast<float *>(a.out)[oi] = o / cmb_l[h];
    else
      static_cast<uint16_t *>(a.out)[oi] = f2bf(o / cmb_l[h]);
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int RBW>
__global__ __launch_bounds__(kThreads, 1) void attn_decode_kernel(AttnDecodeArgs a) {
  using T = Tile<D>;
  constexpr int NB = T::NB, NE = T::NE, HALF = T::HALF;
  constexpr int OBW = NB / kNW;          // output d blocks per wave
  // dynamic LDS: factor fragments [rs_cap][NB][64][8] bf16, scores
  // [G][pitch + 4] f32, probabilities [pitch / 32][64] operand words
  extern __shared__ __attribute__((aligned(16))) char dlds[];
  uint16_t *bs = reinterpret_cast<uint16_t *>(dlds);
  float *sS = reinterpret_cast<float *>(dlds + a.lds_bs);
  u32x4 *pbuf = reinterpret_cast<u32x4 *>(dlds + a.lds_bs + a.lds_s);
  __shared__ __attribute__((aligned(16))) u32x4 qfs[NB / 2][64];   // score operands, lane order
  __shared__ double rev64[HALF];
  __shared__ float rev32[HALF];
  __shared__ float2 step16[HALF];   // (cos, sin) of the rotation over 16 positions
  __shared__ float smax[kNW][16], psw[kNW][16];
  __shared__ float mfin[16], lfin[16], cmb_m[16], cmb_l[16];
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, grp = lane >> 4;
  const int total = a.Bsz * a.n_kv * a.nsplit;
  const int w = xcd_item(blockIdx.x, gridDim.x);
  if (w >= total) return;
  const int g = w % a.n_kv;
  const int split = (w / a.n_kv) % a.nsplit;
  const int b = w / (a.n_kv * a.nsplit);
  const int G = a.n_q / a.n_kv;
  const int ctx = a.ctx_lens[b] + a.ctx_offset;
  const int qpos = ctx - 1;
  const int p_begin = split * a.split_len;
  const int p_end = min(p_begin + a.split_len, ctx);
  const bool rope_on = a.theta != 0.f;
  const int nrs = a.r_k / 32;
  // rank steps [0, rs_cap) of the key factor stay in LDS for the whole work
  // item; the rest (ranks too large for LDS) are restaged per group in
  // chunks of rs_tail steps into the area after them
  const int rs_cap = a.rs_cap, rs_tail = a.rs_tail;
  const int n_tail = rs_tail > 0 ? (nrs - rs_cap + rs_tail - 1) / rs_tail : 0;
  const int nrb = a.r_v / 16;
  const int pitch = a.pitch;   // positions per chunk, a multiple of the slice
  // score row stride: four floats more than the chunk, so the rows of the
  // heads (read and written at the same column by lanes j = head) start in
  // different LDS banks (a multiple of 64 floats would put them all in one)
  // and stay 16-byte aligned
  const int spitch = pitch + 4;
  // cache pages of this sequence: key page = [kPage, r_k] tiles, value page
  // = [r_v, kPage] tiles (a position's page is looked up once per 16- or
  // 32-position block; the page index is uniform across the wave)
  auto page_of = [&](int p64) {
    return cache_page_uniform(a.block_table, a.page_stride, b, p64);
  };

  // up-factor fragments of rank steps [rs0, rs0 + cnt) -> dst[rs - rs0][x][lane][8]
  uint16_t *bs_tail = bs + static_cast<size_t>(rs_cap) * NB * 64 * 8;
  auto factor_src = [&](int rs0, int u) {
    const int ln = u & 63, x = (u >> 6) % NB, rs = (u >> 6) / NB;
    return a.bk + frag_off(g * NB + x, rs0 + rs, a.r_k, ln);
  };
  auto load_factor = [&](uint16_t *dst, int rs0, int cnt) {
    const int units = cnt * NB * 64;
    for (int u = tid; u < units; u += kThreads)
      *reinterpret_cast<u32x4 *>(dst + static_cast<size_t>(u) * 8) = ld16(factor_src(rs0, u));
  };

  // Prologue, ordered so the latencies overlap: this thread's query values
  // are requested first, then the first batch of the resident factor; the
  // float64 rotary tables and the query operands are computed while those
  // loads are in flight; the factor goes to LDS last.
  //
  // Score B operands (rotated, scaled queries of this kv head's G heads,
  // rows >= G zero): entry (t, lane (head j, grp)) holds slots 0..3 =
  // q[j][dim(2t, 4grp+r)], slots 4..7 = q[j][dim(2t+1, 4grp+r)]; entry tid.
  constexpr int kQE = (NB / 2) * 64;
  static_assert(kQE <= kThreads, "one query operand entry per thread");
  const int qt = tid >> 6, qj = lane & 15, qg = lane >> 4;
  const bool q_mine = tid < kQE && qj < G;
  float qlo[8], qhi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int i = T::dim(2 * qt + (e >> 2), 4 * qg + (e & 3)) % HALF;
    const size_t off = (static_cast<size_t>(b) * a.n_q + g * G + min(qj, G - 1)) * D + i;
    if (a.q_f32) {
      qlo[e] = static_cast<const float *>(a.q)[off];
      qhi[e] = static_cast<const float *>(a.q)[off + HALF];
    } else {
      qlo[e] = bf2f(static_cast<const uint16_t *>(a.q)[off]);
      qhi[e] = bf2f(static_cast<const uint16_t *>(a.q)[off + HALF]);
    }
  }
  // resident factor: batches of kPer loads per thread in flight before their
  // LDS stores; the first batch is issued here
  constexpr int kPer = 32;
  const int funits = rs_cap * NB * 64;
  u32x4 fv[kPer];
  auto factor_batch_load = [&](int u0) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) fv[k] = ld16(factor_src(0, min(u0 + tid + kThreads * k, funits - 1)));
  };
  auto factor_batch_store = [&](int u0) {
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (u0 + tid + kThreads * k < funits)
        *reinterpret_cast<u32x4 *>(bs + static_cast<size_t>(u0 + tid + kThreads * k) * 8) = fv[k];
  };
  if (funits > 0) factor_batch_load(0);
  for (int i = tid; i < HALF; i += kThreads) {
    rev64[i] = rope_on ? rope_rev(i, D, a.theta) : 0.0;
    rev32[i] = static_cast<float>(rev64[i]);
    float c16, s16;
    rope_cs(16, rev64[i], c16, s16);
    step16[i] = float2{c16, s16};
  }
  __syncthreads();
  if (tid < kQE) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dm = T::dim(2 * qt + (e >> 2), 4 * qg + (e & 3));
      float x = 0.f;
      if (q_mine) {
        if (rope_on) {
          float c, sn;
          rope_cs(qpos, rev64[dm % HALF], c, sn);
          x = dm < HALF ? qlo[e] * c - qhi[e] * sn : qlo[e] * sn + qhi[e] * c;
        } else {
          x = dm < HALF ? qlo[e] : qhi[e];
        }
      }
      v[e] = x * a.scale_log2;
    }
    qfs[qt][lane] = u32x4{pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
  }
  if (funits > 0) {
    factor_batch_store(0);
    for (int u0 = kPer * kThreads; u0 < funits; u0 += kPer * kThreads) {
      factor_batch_load(u0);
      factor_batch_store(u0);
    }
  }
  __syncthreads();

  // running softmax state of head j (every lane tracks its own column)
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 uacc[RBW];
#pragma unroll
  for (int i = 0; i < RBW; ++i) uacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this wave's rank blocks (clamped duplicates of the last one are computed
  // and discarded, so every load stays unconditional)
  int rb[RBW];
#pragma unroll
  for (int i = 0; i < RBW; ++i) rb[i] = min(wave + kNW * i, nrb - 1);
  // More rank blocks than the accumulators hold (r_v > 64 RBW): phase 2
  // runs in passes of kNW * RBW blocks and U lives in the workspace between
  // chunks (row j of this work item's [16, r_v] block; each lane reads and
  // writes only its own elements until the final product).
  const int npass = a.vpasses;
  float *ug = npass > 1 ? a.uglob + (static_cast<size_t>(w) * 16 + j) * a.r_v : nullptr;

  // Work items w = 1, 2, 3 (mod 4) take a first chunk shorter by a quarter,
  // a half and three quarters, so the value phases of a quarter of the
  // workgroups fall within the key phases of the rest: all workgroups start
  // together, and in step every value phase would pull its tiles from L2
  // at the same time.
  const int first_len = max(kSlice, (pitch - (w & 3) * (pitch / 4)) & ~(kSlice - 1));
  for (int c0 = p_begin, c1; c0 < p_end; c0 = c1) {
    c1 = min(c0 + (c0 == p_begin ? first_len : pitch), p_end);
    // ------------------------------ phase 1 ------------------------------
    // the chunk's 16-position blocks are shared out evenly, a contiguous
    // range per wave, taken kNP blocks at a time (the last group may be
    // partial: its missing blocks repeat the last one and are not scored)
    const int nblk = (c1 - c0 + 15) >> 4;
    const int share = (nblk + kNW - 1) / kNW;
    const int b_lo = min(wave * share, nblk), b_hi = min(b_lo + share, nblk);
    float mx = -INFINITY;
    const int ngr = (share + kNP - 1) / kNP;   // same count in every wave
    // key tiles of group gi: the first rank step of each 16-position block
    // (wave-uniform base; the lane's 16 bytes are added at the load); blocks
    // past the wave's range repeat its last block, are multiplied only
    // inside a group of four and never scored
    const uint16_t *kblk[kNP];
    auto set_rows = [&](int gi) {
#pragma unroll
      for (int pb = 0; pb < kNP; ++pb) {
        const int kb = (c0 >> 4) + min(b_lo + kNP * gi + pb, max(b_hi - 1, 0));
        kblk[pb] = a.ck + static_cast<size_t>(page_of(kb >> 2)) * (kPage * a.r_k) +
                   frag_off(kb & 3, 0, a.r_k, 0);
      }
    };
    for (int gi = 0; gi < ngr; ++gi) {
      const int g0 = b_lo + kNP * gi;
      const int np = max(0, min(kNP, b_hi - g0));   // blocks of this group; a partial group is the wave's last
      if (np == 0) {
        // no blocks: still take part in the workgroup's tail staging
        for (int tc = 0; tc < n_tail; ++tc) {
          const int rs0 = rs_cap + tc * rs_tail;
          __syncthreads();
          load_factor(bs_tail, rs0, min(rs_tail, nrs - rs0));
          __syncthreads();
        }
        continue;
      }
      const int P0 = c0 + 16 * g0;
      set_rows(gi);
      // the group: K^T for NPA blocks of 16 positions, rotated, scored
      auto group = [&](auto npc) {
        constexpr int NPA = decltype(npc)::value;
        f32x4 acc[NB][NPA];
#pragma unroll
        for (int x = 0; x < NB; ++x)
#pragma unroll
          for (int pb = 0; pb < NPA; ++pb) acc[x][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int rc = 0; rc <= n_tail; ++rc) {
          // chunk 0: the resident steps; chunk rc > 0: tail chunk rc - 1
          const int rs0 = rc == 0 ? 0 : rs_cap + (rc - 1) * rs_tail;
          const int cnt = rc == 0 ? rs_cap : min(rs_tail, nrs - rs0);
          const uint16_t *fb = rc == 0 ? bs : bs_tail;
          if (rc > 0) {
            __syncthreads();
            load_factor(bs_tail, rs0, cnt);
            __syncthreads();
          }
          // cache tiles kCDepth rank steps ahead; prefetches past the last
          // step repeat it (every load stays unconditional) and are never
          // multiplied
          u32x4 cf[kCDepth][NPA];
#pragma unroll
          for (int d = 0; d < kCDepth; ++d)
#pragma unroll
            for (int pb = 0; pb < NPA; ++pb) cf[d][pb] = ld16(kblk[pb] + lane * 8 + 512 * (rs0 + min(d, cnt - 1)));
          // factor fragments one rank step ahead
          u32x4 bop[2][NB];
#pragma unroll
          for (int x = 0; x < NB; ++x)
            bop[0][x] = *reinterpret_cast<const u32x4 *>(fb + (static_cast<size_t>(x) * 64 + lane) * 8);
          // One rank step: next step's factor fragments from LDS, the
          // products of this step (position block by position block, so
          // each cache tile is free for its refill after NB products), the
          // refills. With one wave per SIMD nothing else fills the matrix
          // pipe, so the LDS reads and loads are spread between the
          // products instead of issued in runs.
          auto rank_step = [&](auto dc, int s, auto refill) {
            constexpr int d = decltype(dc)::value;
            constexpr bool kRefill = decltype(refill)::value;
            const uint16_t *fr = fb + (static_cast<size_t>(min(s + 1, cnt - 1) * NB) * 64 + lane) * 8;
#pragma unroll
            for (int x = 0; x < NB; ++x) bop[(d + 1) & 1][x] = *reinterpret_cast<const u32x4 *>(fr + x * 64 * 8);
#pragma unroll
            for (int pb = 0; pb < NPA; ++pb)
#pragma unroll
              for (int x = 0; x < NB; ++x) acc[x][pb] = mfma_bf16(bop[d & 1][x], cf[d][pb], acc[x][pb]);
            if constexpr (kRefill) {
              const int sn = rs0 + min(s + kCDepth, cnt - 1);
#pragma unroll
              for (int pb = 0; pb < NPA; ++pb) cf[d][pb] = ld16(kblk[pb] + lane * 8 + 512 * sn);
            }
#pragma unroll
            for (int pb = 0; pb < NPA; ++pb) {
#pragma unroll
              for (int q = 0; q < NB / NPA; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, NPA, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // LDS read
              }
              if constexpr (kRefill) {
                __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // VALU (load address)
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
              }
            }
          };
          // Whole rounds of kCDepth steps refill the ring; the remaining
          // steps (their tiles already in flight) issue no loads, so taking
          // or skipping one leaves the same loads outstanding and the
          // compiler's per-step waits stay exact instead of draining the ring.
          int s0 = 0;
          for (; s0 + kCDepth <= cnt; s0 += kCDepth) {
            static_for<kCDepth>([&](auto dc) { rank_step(dc, s0 + decltype(dc)::value, IntC<1>{}); });
          }
          static_for<kCDepth>([&](auto dc) {
            constexpr int d = decltype(dc)::value;
            if (s0 + d < cnt) {
              // this step's tiles are the (kCDepth - d)-th newest loads
              // group: the ones issued after them may stay in flight
              __builtin_amdgcn_s_waitcnt(vmcnt_only((kCDepth - 1 - d) * NPA));
              rank_step(dc, s0 + d, IntC<0>{});
            }
          });
        }
        // lane (pos j, grp) holds K^T[16x + 4grp + r][P0 + 16pb + j]; block
        // e < NE pairs with block NE + e. The angle of block 0 is evaluated
        // (exact float64 turn base, float32 offset); each further block
        // rotates it by the 16-position step.
        if (rope_on) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < NE; ++e) {
              const int fi = 16 * e + 4 * grp + r;
              double tb = static_cast<double>(P0) * rev64[fi];
              tb -= rint(tb);
              float c, sn;
              turn_cs(static_cast<float>(tb) + static_cast<float>(j) * rev32[fi], c, sn);
              const float2 st = step16[fi];
#pragma unroll
              for (int pb = 0; pb < NPA; ++pb) {
                const float x = acc[e][pb][r], y = acc[NE + e][pb][r];
                acc[e][pb][r] = x * c - y * sn;
                acc[NE + e][pb][r] = x * sn + y * c;
                const float cn = c * st.x - sn * st.y;
                sn = c * st.y + sn * st.x;
                c = cn;
              }
            }
        }
        // S^T[pos, h]: lane (head j, grp) holds S^T[P0 + 16pb + 4grp + r][j]
#pragma unroll
        for (int pb = 0; pb < NPA; ++pb) {
          f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < NB / 2; ++t)
            sc = mfma_bf16(pack_acc(acc[2 * t][pb], acc[2 * t + 1][pb]), qfs[t][lane], sc);
          if (pb < np) {   // uniform
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int off = P0 - c0 + 16 * pb + 4 * grp + r;
              const float v = c0 + off < c1 ? sc[r] : -INFINITY;
              mx = fmaxf(mx, v);
              if (j < G) sS[j * spitch + off] = v;
            }
          }
        }
      };
      if (np >= 3) group(IntC<kNP>{});
      else if (np == 2) group(IntC<2>{});
      else group(IntC<1>{});
    }
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    if (grp == 0) smax[wave][j] = mx;
    // phase-2 value tiles do not depend on the probabilities: start them
    // now. A operand: lane (rank row j, grp) = C_v^T[16 rb + j][c0 + 32u + 8grp ..+8]
    const int nU = (c1 - c0 + 31) >> 5;
    auto vload = [&](u32x4 (&dst)[RBW], int u) {
      // 32-position group (c0 >> 5) + u: column step of its page
      const int pg32 = (c0 >> 5) + u;
      const uint16_t *vb = a.cv + static_cast<size_t>(page_of(pg32 >> 1)) * (kPage * a.r_v) +
                           (pg32 & 1) * 512 + lane * 8;
#pragma unroll
      for (int i = 0; i < RBW; ++i) dst[i] = ld16(vb + rb[i] * 1024);
    };
    u32x4 vr[kVDepth][RBW];
#pragma unroll
    for (int d = 0; d < kVDepth; ++d) {
      vload(vr[d], min(d, nU - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    // ------------------------------ softmax ------------------------------
    float m_new = m_run;
#pragma unroll
    for (int wv = 0; wv < kNW; ++wv) m_new = fmaxf(m_new, smax[wv][j]);
    const float alpha = m_run == -INFINITY ? 0.f : exp2_hw(m_run - m_new);
    m_run = m_new;
    float ps = 0.f;
    for (int u = wave; u < nU; u += kNW) {
      // eight scores of a valid row, read unconditionally (two 16-byte
      // reads); masked entries become exp2(-inf) = 0 by a select, so the
      // lanes do not branch around each read and wait on it separately
      const int off = 32 * u + 8 * grp;
      const float *srow = sS + min(j, G - 1) * spitch + off;
      const f32x4 sa = *reinterpret_cast<const f32x4 *>(srow);
      const f32x4 sb = *reinterpret_cast<const f32x4 *>(srow + 4);
      const float sv[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = exp2_hw(j < G && c0 + off + e < c1 ? sv[e] - m_new : -INFINITY);
        ps += v[e];
      }
      pbuf[u * 64 + lane] = u32x4{pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
    }
    ps = wave_sum_xor(ps, 16);
    ps = wave_sum_xor(ps, 32);
    if (grp == 0) psw[wave][j] = ps;
    __syncthreads();
    // ------------------------------ phase 2 ------------------------------
    float lsum = 0.f;
#pragma unroll
    for (int wv = 0; wv < kNW; ++wv) lsum += psw[wv][j];
    l_run = l_run * alpha + lsum;
    for (int pass = 0; pass < npass; ++pass) {
    if (npass > 1) {
      if (pass > 0) {
#pragma unroll
        for (int i = 0; i < RBW; ++i) rb[i] = min(wave + kNW * (RBW * pass + i), nrb - 1);
#pragma unroll
        for (int d = 0; d < kVDepth; ++d) {
          vload(vr[d], min(d, nU - 1));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // these blocks' U so far (none before the first chunk), rescaled
#pragma unroll
      for (int i = 0; i < RBW; ++i) {
        const f32x4 prev = c0 != p_begin ? load4_coherent(ug + 16 * rb[i] + 4 * grp) : f32x4{0.f, 0.f, 0.f, 0.f};
        uacc[i] = prev * alpha;
      }
    } else {
#pragma unroll
      for (int i = 0; i < RBW; ++i) uacc[i] *= alpha;
    }
    for (int u0 = 0; u0 < nU; u0 += kVDepth) {
#pragma unroll
      for (int d = 0; d < kVDepth; ++d) {
        const int u = min(u0 + d, nU - 1);
        u32x4 pop = pbuf[u * 64 + lane];
        if (u0 + d >= nU) pop = u32x4{0u, 0u, 0u, 0u};
        // value rows at positions >= ctx (unwritten cache) are zeroed: the
        // probabilities there are zero, but 0 * NaN would not be. Only the
        // context's last group can be ragged: a branch (uniform across the
        // wave), not a select, so the other groups carry no masking work.
        if (c0 + 32 * u + 32 > ctx) {
          const int nv = ctx - (c0 + 32 * u + 8 * grp);
#pragma unroll
          for (int i = 0; i < RBW; ++i) vr[d][i] = keep_first(vr[d][i], nv);
        }
#pragma unroll
        for (int i = 0; i < RBW; ++i) uacc[i] = mfma_bf16(vr[d][i], pop, uacc[i]);
        __builtin_amdgcn_sched_barrier(0);
        vload(vr[d], min(u0 + d + kVDepth, nU - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (npass > 1) {
#pragma unroll
      for (int i = 0; i < RBW; ++i)
        if (wave + kNW * (RBW * pass + i) < nrb) store4_coherent(ug + 16 * rb[i] + 4 * grp, uacc[i]);
    }
    }   // passes
    if (npass > 1) {
      // the next chunk's early value loads are for the first pass
#pragma unroll
      for (int i = 0; i < RBW; ++i) rb[i] = min(wave + kNW * i, nrb - 1);
    }
  }

  // ---------------- O^T = B_v^T U^T (MFMA, U rounded to bf16) ----------------
  if (npass > 1) wait_memory();   // U rows of the other waves complete before the barrier
  __syncthreads();   // LDS is reused for U
  float *ulds = reinterpret_cast<float *>(dlds);   // [16][r_v], rows >= G zero
  // lane (head j, grp) holds U^T[16 rb + 4grp + r][j]
  if (npass == 1) {
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) ulds[j * a.r_v + 16 * rb[i] + 4 * grp + r] = j < G ? uacc[i][r] : 0.f;
  }
  if (wave == 0 && grp == 0) {
    mfin[j] = m_run;
    lfin[j] = l_run;
  }
  const float *ugi = npass > 1 ? a.uglob + static_cast<size_t>(w) * 16 * a.r_v : nullptr;
  __syncthreads();
  finish_item<D, kThreads>(a, dlds, ugi, mfin, lfin, cmb_m, cmb_l, &last_flag, w, b, g, split);
}

// ---------------------------------------------------------------------------
// Warp-specialised variant (r_v <= 512, whole key factor in LDS): PW
// producer waves and four consumer waves. The producers run phase 1 of
// chunk t (key rebuild, rotation, scores into one of two score buffers)
// while the consumers run the softmax and the value products of chunk t - 1
// from the other buffer; one workgroup barrier per chunk hands the buffers
// over. With PW = 8 each SIMD holds two producers and one consumer: one
// producer's VALU epilogue and load waits overlap the other's MFMAs, and the
// consumer's value loads, exponentials and MFMAs fill what is left. Each
// consumer forms the probabilities it multiplies straight from the scores,
// so the consumers never wait for one another.
// ---------------------------------------------------------------------------
constexpr int kWsGran = 128;   // chunk lengths are multiples of this (whole value-ring rounds)

template <int D, int NPA, int CD, int PW, int VD, int BD>
__global__ __launch_bounds__(64 * (PW + kNW), 1) void attn_decode_ws_kernel(AttnDecodeArgs a) {
  constexpr int kT = 64 * (PW + kNW);   // PW producer waves, then kNW consumer waves
  using T = Tile<D>;
  constexpr int NB = T::NB, NE = T::NE, HALF = T::HALF;
  constexpr int RBW = 8;
  // dynamic LDS: factor fragments [nrs][NB][64][8] bf16, scores
  // [2][G][pitch + 4] f32, probabilities [pitch / 32][64] operand words
  extern __shared__ __attribute__((aligned(16))) char dlds[];
  uint16_t *bs = reinterpret_cast<uint16_t *>(dlds);
  float *sSall = reinterpret_cast<float *>(dlds + a.lds_bs);
  u32x4 *pbuf = reinterpret_cast<u32x4 *>(dlds + a.lds_bs + a.lds_s);
  __shared__ __attribute__((aligned(16))) u32x4 qfs[NB / 2][64];   // score operands, lane order
  __shared__ double rev64[HALF];
  __shared__ float rev32[HALF];
  __shared__ float2 step16[HALF];
  __shared__ float smax[2][PW][16];
  __shared__ float lpart[kNW][16];
  __shared__ int pdone;   // consumer probability shares published so far
  __shared__ float mfin[16], lfin[16], cmb_m[16], cmb_l[16];
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave < PW;   // uniform across the wave
  const int rw = producer ? wave : wave - PW;   // wave index within its role
  const int j = lane & 15, grp = lane >> 4;
  const int total = a.Bsz * a.n_kv * a.nsplit;
  const int w = xcd_item(blockIdx.x, gridDim.x);
  if (w >= total) return;
  const int g = w % a.n_kv;
  const int split = (w / a.n_kv) % a.nsplit;
  const int b = w / (a.n_kv * a.nsplit);
  const int G = a.n_q / a.n_kv;
  const int ctx = a.ctx_lens[b] + a.ctx_offset;
  const int qpos = ctx - 1;
  const int p_begin = split * a.split_len;
  const int p_end = min(p_begin + a.split_len, ctx);
  const bool rope_on = a.theta != 0.f;
  const int nrs = a.r_k / 32;
  const int nrb = a.r_v / 16;
  const int pitch = a.pitch;          // chunk length, a multiple of kWsGran
  const int spitch = pitch + 4;       // score row stride (bank spread, 16-byte rows)
  auto page_of = [&](int p64) { return cache_page_uniform(a.block_table, a.page_stride, b, p64); };

  // ------------------------------ prologue ------------------------------
  // query values first, then the factor in batches (loads in flight while
  // the rotary tables and the query operands are formed)
  constexpr int kQE = (NB / 2) * 64;
  static_assert(kQE <= kT, "one query operand entry per thread");
  const int qt = min(tid >> 6, NB / 2 - 1), qj = lane & 15, qg = lane >> 4;
  const bool q_mine = tid < kQE && qj < G;
  float qlo[8], qhi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int i = T::dim(2 * qt + (e >> 2), 4 * qg + (e & 3)) % HALF;
    const size_t off = (static_cast<size_t>(b) * a.n_q + g * G + min(qj, G - 1)) * D + i;
    if (a.q_f32) {
      qlo[e] = static_cast<const float *>(a.q)[off];
      qhi[e] = static_cast<const float *>(a.q)[off + HALF];
    } else {
      qlo[e] = bf2f(static_cast<const uint16_t *>(a.q)[off]);
      qhi[e] = bf2f(static_cast<const uint16_t *>(a.q)[off + HALF]);
    }
  }
  constexpr int kPer = 16;
  const int funits = nrs * NB * 64;
  auto factor_src = [&](int u) {
    const int ln = u & 63, x = (u >> 6) % NB, rs = (u >> 6) / NB;
    return a.bk + frag_off(g * NB + x, rs, a.r_k, ln);
  };
  u32x4 fv[kPer];
  auto factor_batch_load = [&](int u0) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) fv[k] = ld16(factor_src(min(u0 + tid + kT * k, funits - 1)));
  };
  auto factor_batch_store = [&](int u0) {
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (u0 + tid + kT * k < funits)
        *reinterpret_cast<u32x4 *>(bs + static_cast<size_t>(u0 + tid + kT * k) * 8) = fv[k];
  };
  factor_batch_load(0);
  if (tid == 0) pdone = 0;
  for (int i = tid; i < HALF; i += kT) {
    rev64[i] = rope_on ? rope_rev(i, D, a.theta) : 0.0;
    rev32[i] = static_cast<float>(rev64[i]);
    float c16, s16;
    rope_cs(16, rev64[i], c16, s16);
    step16[i] = float2{c16, s16};
  }
  __syncthreads();
  if (tid < kQE) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dm = T::dim(2 * qt + (e >> 2), 4 * qg + (e & 3));
      float x = 0.f;
      if (q_mine) {
        if (rope_on) {
          float c, sn;
          rope_cs(qpos, rev64[dm % HALF], c, sn);
          x = dm < HALF ? qlo[e] * c - qhi[e] * sn : qlo[e] * sn + qhi[e] * c;
        } else {
          x = dm < HALF ? qlo[e] : qhi[e];
        }
      }
      v[e] = x * a.scale_log2;
    }
    qfs[qt][lane] = u32x4{pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
  }
  factor_batch_store(0);
  for (int u0 = kPer * kT; u0 < funits; u0 += kPer * kT) {
    factor_batch_load(u0);
    factor_batch_store(u0);
  }
  __syncthreads();

  // chunks of pitch positions (a multiple of kWsGran; the last may be
  // shorter). The work items of one sequence stay in step, so the kv heads
  // that read the same cache tiles share them in L2 (staggering the items
  // measured no faster here and fetched 24% more from memory).
  const int span = max(0, p_end - p_begin);
  const int nch = (span + pitch - 1) / pitch;
  auto chunk_lo = [&](int t) { return p_begin + t * pitch; };
  auto chunk_hi = [&](int t) { return min(p_begin + (t + 1) * pitch, p_end); };

  // Each role runs its own loop over the chunks (its state stays out of the
  // other's register budget), with one barrier per iteration in both.
  float *ulds = reinterpret_cast<float *>(dlds);   // [16][r_v] at the end, rows >= G zero
  if (producer) {
    for (int it = 0; it <= nch; ++it) {
      if (it < nch) {
        // --------------------- phase 1 of chunk it ---------------------
        const int c0 = chunk_lo(it), c1 = chunk_hi(it);
        float *sS = sSall + (it & 1) * G * spitch;
        const int nblk = (c1 - c0 + 15) >> 4;
        const int share = (nblk + PW - 1) / PW;
        const int b_lo = min(rw * share, nblk), b_hi = min(b_lo + share, nblk);
        float mx = -INFINITY;
        const int ngr = (share + NPA - 1) / NPA;
        const uint16_t *kblk[NPA];
        for (int gi = 0; gi < ngr; ++gi) {
          const int g0 = b_lo + NPA * gi;
          const int np = max(0, min(NPA, b_hi - g0));
          if (np == 0) continue;
          const int P0 = c0 + 16 * g0;
#pragma unroll
          for (int pb = 0; pb < NPA; ++pb) {
            const int kb = (c0 >> 4) + min(g0 + pb, max(b_hi - 1, 0));
            kblk[pb] = a.ck + static_cast<size_t>(page_of(kb >> 2)) * (kPage * a.r_k) + frag_off(kb & 3, 0, a.r_k, 0);
          }
          auto group = [&](auto npc) {
            constexpr int NPG = decltype(npc)::value;
            f32x4 acc[NB][NPG];
#pragma unroll
            for (int x = 0; x < NB; ++x)
#pragma unroll
              for (int pb = 0; pb < NPG; ++pb) acc[x][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int cnt = nrs;
            u32x4 cf[CD][NPG];
#pragma unroll
            for (int d = 0; d < CD; ++d)
#pragma unroll
              for (int pb = 0; pb < NPG; ++pb) cf[d][pb] = ld16(kblk[pb] + lane * 8 + 512 * min(d, cnt - 1));
            // factor fragments: BD = 2 reads the next step's during this one;
            // BD = 1 reads each step's at its start (other waves on the SIMD
            // cover the latency)
            u32x4 bop[BD][NB];
            if constexpr (BD == 2) {
#pragma unroll
              for (int x = 0; x < NB; ++x)
                bop[0][x] = *reinterpret_cast<const u32x4 *>(bs + (static_cast<size_t>(x) * 64 + lane) * 8);
            }
            auto rank_step = [&](auto dc, int s, auto refill) {
              constexpr int d = decltype(dc)::value;
              constexpr bool kRefill = decltype(refill)::value;
              constexpr int cur = BD == 2 ? (d & 1) : 0;
              const uint16_t *fr =
                  bs + (static_cast<size_t>((BD == 2 ? min(s + 1, cnt - 1) : s) * NB) * 64 + lane) * 8;
#pragma unroll
              for (int x = 0; x < NB; ++x)
                bop[BD == 2 ? (d + 1) & 1 : 0][x] = *reinterpret_cast<const u32x4 *>(fr + x * 64 * 8);
#pragma unroll
              for (int pb = 0; pb < NPG; ++pb)
#pragma unroll
                for (int x = 0; x < NB; ++x) acc[x][pb] = mfma_bf16(bop[cur][x], cf[d][pb], acc[x][pb]);
              if constexpr (kRefill) {
                const int sn = min(s + CD, cnt - 1);
#pragma unroll
                for (int pb = 0; pb < NPG; ++pb) cf[d][pb] = ld16(kblk[pb] + lane * 8 + 512 * sn);
              }
            };
            int s0 = 0;
            for (; s0 + CD <= cnt; s0 += CD) {
              static_for<CD>([&](auto dc) { rank_step(dc, s0 + decltype(dc)::value, IntC<1>{}); });
            }
            static_for<CD>([&](auto dc) {
              constexpr int d = decltype(dc)::value;
              if (s0 + d < cnt) {
                __builtin_amdgcn_s_waitcnt(vmcnt_only((CD - 1 - d) * NPG));
                rank_step(dc, s0 + d, IntC<0>{});
              }
            });
            // rotation (as in the one-role kernel), then scores
            if (rope_on) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int e = 0; e < NE; ++e) {
                  const int fi = 16 * e + 4 * grp + r;
                  double tb = static_cast<double>(P0) * rev64[fi];
                  tb -= rint(tb);
                  float c, sn;
                  turn_cs(static_cast<float>(tb) + static_cast<float>(j) * rev32[fi], c, sn);
                  const float2 st = step16[fi];
#pragma unroll
                  for (int pb = 0; pb < NPG; ++pb) {
                    const float x = acc[e][pb][r], y = acc[NE + e][pb][r];
                    acc[e][pb][r] = x * c - y * sn;
                    acc[NE + e][pb][r] = x * sn + y * c;
                    const float cn = c * st.x - sn * st.y;
                    sn = c * st.y + sn * st.x;
                    c = cn;
                  }
                }
            }
#pragma unroll
            for (int pb = 0; pb < NPG; ++pb) {
              f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int t = 0; t < NB / 2; ++t)
                sc = mfma_bf16(pack_acc(acc[2 * t][pb], acc[2 * t + 1][pb]), qfs[t][lane], sc);
              if (pb < np) {   // uniform
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const int off = P0 - c0 + 16 * pb + 4 * grp + r;
                  const float v = c0 + off < c1 ? sc[r] : -INFINITY;
                  mx = fmaxf(mx, v);
                  if (j < G) sS[j * spitch + off] = v;
                }
              }
            }
          };
          if constexpr (NPA == 4) {
            if (np >= 3) group(IntC<4>{});
            else if (np == 2) group(IntC<2>{});
            else group(IntC<1>{});
          } else {
            if (np == 2) group(IntC<2>{});
            else group(IntC<1>{});
          }
        }
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);
        if (grp == 0) smax[it & 1][rw][j] = mx;
      }
      __syncthreads();
    }
  } else {
    // ------------------------- consumer state -------------------------
    float m_run = -INFINITY, l_part = 0.f;   // running max; this lane's share of the running sum
    f32x4 uacc[RBW];
#pragma unroll
    for (int i = 0; i < RBW; ++i) uacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    int rb[RBW];
#pragma unroll
    for (int i = 0; i < RBW; ++i) rb[i] = min(rw + kNW * i, nrb - 1);
    // value ring over the split's 32-position groups: slot d holds group
    // gu0 + d; groups past the last repeat it (never multiplied by a nonzero
    // probability)
    const int ngu = (span + 31) >> 5;
    u32x4 vr[VD][RBW];
    auto vload = [&](u32x4 (&dst)[RBW], int gu) {
      const int pg32 = (p_begin >> 5) + min(gu, max(ngu - 1, 0));
      const uint16_t *vb = a.cv + static_cast<size_t>(page_of(pg32 >> 1)) * (kPage * a.r_v) +
                           (pg32 & 1) * 512 + lane * 8;
#pragma unroll
      for (int i = 0; i < RBW; ++i) dst[i] = ld16(vb + rb[i] * 1024);
    };
    if (span > 0) {
#pragma unroll
      for (int d = 0; d < VD; ++d) {
        vload(vr[d], d);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    for (int it = 0; it <= nch; ++it) {
      if (it > 0) {
        // ------------- softmax and value products of chunk it - 1 -------------
        const int t = it - 1;
        const int c0 = chunk_lo(t), c1 = chunk_hi(t);
        const float *sS = sSall + (t & 1) * G * spitch;
        float m_new = m_run;
  #pragma unroll
        for (int wv = 0; wv < PW; ++wv) m_new = fmaxf(m_new, smax[t & 1][wv][j]);
        const float alpha = m_run == -INFINITY ? 0.f : exp2_hw(m_run - m_new);
        m_run = m_new;
        l_part *= alpha;
  #pragma unroll
        for (int i = 0; i < RBW; ++i) uacc[i] *= alpha;
        const float *srow = sS + min(j, G - 1) * spitch + 8 * grp;
        const int gu_lo = (c0 - p_begin) >> 5;
        const int nU = (c1 - c0 + 31) >> 5;   // a multiple of VD except in the last chunk
        // this consumer's share of the probabilities (32-position groups
        // u = rw, rw + 4, ...), in operand order: lane (head j, grp) holds
        // positions 32 u + 8 grp .. +7; positions past the chunk are zero
        for (int u = rw; u < nU; u += kNW) {
          const int off = 32 * u;
          const f32x4 sa = *reinterpret_cast<const f32x4 *>(srow + off);
          const f32x4 sb = *reinterpret_cast<const f32x4 *>(srow + off + 4);
          const float sv[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
          float v[8];
  #pragma unroll
          for (int e = 0; e < 8; ++e) {
            v[e] = exp2_hw(j < G && c0 + off + 8 * grp + e < c1 ? sv[e] - m_new : -INFINITY);
            l_part += v[e];
          }
          pbuf[u * 64 + lane] = u32x4{pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
        }
        // publish the share (this wave's LDS writes complete, then one count),
        // then wait for the other consumers' shares of this chunk; the wait is
        // bounded (a missing count would give wrong results, not a hang)
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt, expcnt free
        if (lane == 0) __hip_atomic_fetch_add(&pdone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        for (int spin = 0; spin < (1 << 20); ++spin) {
          const int n = __builtin_amdgcn_readfirstlane(
              __hip_atomic_load(&pdone, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
          if (n >= kNW * it) break;
          __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
        for (int u0 = 0; u0 < nU; u0 += VD) {
  #pragma unroll
          for (int d = 0; d < VD; ++d) {
            const int u = u0 + d;
            const int off = 32 * u;
            u32x4 pop = pbuf[min(u, nU - 1) * 64 + lane];
            if (u >= nU) pop = u32x4{0u, 0u, 0u, 0u};
            // value rows at positions >= ctx (unwritten cache) are zeroed: the
            // probabilities there are zero, but 0 * NaN would not be
            if (c0 + off + 32 > ctx) {   // uniform; only the context's last group
              const int nv = ctx - (c0 + off + 8 * grp);
  #pragma unroll
              for (int i = 0; i < RBW; ++i) vr[d][i] = keep_first(vr[d][i], nv);
            }
  #pragma unroll
            for (int i = 0; i < RBW; ++i) uacc[i] = mfma_bf16(vr[d][i], pop, uacc[i]);
            __builtin_amdgcn_sched_barrier(0);
            vload(vr[d], gu_lo + u + VD);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __syncthreads();
    }
    l_part = wave_sum_xor(l_part, 16);
    l_part = wave_sum_xor(l_part, 32);
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) ulds[j * a.r_v + 16 * rb[i] + 4 * grp + r] = j < G ? uacc[i][r] : 0.f;
    if (grp == 0) lpart[rw][j] = l_part;   // this consumer's share of the sums
    if (rw == 0 && grp == 0) mfin[j] = m_run;
  }
  // ---------------------------- finish ----------------------------
  __syncthreads();
  if (tid < 16) {
    float l = 0.f;
#pragma unroll
    for (int c = 0; c < kNW; ++c) l += lpart[c][tid];
    lfin[tid] = l;
  }
  __syncthreads();
  finish_item<D, kT>(a, dlds, nullptr, mfin, lfin, cmb_m, cmb_l, &last_flag, w, b, g, split);
}

// LDS of one workgroup on this device (160 KB on gfx950)
int lds_per_block() {
  static int bytes = 0;
  if (bytes == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeSharedMemPerBlockOptin, dev) == hipSuccess && v > 0)
      bytes = v;
    else
      bytes = 65536;
  }
  return bytes;
}

// Dynamic LDS plan: the resident factor (else the largest even number of
// rank steps that leaves a 256-position chunk and a 2-step tail area, the
// remaining steps being restaged per group), then the longest chunk the rest
// holds, at most the split length. Returns the dynamic bytes, 0 if the shape
// does not fit.
int plan_lds(AttnDecodeArgs &a, int dyn, int nb) {
  const int G = a.n_q / a.n_kv;
  const int step_bytes = nb * 1024;
  const int nrs = a.r_k / 32;
  const int per_pos = 4 * G + 32;
  const int pad = 16 * G + 16;   // four floats more per score row, rounding
  const int want = min(kMaxPitch, (a.split_len + kSlice - 1) / kSlice * kSlice);
  int rs_cap = nrs, rs_tail = 0;
  int pitch = ((dyn - pad - nrs * step_bytes) / per_pos) & ~(kSlice - 1);
  if (pitch < kSlice) {
    rs_tail = 2;
    pitch = min(want, 256);
    rs_cap = ((dyn - pad - pitch * per_pos - rs_tail * step_bytes) / step_bytes) & ~1;
    if (rs_cap < 2) {
      rs_cap = 2;
      pitch = ((dyn - pad - (rs_cap + rs_tail) * step_bytes) / per_pos) & ~(kSlice - 1);
    }
    rs_cap = min(rs_cap, nrs);
  }
  pitch = min(pitch, want);
  if (pitch < kSlice || rs_cap < 2 || (a.vpasses == 1 && 64 * a.r_v > dyn)) return 0;
  a.rs_cap = rs_cap;
  a.rs_tail = rs_tail;
  a.pitch = pitch;
  a.lds_bs = (rs_cap + rs_tail) * step_bytes;
  a.lds_s = G * (pitch + 4) * 4;
  return dyn;
}

template <int D, int RBW>
hipError_t launch_cfg(AttnDecodeArgs a, int grid, hipStream_t s) {
  const void *fn = reinterpret_cast<const void *>(&attn_decode_kernel<D, RBW>);
  static int dyn = -1;   // dynamic LDS of this instantiation (set up once)
  if (dyn < 0) {
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, fn);
    if (e != hipSuccess) return e;
    const int d = lds_per_block() - static_cast<int>(fa.sharedSizeBytes);
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, d);
    if (e != hipSuccess) return e;
    dyn = d;
  }
  if (plan_lds(a, dyn, Tile<D>::NB) == 0) return hipErrorInvalidValue;
  attn_decode_kernel<D, RBW><<<grid, kThreads, dyn, s>>>(a);
  return hipGetLastError();
}

// Warp-specialised kernel: the whole key factor in LDS and two score buffers
// of at least two chunk granules each. Default: 8 producers (groups of two
// 16-position blocks, a 4-step key ring, factor fragments read per step) and
// consumers with a 2-group value ring, 161 registers for three waves per SIMD;
// DL_ATTN_WS_PW=4 selects 4 producers (8-step key ring, double-buffered
// factor fragments, 4-group value ring), DL_ATTN_WS=0 the one-role kernel.
int env_or(const char *name, int dflt) {
  const char *v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}
template <int D, int NPA, int CD, int PW, int VD, int BD>
hipError_t launch_ws_cfg(AttnDecodeArgs a, int grid, hipStream_t s) {
  const void *fn = reinterpret_cast<const void *>(&attn_decode_ws_kernel<D, NPA, CD, PW, VD, BD>);
  static int dyn = -1;
  if (dyn < 0) {
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, fn);
    if (e != hipSuccess) return e;
    const int d = lds_per_block() - static_cast<int>(fa.sharedSizeBytes);
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, d);
    if (e != hipSuccess) return e;
    dyn = d;
  }
  const int G = a.n_q / a.n_kv;
  a.lds_bs = (a.r_k / 32) * Tile<D>::NB * 1024;
  // chunk granule: one group per producer, so every producer gets the same
  // number of whole groups (a chunk of 384 positions gave 8 producers one
  // full and one single-block group each: 310 against 288 us at 256), and at
  // least kWsGran (whole value-ring rounds)
  const int gran = max(kWsGran, 16 * NPA * PW);
  const int want = min(kMaxPitch, (a.split_len + gran - 1) / gran * gran);
  // two score buffers (4 G bytes per position, rows padded by 16 bytes) and
  // one probability buffer (32 bytes per position)
  int pitch = ((dyn - a.lds_bs - 2 * 16 * G) / (2 * 4 * G + 32)) / gran * gran;
  pitch = min(pitch, want);
  if (pitch < max(gran, 2 * kWsGran) || 64 * a.r_v > dyn) return hipErrorNotSupported;
  a.pitch = pitch;
  a.lds_s = 2 * G * (pitch + 4) * 4;
  a.rs_cap = a.r_k / 32;
  a.rs_tail = 0;
  a.vpasses = 1;
  attn_decode_ws_kernel<D, NPA, CD, PW, VD, BD><<<grid, 64 * (PW + kNW), dyn, s>>>(a);
  return hipGetLastError();
}
template <int D>
hipError_t launch_ws(const AttnDecodeArgs &a, int grid, hipStream_t s) {
  if (a.r_v / 16 > 8 * kNW || env_or("DL_ATTN_WS", 1) == 0) return hipErrorNotSupported;
  // producers: groups of two 16-position blocks and an 8-step key ring at
  // d = 128 (four blocks and a 4-step ring do not fit 256 registers), four
  // blocks at d = 64
  if (env_or("DL_ATTN_WS_PW", 8) == 8) return launch_ws_cfg<D, 2, 4, 8, 2, 1>(a, grid, s);
  const int npa = env_or("DL_ATTN_WS_NPA", D == 128 ? 2 : 4);
  if (npa == 2) return launch_ws_cfg<D, 2, 8, 4, 4, 2>(a, grid, s);
  return launch_ws_cfg<D, 4, 4, 4, 4, 2>(a, grid, s);
}

template <int D>
hipError_t launch_d(AttnDecodeArgs a, int grid, hipStream_t s) {
  const int nrb = a.r_v / 16;
  if (nrb <= 8 * kNW) {
    const hipError_t e = launch_ws<D>(a, grid, s);
    if (e != hipErrorNotSupported) return e;
    a.vpasses = 1;
    return launch_cfg<D, 8>(a, grid, s);
  }
  a.vpasses = attn_decode_value_passes(a.r_v);
  if (a.vpasses > 1 && !a.uglob) return hipErrorInvalidValue;
  return launch_cfg<D, 16>(a, grid, s);
}

}  // namespace

int attn_decode_split_granule() { return kSlice; }
int attn_decode_value_passes(int r_v) {
  const int nrb = r_v / 16;
  return nrb <= 8 * kNW ? 1 : (nrb + 16 * kNW - 1) / (16 * kNW);
}

hipError_t launch_attn_decode_bf16(const AttnDecodeArgs &a, hipStream_t s) {
  TraceGuard trace_guard(K_ATTN_DECODE, s);
  const int total = a.Bsz * a.n_kv * a.nsplit;
  const int grid = (total + 7) / 8 * 8;
  if (a.d == 128) return launch_d<128>(a, grid, s);
  return launch_d<64>(a, grid, s);
}

}  // namespace dl
