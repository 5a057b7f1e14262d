// Decode attention over the low-rank KV cache, bf16 MFMA (DeInfer section
// 4.2: rebuild K = C_k B_k and V = C_v B_v from the cached latents, rotate
// the rebuilt keys, attend). One query token per sequence.
//
// Work item = (sequence b, kv head g, context split). A workgroup of eight
// waves walks its split in iterations of 256 positions, 32 per wave:
//
//  * The up factors are read straight from their row-major [r, n_kv*d]
//    layout. Per pair of 32-rank steps 256 of the threads cooperatively load
//    B[32rs + 8grp + s][g*d + (d/2)hh + (d/32)c + 0..] (s = 0..7), transpose
//    each 8-row block in registers into MFMA operand fragments and store
//    them in LDS (double buffered); every wave then reads its operands with
//    one 16-byte ds_read each. Operand e of column group hh holds columns
//    d(blk, row) = (d/2)hh + (d/32)row + e, so the rotary partners d and
//    d + d/2 (hh = 0 and 1) land in the same lane and register.
//  * A wave rebuilds K^T for its 32 positions (accumulator column =
//    position), 2 MFMAs per operand fragment, rotates the pairs in
//    registers, feeds the accumulators straight into S^T = K Q^T (the
//    reduction slots of an operand may be any permutation shared by both
//    operands), updates an online softmax, rebuilds V for the same
//    positions and accumulates O^T += V^T P^T. Neither K nor V touches
//    memory.
//  * Rotary angles: the turn fraction pos * w_i / (2 pi) is split into a
//    per-iteration base reduced exactly in float64 and a small float32
//    offset, so float32 sin/cos see an argument in [-pi, pi] at any
//    position.
//  * The eight waves merge in LDS; splits are merged by the last workgroup
//    of each (b, g) to finish (device-coherent partials, one counter
//    atomic per workgroup), which writes the output row.
#include <math.h>

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

constexpr int kDecodeWaves = 8;
constexpr int kDecodeThreads = 64 * kDecodeWaves;

template <int D>
struct DecodeTile {
  static constexpr int CPL = D / 32;   // columns per lane per column group
  static constexpr int NE = CPL;       // operands per column group
  static constexpr int NB = 2 * NE;    // 16-wide d blocks
  static constexpr int HALF = D / 2;
  // dimension index of row `row` (0..15) of block blk
  __device__ static constexpr int dim(int blk, int row) {
    return HALF * (blk / NE) + CPL * row + (blk % NE);
  }
};

// Cooperative load of two 32-rank steps of an up factor for kv head g:
// thread t handles rows 32(2 round + t/128) + 8 grp + s, columns
// g*D + HALF*hh + CPL*c .. +CPL-1.
template <int D>
struct FactorStage {
  uint32_t w[8][D / 64];   // 8 rows x CPL bf16 columns
};

template <int D>
__device__ __forceinline__ void factor_load(FactorStage<D> &st, const uint16_t *B, int ldb, int g,
                                            int round, int tid) {
  using T = DecodeTile<D>;
  const int rsl = tid >> 7, grp = (tid >> 5) & 3, hh = (tid >> 4) & 1, c = tid & 15;
  const int row0 = 32 * (2 * round + rsl) + 8 * grp;
  const uint16_t *p = B + static_cast<size_t>(row0) * ldb + g * D + T::HALF * hh + T::CPL * c;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if constexpr (D == 128) {
      const u32x2 v = *reinterpret_cast<const u32x2 *>(p + static_cast<size_t>(s) * ldb);
      st.w[s][0] = v.x;
      st.w[s][1] = v.y;
    } else {
      st.w[s][0] = *reinterpret_cast<const uint32_t *>(p + static_cast<size_t>(s) * ldb);
    }
  }
}

// transpose to operand fragments and store: bs[rsl][blk][lane][8]
template <int D>
__device__ __forceinline__ void factor_store(const FactorStage<D> &st, uint16_t *bs, int tid) {
  using T = DecodeTile<D>;
  const int rsl = tid >> 7, grp = (tid >> 5) & 3, hh = (tid >> 4) & 1, c = tid & 15;
  const int lane = 16 * grp + c;
#pragma unroll
  for (int e = 0; e < T::NE; ++e) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = st.w[2 * q][e >> 1], hi = st.w[2 * q + 1][e >> 1];
      o[q] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    const int blk = T::NE * hh + e;
    *reinterpret_cast<u32x4 *>(bs + ((rsl * T::NB + blk) * 64 + lane) * 8) = o;
  }
}

template <int D>
__global__ __launch_bounds__(kDecodeThreads, 1) void attn_decode_kernel(AttnDecodeArgs a) {
  using T = DecodeTile<D>;
  constexpr int NB = T::NB, NE = T::NE, HALF = T::HALF;
  constexpr int PT = 32;         // positions per wave and iteration
  constexpr int NP = PT / 16;    // 16-position blocks per wave
  constexpr int NW = kDecodeWaves;
  constexpr int WT = NW * PT;    // positions per workgroup iteration
  constexpr int BS_ELEMS = 2 * 2 * NB * 64 * 8;  // [buf][rsl][blk][lane][8] bf16
  constexpr int MRG_FLOATS = NW * 16 * D;        // [wave][head][d] merge buffer
  __shared__ __attribute__((aligned(16))) float smem[MRG_FLOATS > BS_ELEMS / 2 ? MRG_FLOATS : BS_ELEMS / 2];
  uint16_t *bs = reinterpret_cast<uint16_t *>(smem);
  __shared__ __attribute__((aligned(16))) uint16_t qs[16 * D];
  __shared__ __attribute__((aligned(16))) u32x4 qfs[NB / 2][64];   // score operands, lane order
  __shared__ double rev64[HALF];
  __shared__ float rev32[HALF];
  __shared__ float mrg_m[NW][16], mrg_l[NW][16];
  __shared__ float cmb_m[16], cmb_l[16];
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
  const int ldb = a.n_kv * D;

  for (int i = tid; i < HALF; i += kDecodeThreads) {
    rev64[i] = rope_on ? rope_rev(i, D, a.theta) : 0.0;
    rev32[i] = static_cast<float>(rev64[i]);
  }
  __syncthreads();
  // rotated, scaled queries of this kv head's G heads; rows >= G are zero
  for (int idx = tid; idx < 16 * HALF; idx += kDecodeThreads) {
    const int hl = idx / HALF, i = idx % HALF;
    float x = 0.f, y = 0.f;
    if (hl < G) {
      const size_t off = (static_cast<size_t>(b) * a.n_q + g * G + hl) * D;
      if (a.q_f32) {
        x = static_cast<const float *>(a.q)[off + i];
        y = static_cast<const float *>(a.q)[off + i + HALF];
      } else {
        x = bf2f(static_cast<const uint16_t *>(a.q)[off + i]);
        y = bf2f(static_cast<const uint16_t *>(a.q)[off + i + HALF]);
      }
      if (rope_on) {
        float c, s;
        rope_cs(qpos, rev64[i], c, s);
        const float x2 = x * c - y * s;
        y = x * s + y * c;
        x = x2;
      }
    }
    qs[hl * D + i] = f2bf(x * a.scale_log2);
    qs[hl * D + i + HALF] = f2bf(y * a.scale_log2);
  }
  __syncthreads();
  // score B operand: lane (head j, grp) slots 0..3 = q[j][dim(2t, 4grp+r)],
  // slots 4..7 = q[j][dim(2t+1, 4grp+r)]
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < NB / 2; ++t) {
      uint16_t v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = qs[j * D + T::dim(2 * t, 4 * grp + r)];
        v[4 + r] = qs[j * D + T::dim(2 * t + 1, 4 * grp + r)];
      }
      u32x4 f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        f[q] = static_cast<uint32_t>(v[2 * q]) | (static_cast<uint32_t>(v[2 * q + 1]) << 16);
      qfs[t][lane] = f;
    }
  }
  __syncthreads();
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 accO[NB];
#pragma unroll
  for (int x = 0; x < NB; ++x) accO[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc[NB][NP];

  const size_t seq_row = static_cast<size_t>(b) * a.L_max;
  for (int T0 = p_begin; T0 < p_end; T0 += WT) {
    const int P0 = T0 + wave * PT;
    const bool active = P0 < p_end;
    const int last = p_end - 1;

    // ---------------- K^T[d, pos] = B_k^T C_k^T for the wave's positions ----------------
#pragma unroll
    for (int x = 0; x < NB; ++x)
#pragma unroll
      for (int pb = 0; pb < NP; ++pb) acc[x][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      // One round = two 32-rank steps. The factor fragments and the cache
      // rows of round r + 1 are loaded while round r computes; loads past
      // the last round repeat it (unconditional loads keep the wait counts
      // exact; the extra stage lands in the buffer nobody reads).
      const int nrounds = a.r_k / 64;
      const uint16_t *cbase = a.ck + seq_row * a.r_k + 8 * grp;
      int crow[NP];
#pragma unroll
      for (int pb = 0; pb < NP; ++pb) crow[pb] = min(P0 + 16 * pb + j, last) * a.r_k;
      auto load_rows = [&](u32x4 (&cf)[2][NP], int round) {
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
          for (int pb = 0; pb < NP; ++pb) cf[r2][pb] = ld16(cbase + crow[pb] + (2 * round + r2) * 32);
      };
      FactorStage<D> st;
      u32x4 cf[2][NP], cfn[2][NP];
      const bool loader = tid < 256;
      if (loader) factor_load<D>(st, a.bk, ldb, g, 0, tid);
      load_rows(cfn, 0);
      if (loader) factor_store<D>(st, bs, tid);
      __syncthreads();
      for (int round = 0; round < nrounds; ++round) {
        const int buf = round & 1;
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
          for (int pb = 0; pb < NP; ++pb) cf[r2][pb] = cfn[r2][pb];
        const int nxt = min(round + 1, nrounds - 1);
        if (loader) factor_load<D>(st, a.bk, ldb, g, nxt, tid);
        load_rows(cfn, nxt);
        if (active) {
#pragma unroll
          for (int r2 = 0; r2 < 2; ++r2) {
            const uint16_t *bsrc = bs + ((buf * 2 + r2) * NB * 64 + lane) * 8;
            // all operand fragments of the step in flight before the MFMAs
            u32x4 bop[NB];
#pragma unroll
            for (int x = 0; x < NB; ++x) bop[x] = *reinterpret_cast<const u32x4 *>(bsrc + x * 64 * 8);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = 0; x < NB; ++x)
#pragma unroll
              for (int pb = 0; pb < NP; ++pb) acc[x][pb] = mfma_bf16(bop[x], cf[r2][pb], acc[x][pb]);
          }
        }
        if (loader) factor_store<D>(st, bs + (buf ^ 1) * 2 * NB * 64 * 8, tid);
        __syncthreads();
      }
    }

    u32x4 pf[NP / 2];
    float alpha = 1.f;
    if (active) {
      // lane (pos j, grp) holds K^T[dim(x, 4grp + r)][P0 + 16pb + j]
      if (rope_on) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int e = 0; e < NE; ++e) {
            const int fi = T::CPL * (4 * grp + r) + e;
            double tb = static_cast<double>(P0) * rev64[fi];
            tb -= rint(tb);
            const float base = static_cast<float>(tb);
            const float rf = rev32[fi];
#pragma unroll
            for (int pb = 0; pb < NP; ++pb) {
              float c, s;
              turn_cs(base + static_cast<float>(16 * pb + j) * rf, c, s);
              const float x = acc[e][pb][r], y = acc[NE + e][pb][r];
              acc[e][pb][r] = x * c - y * s;
              acc[NE + e][pb][r] = x * s + y * c;
            }
          }
      }
      // S^T[pos, h]: lane (head j, grp) holds S^T[P0 + 16pb + 4grp + r][j]
      f32x4 sc[NP];
#pragma unroll
      for (int pb = 0; pb < NP; ++pb) {
        sc[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NB / 2; ++t)
          sc[pb] = mfma_bf16(pack_acc(acc[2 * t][pb], acc[2 * t + 1][pb]), qfs[t][lane], sc[pb]);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int pb = 0; pb < NP; ++pb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (P0 + 16 * pb + 4 * grp + r >= p_end) sc[pb][r] = -INFINITY;
          mx = fmaxf(mx, sc[pb][r]);
        }
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      const float m_new = fmaxf(m_run, mx);
      alpha = exp2f(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int pb = 0; pb < NP; ++pb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sc[pb][r] = exp2f(sc[pb][r] - m_new);
          psum += sc[pb][r];
        }
      psum = wave_sum_xor(psum, 16);
      psum = wave_sum_xor(psum, 32);
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int u = 0; u < NP / 2; ++u) pf[u] = pack_acc(sc[2 * u], sc[2 * u + 1]);
    }

    // ---------------- V[pos, d] = C_v B_v, same positions ----------------
#pragma unroll
    for (int x = 0; x < NB; ++x)
#pragma unroll
      for (int pb = 0; pb < NP; ++pb) acc[x][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      // One round = two 32-rank steps. The factor fragments and the cache
      // rows of round r + 1 are loaded while round r computes; loads past
      // the last round repeat it (unconditional loads keep the wait counts
      // exact; the extra stage lands in the buffer nobody reads).
      const int nrounds = a.r_v / 64;
      const uint16_t *cbase = a.cv + seq_row * a.r_v + 8 * grp;
      int crow[NP];
#pragma unroll
      for (int pb = 0; pb < NP; ++pb) crow[pb] = min(P0 + 16 * pb + j, last) * a.r_v;
      auto load_rows = [&](u32x4 (&cf)[2][NP], int round) {
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
          for (int pb = 0; pb < NP; ++pb) cf[r2][pb] = ld16(cbase + crow[pb] + (2 * round + r2) * 32);
      };
      FactorStage<D> st;
      u32x4 cf[2][NP], cfn[2][NP];
      const bool loader = tid < 256;
      if (loader) factor_load<D>(st, a.bv, ldb, g, 0, tid);
      load_rows(cfn, 0);
      if (loader) factor_store<D>(st, bs, tid);
      __syncthreads();
      for (int round = 0; round < nrounds; ++round) {
        const int buf = round & 1;
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
          for (int pb = 0; pb < NP; ++pb) cf[r2][pb] = cfn[r2][pb];
        const int nxt = min(round + 1, nrounds - 1);
        if (loader) factor_load<D>(st, a.bv, ldb, g, nxt, tid);
        load_rows(cfn, nxt);
        if (active) {
#pragma unroll
          for (int r2 = 0; r2 < 2; ++r2) {
            const uint16_t *bsrc = bs + ((buf * 2 + r2) * NB * 64 + lane) * 8;
            // all operand fragments of the step in flight before the MFMAs
            u32x4 bop[NB];
#pragma unroll
            for (int x = 0; x < NB; ++x) bop[x] = *reinterpret_cast<const u32x4 *>(bsrc + x * 64 * 8);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = 0; x < NB; ++x)
#pragma unroll
              for (int pb = 0; pb < NP; ++pb) acc[x][pb] = mfma_bf16(cf[r2][pb], bop[x], acc[x][pb]);
          }
        }
        if (loader) factor_store<D>(st, bs + (buf ^ 1) * 2 * NB * 64 * 8, tid);
        __syncthreads();
      }
    }
    if (active) {
      // lane (column j, grp) holds V[P0 + 16pb + 4grp + r][dim(x, j)]
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        accO[x] *= alpha;
#pragma unroll
        for (int u = 0; u < NP / 2; ++u)
          accO[x] = mfma_bf16(pack_acc(acc[x][2 * u], acc[x][2 * u + 1]), pf[u], accO[x]);
      }
    }
  }

  // ---------------- merge the waves (LDS, aliasing the factor stage) ----------------
  float *mrg_o = smem;   // [NW][16][D]
  if (grp == 0) {
    mrg_m[wave][j] = m_run;
    mrg_l[wave][j] = l_run;
  }
  // lane (head j, grp) holds O^T[dim(x, 4grp + r)][j]
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int r = 0; r < 4; ++r) mrg_o[(wave * 16 + j) * D + T::dim(x, 4 * grp + r)] = accO[x][r];
  __syncthreads();
  const int D2 = D + 2;
  float *part = a.part + ((static_cast<size_t>(b) * a.n_q + g * G) * a.nsplit) * D2;
  for (int idx = tid; idx < G * D; idx += kDecodeThreads) {
    const int h = idx / D, dd = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) M = fmaxf(M, mrg_m[wv][h]);
    float o = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) {
        const float sc = exp2f(mrg_m[wv][h] - M);
        o += sc * mrg_o[(wv * 16 + h) * D + dd];
        L += sc * mrg_l[wv][h];
      }
    }
    if (a.nsplit == 1) {
      const size_t oi = (static_cast<size_t>(b) * a.n_q + g * G + h) * D + dd;
      if (a.out_f32)
        static_cast<float *>(a.out)[oi] = o / L;
      else
        static_cast<uint16_t *>(a.out)[oi] = f2bf(o / L);
    } else {
      float *dst = part + (static_cast<size_t>(h) * a.nsplit + split) * D2;
      store_coherent(dst + dd, o);
      if (dd == 0) {
        store_coherent(dst + D, M);
        store_coherent(dst + D + 1, L);
      }
    }
  }
  if (a.nsplit == 1) return;

  // ---------------- last workgroup of (b, g) merges the splits ----------------
  wait_memory();
  __syncthreads();
  int *counter = a.counters + b * a.n_kv + g;
  if (tid == 0)
    last_flag = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                a.nsplit - 1;
  __syncthreads();
  if (!last_flag) return;
  // split statistics -> LDS (reuse mrg_o space): sm[h][s], sl[h][s]
  float *sm = mrg_o, *sl = mrg_o + 16 * a.nsplit;
  for (int idx = tid; idx < G * a.nsplit; idx += kDecodeThreads) {
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
  for (int idx = tid; idx < G * D; idx += kDecodeThreads) {
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
    const size_t oi = (static_cast<size_t>(b) * a.n_q + g * G + h) * D + dd;
    if (a.out_f32)
      static_cast<float *>(a.out)[oi] = o / cmb_l[h];
    else
      static_cast<uint16_t *>(a.out)[oi] = f2bf(o / cmb_l[h]);
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

int attn_decode_positions_per_tile() { return 32 * kDecodeWaves; }
int attn_decode_split_granule() { return 32; }

hipError_t launch_attn_decode_bf16(const AttnDecodeArgs &a, hipStream_t s) {
  TraceGuard trace_guard(K_ATTN_DECODE, s);
  const int total = a.Bsz * a.n_kv * a.nsplit;
  const int grid = (total + 7) / 8 * 8;
  if (a.d == 128)
    attn_decode_kernel<128><<<grid, kDecodeThreads, 0, s>>>(a);
  else
    attn_decode_kernel<64><<<grid, kDecodeThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dl
