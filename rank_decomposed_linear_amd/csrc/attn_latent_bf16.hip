// Decode attention in the latent space, bf16 MFMA, for layers without the
// rotary embedding (DeInfer section 4.2 rebuilds K = C_k B_k and V = C_v B_v
// and rotates the rebuilt keys; Table 2 lists rotary embedding as optional).
// Without the rotation both up factors can be moved to the query / output
// side by associativity (only the rounding order changes):
//   s_h(pos) = q_h . (C_k B_k,g)(pos) = (B_k,g q_h) . C_k(pos)
//   o_h      = P_h (C_v B_v,g)      = (P_h C_v) B_v,g
// with g the kv head of query head h. The latents are shared by every head,
// so attention reads each cached row once per group of 16 query heads and
// never rebuilds K or V: per position 2 * 16 * (r_k + r_v) flops against
// (r_k + r_v) * 2 bytes, an HBM-bound pass.
//
// Three launches:
//   qabs  Q~[b][h][r] = scale * log2(e) * sum_i q[b][h][i] B_k^T[g d + i][r].
//         Workgroup = (kv head g, 64 ranks); the B_k^T slice is copied into
//         LDS transposed (ranks x dims), so the reduction over dims reads one
//         16-byte operand per lane; rows are (sequence, head) pairs.
//   attn  Workgroup = (sequence b, group of 16 query heads, context split),
//         four waves; Q~ of the group in LDS as a [16, r_k] operand-tiled
//         matrix. The split is walked in one pass:
//           scores: S^T[pos][h] = C_k[pos] . Q~[h] (A = key-cache tile of 16
//             positions, B = Q~ fragment), 64 positions per wave at a time,
//             key tiles eight rank steps ahead;
//           softmax over the split (all scores in LDS), probabilities in
//             bf16 operand order;
//           values: U^T[r][h] = sum_pos C_v^T[r][pos] P^T[pos][h], each wave
//             owning 16-rank blocks of U, eight at a time, value tiles four
//             32-position blocks ahead.
//         One split: U / l goes out as bf16; several: f32 partials (U, max,
//         sum) merged by the last workgroup of (b, group).
//   bv    o[b][h][:] = U[b][h][:] B_v,g: workgroup = (query head, 16
//         sequences); A = U rows, B = B_v^T tiles as stored (rows = dims).
#include <math.h>

#include <algorithm>

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

// zero the bf16 elements e >= nv of an 8-element operand
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int nv) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t m = (2 * q < nv ? 0x0000ffffu : 0u) | (2 * q + 1 < nv ? 0xffff0000u : 0u);
    v[q] &= m;
  }
  return v;
}

// eight consecutive query values of row (b, h) as one bf16 operand
__device__ __forceinline__ u32x4 q_operand(const void *q, int q_f32, size_t off) {
  if (q_f32) {
    const f32x4 lo = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(q) + off);
    const f32x4 hi = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(q) + off + 4);
    return u32x4{pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]), pack2(hi[2], hi[3])};
  }
  return ld16(static_cast<const uint16_t *>(q) + off);
}

constexpr int kNW = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kNW;
constexpr int kHG = 16;                // query heads per attention workgroup
constexpr int kQRanks = 64;            // ranks per qabs workgroup
constexpr int kNP = 4;                 // 16-position blocks per wave group
constexpr int kCDepth = 8;             // key-tile prefetch depth (rank steps)
constexpr int kRB = 8;                 // value rank blocks per wave pass
constexpr int kVDepth = 4;             // value prefetch depth (32-position blocks)
constexpr int kPerPos = 4 * kHG + 2 * kHG;   // LDS bytes per position: scores f32, probabilities bf16

// ---------------------------------------------------------------------------
// qabs
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void latent_query_kernel(LatentAttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t bt[kQRanks][D + 8];   // [rank][dim], padded rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrc = a.r_k / kQRanks;
  const int g = blockIdx.x / nrc, rc = blockIdx.x % nrc;
  const int G = a.n_q / a.n_kv;
  // B_k^T[g d + i][64 rc + c] -> bt[c][i]: each unit is 8 consecutive ranks of one dim
  for (int u = tid; u < D * kQRanks / 8; u += kThreads) {
    const int i = u / (kQRanks / 8), c8 = u % (kQRanks / 8);
    const u32x4 v = ld16(a.bk + tile_off(g * D + i, kQRanks * rc + 8 * c8, a.r_k));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bt[8 * c8 + 2 * e][i] = static_cast<uint16_t>(v[e] & 0xffffu);
      bt[8 * c8 + 2 * e + 1][i] = static_cast<uint16_t>(v[e] >> 16);
    }
  }
  __syncthreads();
  const int j = lane & 15, grp = lane >> 4;
  const int nbt = (a.Bsz + 15) / 16;
  // row tiles (head of the group jh, 16 sequences from b0), dealt to the waves
  for (int t = wave; t < G * nbt; t += kNW) {
    const int jh = t / nbt, b0 = 16 * (t % nbt);
    const int h = g * G + jh;
    const int bq = min(b0 + j, a.Bsz - 1);
    f32x4 acc[kQRanks / 16];
#pragma unroll
    for (int nb = 0; nb < kQRanks / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      u32x4 aop = q_operand(a.q, a.q_f32, (static_cast<size_t>(bq) * a.n_q + h) * D + 32 * ks + 8 * grp);
      if (b0 + j >= a.Bsz) aop = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int nb = 0; nb < kQRanks / 16; ++nb) {
        const u32x4 bop = *reinterpret_cast<const u32x4 *>(&bt[16 * nb + j][32 * ks + 8 * grp]);
        acc[nb] = mfma_bf16(aop, bop, acc[nb]);
      }
    }
    // lane (rank j, grp) holds Q~[b0 + 4grp + r][64 rc + 16 nb + j]
    const int hg = h / kHG, hl = h % kHG;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int b = b0 + 4 * grp + r;
      if (b >= a.Bsz) continue;
      uint16_t *dst = a.qt + (static_cast<size_t>(b) * a.ngroups + hg) * kHG * a.r_k;
#pragma unroll
      for (int nb = 0; nb < kQRanks / 16; ++nb)
        dst[tile_off(hl, kQRanks * rc + 16 * nb + j, a.r_k)] = f2bf(acc[nb][r] * a.scale_log2);
    }
  }
}

// ---------------------------------------------------------------------------
// attention over the latents
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads, 1) void latent_attn_kernel(LatentAttnArgs a) {
  // dynamic LDS: Q~ [16, r_k] operand tiles, scores [16][pitch + 4] f32,
  // probabilities [pitch / 32][64] operand words
  extern __shared__ __attribute__((aligned(16))) char dlds[];
  uint16_t *qs = reinterpret_cast<uint16_t *>(dlds);
  float *sS = reinterpret_cast<float *>(dlds + a.lds_q);
  // score row stride four floats longer than the split, so the 16 heads'
  // rows (read and written at one column by lanes j = head) start in
  // different LDS banks and stay 16-byte aligned
  const int spitch = a.pitch + 4;
  u32x4 *pbuf = reinterpret_cast<u32x4 *>(dlds + a.lds_q + a.lds_s);
  __shared__ float smax[kNW][16], psw[kNW][16];
  __shared__ float cmb_m[16], cmb_l[16];
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, grp = lane >> 4;
  const int total = a.Bsz * a.ngroups * a.nsplit;
  // consecutive work items (the head groups and splits of one sequence,
  // which read the same cache rows) share an XCD
  const int per = gridDim.x >> 3;
  const int w = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (w >= total) return;
  const int split = w % a.nsplit;
  const int hg = (w / a.nsplit) % a.ngroups;
  const int b = w / (a.nsplit * a.ngroups);
  const int ctx = a.ctx_lens[b] + a.ctx_offset;
  const int p_begin = split * a.split_len;
  const int p_end = min(p_begin + a.split_len, ctx);
  const int nrs = a.r_k / 32, nrb = a.r_v / 16;
  const int heads_here = min(kHG, a.n_q - kHG * hg);
  auto page_of = [&](int p64) {
    return cache_page_uniform(a.block_table, a.page_stride, b, p64);
  };

  // Q~ of the group into LDS (rows of heads past n_q are zero)
  {
    const uint16_t *src = a.qt + (static_cast<size_t>(b) * a.ngroups + hg) * kHG * a.r_k;
    for (int u = tid; u < kHG * a.r_k / 8; u += kThreads) {
      // unit u = lane (u % 64) of fragment u / 64; its row is (u % 64) % 16
      u32x4 v = ld16(src + static_cast<size_t>(u) * 8);
      if ((u & 15) >= heads_here) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4 *>(qs + static_cast<size_t>(u) * 8) = v;
    }
  }
  __syncthreads();

  // ------------------------------ scores ------------------------------
  const int npos = max(p_end - p_begin, 0);
  const int nblk = (npos + 15) >> 4;
  const int share = (nblk + kNW - 1) / kNW;
  const int b_lo = min(wave * share, nblk), b_hi = min(b_lo + share, nblk);
  float mx = -INFINITY;
  for (int g0 = b_lo; g0 < b_hi; g0 += kNP) {
    const int np = min(kNP, b_hi - g0);
    const uint16_t *kblk[kNP];
#pragma unroll
    for (int pb = 0; pb < kNP; ++pb) {
      const int kb = (p_begin >> 4) + g0 + min(pb, np - 1);
      kblk[pb] = a.ck + static_cast<size_t>(page_of(kb >> 2)) * (kPage * a.r_k) +
                 frag_off(kb & 3, 0, a.r_k, lane);
    }
    f32x4 acc[kNP];
#pragma unroll
    for (int pb = 0; pb < kNP; ++pb) acc[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 cf[kCDepth][kNP];
#pragma unroll
    for (int d = 0; d < kCDepth; ++d)
#pragma unroll
      for (int pb = 0; pb < kNP; ++pb) cf[d][pb] = ld16(kblk[pb] + 512 * min(d, nrs - 1));
    auto step = [&](auto dc, int s) {
      constexpr int d = decltype(dc)::value;
      const u32x4 bop = *reinterpret_cast<const u32x4 *>(qs + (static_cast<size_t>(s) * 64 + lane) * 8);
#pragma unroll
      for (int pb = 0; pb < kNP; ++pb) acc[pb] = mfma_bf16(cf[d][pb], bop, acc[pb]);
      const int sn = min(s + kCDepth, nrs - 1);
#pragma unroll
      for (int pb = 0; pb < kNP; ++pb) cf[d][pb] = ld16(kblk[pb] + 512 * sn);
    };
    int s0 = 0;
    for (; s0 + kCDepth <= nrs; s0 += kCDepth)
      static_for<kCDepth>([&](auto dc) { step(dc, s0 + decltype(dc)::value); });
    static_for<kCDepth>([&](auto dc) {
      if (s0 + decltype(dc)::value < nrs) step(dc, s0 + decltype(dc)::value);
    });
    // lane (head j, grp) holds S^T[pos 16 pb + 4grp + r][head j]
#pragma unroll
    for (int pb = 0; pb < kNP; ++pb) {
      if (pb >= np) break;   // uniform
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int off = 16 * (g0 + pb) + 4 * grp + r;
        const float v = p_begin + off < p_end ? acc[pb][r] : -INFINITY;
        mx = fmaxf(mx, v);
        sS[j * spitch + off] = v;
      }
    }
  }
  mx = wave_max_xor(mx, 16);
  mx = wave_max_xor(mx, 32);
  if (grp == 0) smax[wave][j] = mx;
  __syncthreads();

  // ------------------------------ softmax ------------------------------
  float m_all = -INFINITY;
#pragma unroll
  for (int wv = 0; wv < kNW; ++wv) m_all = fmaxf(m_all, smax[wv][j]);
  const int nU = (npos + 31) >> 5;
  float ps = 0.f;
  for (int u = wave; u < nU; u += kNW) {
    // eight scores read unconditionally (two 16-byte reads); masked
    // entries become exp2(-inf) = 0 by a select, so the lanes do not branch
    // around each read and wait on it separately
    const int off = 32 * u + 8 * grp;
    const float *srow = sS + j * spitch + off;
    const f32x4 sa = *reinterpret_cast<const f32x4 *>(srow);
    const f32x4 sb = *reinterpret_cast<const f32x4 *>(srow + 4);
    const float sv[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = exp2_hw(off + e < npos && m_all != -INFINITY ? sv[e] - m_all : -INFINITY);
      ps += v[e];
    }
    pbuf[u * 64 + lane] = u32x4{pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
  }
  ps = wave_sum_xor(ps, 16);
  ps = wave_sum_xor(ps, 32);
  if (grp == 0) psw[wave][j] = ps;
  __syncthreads();
  float l_all = 0.f;
#pragma unroll
  for (int wv = 0; wv < kNW; ++wv) l_all += psw[wv][j];

  // ------------------------------ values ------------------------------
  // U^T[16 rb + 4grp + r][head j] for this wave's rank blocks rb = wave +
  // 4 i, kRB at a time (duplicates of the last block are computed and not
  // stored, so every load stays unconditional)
  const int D2 = a.r_v + 2;
  float *part = a.part + ((static_cast<size_t>(b) * a.ngroups + hg) * a.nsplit + split) * kHG * D2;
  // (an empty split, past the sequence's end, has no value rows to read:
  // its partial is U = 0, max = -inf, sum = 0)
  for (int i0 = 0; wave + kNW * i0 < nrb; i0 += kRB) {
    int rb[kRB];
#pragma unroll
    for (int i = 0; i < kRB; ++i) rb[i] = min(wave + kNW * (i0 + i), nrb - 1);
    f32x4 uacc[kRB];
#pragma unroll
    for (int i = 0; i < kRB; ++i) uacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto vload = [&](u32x4 (&dst)[kRB], int u) {
      const int p = p_begin + 32 * u;
      const uint16_t *vb = a.cv + static_cast<size_t>(page_of(p >> 6)) * (kPage * a.r_v) +
                           ((p >> 5) & 1) * 512 + lane * 8;
#pragma unroll
      for (int i = 0; i < kRB; ++i) dst[i] = ld16(vb + rb[i] * 1024);
    };
    u32x4 vr[kVDepth][kRB];
    if (nU > 0) {
#pragma unroll
      for (int d = 0; d < kVDepth; ++d) vload(vr[d], min(d, nU - 1));
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
        const int p = p_begin + 32 * u;
        if (p + 32 > ctx) {
          const int nv = ctx - (p + 8 * grp);
#pragma unroll
          for (int i = 0; i < kRB; ++i) vr[d][i] = keep_first(vr[d][i], nv);
        }
#pragma unroll
        for (int i = 0; i < kRB; ++i) uacc[i] = mfma_bf16(vr[d][i], pop, uacc[i]);
        __builtin_amdgcn_sched_barrier(0);
        vload(vr[d], min(u0 + d + kVDepth, nU - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // lane (head j, grp) holds U^T[16 rb + 4grp + r][j]
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
      if (wave + kNW * (i0 + i) >= nrb || j >= heads_here) continue;
      const int r0 = 16 * rb[i] + 4 * grp;
      if (a.nsplit == 1) {
        const float il = l_all > 0.f ? 1.f / l_all : 0.f;
        *reinterpret_cast<u32x2 *>(a.u + (static_cast<size_t>(b) * a.n_q + kHG * hg + j) * a.r_v + r0) =
            u32x2{pack2(uacc[i][0] * il, uacc[i][1] * il), pack2(uacc[i][2] * il, uacc[i][3] * il)};
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) store_coherent(part + j * D2 + r0 + r, uacc[i][r]);
      }
    }
  }
  if (a.nsplit == 1) return;
  if (wave == 0 && grp == 0 && j < heads_here) {
    store_coherent(part + j * D2 + a.r_v, m_all);
    store_coherent(part + j * D2 + a.r_v + 1, l_all);
  }

  // ---------------- last workgroup of (b, group) merges the splits ----------------
  wait_memory();
  __syncthreads();
  int *counter = a.counters + b * a.ngroups + hg;
  if (tid == 0)
    last_flag = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                a.nsplit - 1;
  __syncthreads();
  if (!last_flag) return;
  const float *p0 = a.part + (static_cast<size_t>(b) * a.ngroups + hg) * a.nsplit * kHG * D2;
  if (tid < heads_here) {
    float M = -INFINITY;
    for (int sp = 0; sp < a.nsplit; ++sp) M = fmaxf(M, load_coherent(p0 + (sp * kHG + tid) * D2 + a.r_v));
    float L = 0.f;
    for (int sp = 0; sp < a.nsplit; ++sp) {
      const float m = load_coherent(p0 + (sp * kHG + tid) * D2 + a.r_v);
      if (m != -INFINITY) L += exp2f(m - M) * load_coherent(p0 + (sp * kHG + tid) * D2 + a.r_v + 1);
    }
    cmb_m[tid] = M;
    cmb_l[tid] = L;
  }
  __syncthreads();
  for (int idx = tid; idx < heads_here * a.r_v; idx += kThreads) {
    const int h = idx / a.r_v, r = idx % a.r_v;
    const float M = cmb_m[h];
    float o = 0.f;
    for (int sp = 0; sp < a.nsplit; ++sp) {
      const float m = load_coherent(p0 + (sp * kHG + h) * D2 + a.r_v);
      if (m != -INFINITY) o += exp2f(m - M) * load_coherent(p0 + (sp * kHG + h) * D2 + r);
    }
    a.u[(static_cast<size_t>(b) * a.n_q + kHG * hg + h) * a.r_v + r] = f2bf(cmb_l[h] > 0.f ? o / cmb_l[h] : 0.f);
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// bv: o = U B_v per query head
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void latent_out_kernel(LatentAttnArgs a) {
  constexpr int NB = D / 16;           // 16-dim output blocks
  constexpr int OBW = NB / kNW;        // per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int nbt = (a.Bsz + 15) / 16;
  const int h = blockIdx.x / nbt, b0 = 16 * (blockIdx.x % nbt);
  const int g = h / (a.n_q / a.n_kv);
  const int bq = min(b0 + j, a.Bsz - 1);
  f32x4 acc[OBW];
#pragma unroll
  for (int x = 0; x < OBW; ++x) acc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t *urow = a.u + (static_cast<size_t>(bq) * a.n_q + h) * a.r_v + 8 * grp;
  const int nks = a.r_v / 32;
  for (int ks = 0; ks < nks; ks += 2) {   // r_v / 32 is even
    u32x4 aop[2], bop[2][OBW];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      aop[q] = ld16(urow + 32 * (ks + q));
#pragma unroll
      for (int x = 0; x < OBW; ++x) bop[q][x] = ld16(a.bv + frag_off(g * NB + OBW * wave + x, ks + q, a.r_v, lane));
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int x = 0; x < OBW; ++x) acc[x] = mfma_bf16(aop[q], bop[q][x], acc[x]);
  }
  // lane (dim j, grp) holds o[b0 + 4grp + r][h][16 (OBW wave + x) + j]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int b = b0 + 4 * grp + r;
    if (b >= a.Bsz) continue;
#pragma unroll
    for (int x = 0; x < OBW; ++x) {
      const int col = h * D + 16 * (OBW * wave + x) + j;
      const size_t oi = a.out_tiled ? tile_off(b, col, a.n_q * D) : static_cast<size_t>(b) * a.n_q * D + col;
      if (a.out_f32)
        static_cast<float *>(a.out)[oi] = acc[x][r];
      else
        static_cast<uint16_t *>(a.out)[oi] = f2bf(acc[x][r]);
    }
  }
}

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

int attn_static_lds() {
  static int bytes = -1;
  if (bytes < 0) {
    hipFuncAttributes fa;
    bytes = hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(&latent_attn_kernel)) == hipSuccess
                ? static_cast<int>(fa.sharedSizeBytes)
                : 4096;
  }
  return bytes;
}

}  // namespace

int latent_attn_max_split(int r_k) {
  const int dyn = lds_per_block() - attn_static_lds() - kHG * r_k * 2;
  const int pitch = ((dyn - kHG * 16) / kPerPos) & ~63;
  return pitch < 64 ? 0 : std::min(pitch, 4096);
}

hipError_t launch_latent_attn_bf16(LatentAttnArgs a, hipStream_t s) {
  if (a.d != 64 && a.d != 128) return hipErrorInvalidValue;
  TraceGuard trace_guard(K_ATTN_LATENT, s);
  // Q~
  {
    const int grid = a.n_kv * (a.r_k / kQRanks);
    if (a.d == 128)
      latent_query_kernel<128><<<grid, kThreads, 0, s>>>(a);
    else
      latent_query_kernel<64><<<grid, kThreads, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // attention
  {
    const void *fn = reinterpret_cast<const void *>(&latent_attn_kernel);
    static int dyn_set = -1;
    const int dyn = lds_per_block() - attn_static_lds();
    if (dyn_set != dyn) {
      hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
      if (e != hipSuccess) return e;
      dyn_set = dyn;
    }
    a.pitch = (a.split_len + 63) / 64 * 64;
    a.lds_q = kHG * a.r_k * 2;
    a.lds_s = kHG * (a.pitch + 4) * 4;
    const int need = a.lds_q + a.lds_s + a.pitch * 32;
    if (need > dyn) return hipErrorInvalidValue;
    const int total = a.Bsz * a.ngroups * a.nsplit;
    const int grid = (total + 7) / 8 * 8;
    latent_attn_kernel<<<grid, kThreads, need, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // o = U B_v
  {
    const int grid = a.n_q * ((a.Bsz + 15) / 16);
    if (a.d == 128)
      latent_out_kernel<128><<<grid, kThreads, 0, s>>>(a);
    else
      latent_out_kernel<64><<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
  }
}

}  // namespace dl
