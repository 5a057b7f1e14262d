// Attention over the low-rank KV cache, bf16 MFMA (DeInfer section 4.2:
// rebuild K = C_k B_k and V = C_v B_v from the cached latents, rotate the
// rebuilt keys, attend).
//
// The rebuilt K and V never leave the chip in decode; in prefill each
// 64-key tile is rebuilt once into a workspace image that all query tiles
// of its (sequence, kv head) then read. Caches and factors are stored
// in 16 x 32 operand tiles (MFMA lane order): a key block of 16 positions x
// 32 ranks and an up-factor fragment are each one contiguous 1 KB read; the
// caches are held in pages of 64 positions (a key page [64, r_k], a value
// page rank-major [r_v, 64]) reached through the sequence's block table or
// contiguously, and a 64-key tile is exactly one page. The rebuilt tiles
// live in MFMA accumulators:
//
//  prefill  A rebuild workgroup turns one 64-key tile of latents into its
//           image: K (rotated) and V^T, swizzled, from latents and factor
//           slices staged in LDS. An attention workgroup owns one kv head
//           and up to 256 (token, head) query rows; per key tile it loads
//           the image into LDS and each wave runs an online-softmax pass
//           for its 32 query rows, its query fragments in registers and
//           each K / V fragment read once for both of its 16-row blocks.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace dl {

namespace {

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// raw buffer resource over `bytes` bytes at p (loads past the end read zero)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0), bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}


// ---------------------------------------------------------------------------
// Prefill
//
// Work item: (sequence b, kv head g, query tile of QT tokens x G heads = 256
// rows). Per 64-key tile the latents are consumed in chunks of 64 ranks:
// all 512 threads stage the chunk's key latents, value latents and the head's
// B_k / B_v slices into LDS with contiguous 16-byte loads, issued one chunk
// ahead into registers. The value latents arrive rank-major and are
// transposed to key-major operand tiles as they are written, so both
// rebuilds reduce over ranks with one ds_read_b128 per operand. Waves 0-3
// rebuild K^T for d-block pairs (x, x + D/32), the rotary partners, waves
// 4-7 rebuild V for pairs of adjacent d blocks; each factor fragment is read
// from LDS once per tile for all its key blocks. After the last chunk the K
// waves rotate and write K, the V waves write V^T, and all eight waves run
// the online-softmax pass for their 32 query rows.
// ---------------------------------------------------------------------------
template <int DB>
__global__ __launch_bounds__(512) void attn_rebuild_kernel(AttnPrefillArgs a) {
  constexpr int D = DB * 16, HALF = DB / 2, KT = 64;
  constexpr int CH = D / 8;       // 16-byte chunks per K row
  constexpr int RS = 2;           // 32-rank steps per chunk
  constexpr int NP = HALF;        // d-block pairs per side
  constexpr int NKB = NP;         // key blocks per wave: 4 waves per side = NP pairs x 4 / NP
  constexpr int U_CK = 4 * RS * 64, U_CV = 4 * RS * 64;  // u32x4 units (64 per 1 KB fragment)
  constexpr int U_BK = DB * RS * 64, U_BV = DB * RS * 64;
  constexpr int O_CV = U_CK, O_BK = U_CK + U_CV, O_BV = O_BK + U_BK;
  constexpr int NU = (O_BV + U_BV) / 512;  // staging units per thread
  constexpr int I_CV = U_CK / 512, I_BK = O_BK / 512, I_BV = O_BV / 512;
  __shared__ u32x4 cs[O_BV + U_BV];
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * KT];
  __shared__ double revs[D / 2];

  // wave is made provably uniform, so every fragment index derived from it
  // stays scalar and each load is a scalar base plus the lane's 16 bytes
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, grp = lane >> 4;
  const int ktile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int past = a.past_lens[b];
  // every key up to the last query position is rebuilt (later tiles are
  // never read)
  const int qmax_pos = past + a.T - 1;
  if (ktile * KT > qmax_pos) return;
  const bool rope_on = a.theta != 0.f;
  for (int i = tid; i < D / 2; i += 512) revs[i] = rope_on ? rope_rev(i, D, a.theta) : 0.0;
  const int rsk = a.r_k / 32, rsv = a.r_v / 32;
  const int nchunk = max((rsk + RS - 1) / RS, (rsv + RS - 1) / RS);

  // ---- staging: unit i of this thread is u = tid + 512 i, fragment
  // (u - group start) / 64, lane `lane`. Keys past the last query position
  // stage zeros (their V rows must not leak NaN into P V). ----
  // Buffer loads: one scalar resource per array (the cache resources span the
  // page pools, whose byte size the launcher bounds below 2^31), the lane's
  // 16 bytes as the only vector offset, the (wave-uniform) fragment offset as
  // soffset. A 64-key tile is one cache page; tiles start at or before the
  // last query position, so their page is always one the sequence owns.
  const __amdgpu_buffer_rsrc_t rck = make_rsrc(a.ck, static_cast<int>(a.pool_pages * kPage * a.r_k * 2));
  const __amdgpu_buffer_rsrc_t rcv = make_rsrc(a.cv, static_cast<int>(a.pool_pages * kPage * a.r_v * 2));
  const __amdgpu_buffer_rsrc_t rbk = make_rsrc(a.bk, a.n_kv * D * a.r_k * 2);
  const __amdgpu_buffer_rsrc_t rbv = make_rsrc(a.bv, a.n_kv * D * a.r_v * 2);
  const int lane16 = lane * 16;
  u32x4 st[NU];
  auto gload = [&](int kt, int c) {
    const int k0 = kt * KT, r0 = c * RS;
    const int nrk = rsk - r0, nrv = rsv - r0;
    const int pg = cache_page_uniform(a.block_table, a.page_stride, b, kt);
    const int kpage = pg * (kPage * a.r_k), vpage = pg * (kPage * a.r_v);   // element offsets
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      if (i < I_CV) {
        const int f = wave + 8 * i, kb = f / RS, rs = f % RS;
        const bool ok = rs < nrk && k0 + 16 * kb + j <= qmax_pos;
        const int so = 2 * (kpage + static_cast<int>(frag_off(kb, r0 + rs, a.r_k, 0)));
        st[i] = ok ? bload(rck, lane16, so) : z;
      } else if (i < I_BK) {
        const int f = wave + 8 * (i - I_CV), rb = f >> 1, ps = f & 1;
        const int so = 2 * (vpage + static_cast<int>(frag_off(2 * r0 + rb, ps, kPage, 0)));
        st[i] = rb < 2 * nrv ? bload(rcv, lane16, so) : z;
      } else if (i < I_BV) {
        const int f = wave + 8 * (i - I_BK), db = f / RS, rs = f % RS;
        const int so = 2 * static_cast<int>(frag_off(g * DB + db, r0 + rs, a.r_k, 0));
        st[i] = rs < nrk ? bload(rbk, lane16, so) : z;
      } else {
        const int f = wave + 8 * (i - I_BV), db = f / RS, rs = f % RS;
        const int so = 2 * static_cast<int>(frag_off(g * DB + db, r0 + rs, a.r_v, 0));
        st[i] = rs < nrv ? bload(rbv, lane16, so) : z;
      }
    }
  };
  auto swrite = [&](int kt) {
    const int k0 = kt * KT;
    uint16_t *cv16 = reinterpret_cast<uint16_t *>(cs + O_CV);
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      if (i >= I_CV && i < I_BK) {
        // value tile (rank rho, positions p .. p + 7) -> key-major tiles:
        // key p + e, rank rho at tile (key / 16, rho / 32), lane
        // key % 16 + 16 ((rho % 32) / 8), slot rho % 8
        // p % 16 is 0 or 8, so keys p .. p + 7 share a key block and sit
        // in consecutive lanes of the destination tile: 16 bytes apart
        const int f = wave + 8 * (i - I_CV), rb = f >> 1, ps = f & 1;
        const int rho = 16 * rb + j, p = 32 * ps + 8 * grp;
        const int rs = rho >> 5, hi = (rho & 31) >> 3, slot = rho & 7;
        uint16_t *dst = cv16 + ((((p >> 4) * RS + rs) * 64 + (p & 15) + 16 * hi) * 8 + slot);
        const int nvalid = qmax_pos - (k0 + p) + 1;  // keys p + e with e < nvalid are visible
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w = st[i][e >> 1];
          const uint16_t v = e < nvalid ? static_cast<uint16_t>((e & 1) ? (w >> 16) : (w & 0xffffu))
                                        : static_cast<uint16_t>(0);
          dst[8 * e] = v;
        }
      } else {
        cs[tid + 512 * i] = st[i];
      }
    }
  };

  const int side = wave >> 2, idx = wave & 3;
  const int pr = idx % NP, kb0 = (idx / NP) * NKB;
  f32x4 acc[NKB][2];
#pragma unroll
  for (int kk = 0; kk < NKB; ++kk) acc[kk][0] = acc[kk][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kt = ktile, k0 = kt * KT;
  gload(kt, 0);
  for (int c = 0; c < nchunk; ++c) {
    const bool last = c == nchunk - 1;
    __syncthreads();
    swrite(kt);
    // the next chunk's loads fly under this chunk's products
    if (!last) gload(kt, c + 1);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // ---- rebuild products of this chunk ----
    const int nrs = min(RS, (side == 0 ? rsk : rsv) - c * RS);
    if (side == 0) {
      // K^T[d][key] = sum_r B_k^T[d][r] C_k[key][r]
#pragma unroll 1
      for (int rs = 0; rs < nrs; ++rs) {
        {
          const u32x4 fa = cs[O_BK + (pr * RS + rs) * 64 + lane];
          const u32x4 fb = cs[O_BK + ((pr + HALF) * RS + rs) * 64 + lane];
#pragma unroll
          for (int kk = 0; kk < NKB; ++kk) {
            const u32x4 cf = cs[((kb0 + kk) * RS + rs) * 64 + lane];
            acc[kk][0] = mfma_bf16(fa, cf, acc[kk][0]);
            acc[kk][1] = mfma_bf16(fb, cf, acc[kk][1]);
          }
        }
      }
    } else {
      // V[key][d] = sum_r C_v[key][r] B_v^T[d][r]
#pragma unroll 1
      for (int rs = 0; rs < nrs; ++rs) {
        {
          const u32x4 f0 = cs[O_BV + ((2 * pr) * RS + rs) * 64 + lane];
          const u32x4 f1 = cs[O_BV + ((2 * pr + 1) * RS + rs) * 64 + lane];
#pragma unroll
          for (int kk = 0; kk < NKB; ++kk) {
            const u32x4 cf = cs[O_CV + ((kb0 + kk) * RS + rs) * 64 + lane];
            acc[kk][0] = mfma_bf16(cf, f0, acc[kk][0]);
            acc[kk][1] = mfma_bf16(cf, f1, acc[kk][1]);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!last) continue;

    // ---- K waves: lane (key = j, grp) holds K^T[16 blk + 4 grp + r][16 kb + j]
    // for blk = pr (acc[.][0]) and its rotary partner pr + HALF (acc[.][1]);
    // V waves: lane (d = j, grp) holds V[16 kb + 4 grp + r][16 (2 pr + h) + j] ----
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      const int kb = kb0 + kk;
      if (side == 0) {
        const int keyrow = k0 + 16 * kb + j;
        if (rope_on) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float cc, ss;
            rope_cs(keyrow, revs[16 * pr + 4 * grp + r], cc, ss);
            const float u = acc[kk][0][r], v = acc[kk][1][r];
            acc[kk][0][r] = u * cc - v * ss;
            acc[kk][1][r] = u * ss + v * cc;
          }
        }
        const int krow = 16 * kb + j;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int dcol = 16 * (pr + hh * HALF) + 4 * grp;
          const int chunk = (dcol >> 3) ^ (krow & (CH - 1));
          *reinterpret_cast<u32x2 *>(&Ks[krow * D + chunk * 8 + (dcol & 7)]) =
              u32x2{pack2(acc[kk][hh][0], acc[kk][hh][1]), pack2(acc[kk][hh][2], acc[kk][hh][3])};
        }
      } else {
        // V^T row dd holds each 32-key half u with key 32u + 16hk + 4grp + r
        // at 32u + 8grp + 4hk + r: the eight keys one lane of the P V
        // product takes are one 16-byte chunk (4u + grp), XOR-swizzled by
        // the row's low three bits
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int dd = 16 * (2 * pr + h) + j;
          const int chunk = (4 * (kb >> 1) + grp) ^ (dd & 7);
          *reinterpret_cast<u32x2 *>(&Vt[dd * KT + chunk * 8 + 4 * (kb & 1)]) =
              u32x2{pack2(acc[kk][h][0], acc[kk][h][1]), pack2(acc[kk][h][2], acc[kk][h][3])};
        }
      }
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // the tile's image: K rows (rotated, swizzled) then V^T rows (swizzled)
    uint16_t *img = a.kv + ((static_cast<size_t>(b) * a.n_kv + g) * (a.L_max / KT) + kt) * (2 * KT * D);
    for (int u = tid; u < KT * D / 8; u += 512) {
      *reinterpret_cast<u32x4 *>(img + 8 * u) = *reinterpret_cast<const u32x4 *>(Ks + 8 * u);
      *reinterpret_cast<u32x4 *>(img + KT * D + 8 * u) = *reinterpret_cast<const u32x4 *>(Vt + 8 * u);
    }
  }
}

template <int DB>
__global__ __launch_bounds__(512) void attn_prefill_kernel(AttnPrefillArgs a) {
  constexpr int D = DB * 16, HALF = DB / 2, KT = 64;
  constexpr int CH = D / 8;       // 16-byte chunks per K row
  constexpr int IMG = 2 * KT * D;           // elements of one key tile's image
  constexpr int NI = IMG / 8 / 512;         // 16-byte units per thread
  __shared__ __attribute__((aligned(16))) uint16_t KVs[2][IMG];   // double-buffered images
  __shared__ double revs[D / 2];

  // wave is made provably uniform, so every fragment index derived from it
  // stays scalar and each load is a scalar base plus the lane's 16 bytes
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, grp = lane >> 4;
  const int G = a.n_q / a.n_kv;
  const int QT = 256 / G;
  const int nqt = (a.T + QT - 1) / QT;
  // Work order: the hardware deals workgroups to the eight XCDs round-robin
  // in linear order; the index is remapped so each XCD runs all query tiles
  // of a few (sequence, kv head) pairs, sharing their latents and factor
  // slices in its L2, heaviest (latest) query tiles first.
  int qt, g, b;
  {
    const int total = static_cast<int>(gridDim.x * gridDim.y * gridDim.z);
    const int L = static_cast<int>(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    const int xcd = L & 7, local = L >> 3, q = total >> 3, rem = total & 7;
    const int Lg = xcd < rem ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
    qt = nqt - 1 - Lg % nqt;
    g = (Lg / nqt) % a.n_kv;
    b = Lg / nqt / a.n_kv;
  }
  const int t0 = qt * QT;
  const int past = a.past_lens[b];
  const bool rope_on = a.theta != 0.f;

  for (int i = tid; i < D / 2; i += 512) revs[i] = rope_on ? rope_rev(i, D, a.theta) : 0.0;

  // ---- query fragments: rows rho = 32*wave + 16*qb + (0..15), rotated
  // and scaled, kept in registers for the whole work item.
  // B operand of S^T = K Q^T: lane (q = j, grp) holds Q[q][32t + 8grp + e].
  int qpos[2];
  bool qok[2];
  u32x4 qf[2][HALF];
  __syncthreads();
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int rho = 32 * wave + 16 * qb + j;
    const int hl = rho / QT, tt = t0 + rho % QT;
    qok[qb] = tt < a.T;
    const int ttc = qok[qb] ? tt : a.T - 1;
    qpos[qb] = past + ttc;
    float x[HALF][8];
    const size_t off = (static_cast<size_t>(b) * a.T + ttc) * a.ldq + static_cast<size_t>(g * G + hl) * D;
#pragma unroll
    for (int t = 0; t < HALF; ++t) {
      if (a.q_f32) {
        const float *p = static_cast<const float *>(a.q) + off + 32 * t + 8 * grp;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[t][e] = p[e];
      } else {
        const u32x4 v = ld16(static_cast<const uint16_t *>(a.q) + off + 32 * t + 8 * grp);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[t][2 * e] = bflo(v[e]);
          x[t][2 * e + 1] = bfhi(v[e]);
        }
      }
    }
    if (rope_on) {
      // partner of d = 32t + 8grp + e (t < HALF/2) is d + D/2 = 32(t + HALF/2) + 8grp + e
#pragma unroll
      for (int t = 0; t < HALF / 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float c, s;
          rope_cs(qpos[qb], revs[32 * t + 8 * grp + e], c, s);
          const float u = x[t][e], v = x[t + HALF / 2][e];
          x[t][e] = u * c - v * s;
          x[t + HALF / 2][e] = u * s + v * c;
        }
    }
#pragma unroll
    for (int t = 0; t < HALF; ++t)
      qf[qb][t] = u32x4{pack2(x[t][0] * a.scale_log2, x[t][1] * a.scale_log2),
                        pack2(x[t][2] * a.scale_log2, x[t][3] * a.scale_log2),
                        pack2(x[t][4] * a.scale_log2, x[t][5] * a.scale_log2),
                        pack2(x[t][6] * a.scale_log2, x[t][7] * a.scale_log2)};
  }

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  f32x4 accO[2][DB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int x = 0; x < DB; ++x) accO[qb][x] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int qmax_pos = past + min(t0 + QT, a.T) - 1;
  const int qpos_lo = min(qpos[0], qpos[1]);  // this lane's earliest query position
  const int nkt = qmax_pos / KT + 1;
  const uint16_t *imgs = a.kv + (static_cast<size_t>(b) * a.n_kv + g) * (a.L_max / KT) * IMG;
  u32x4 st[NI];
  auto iload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < NI; ++i) st[i] = ld16(imgs + static_cast<size_t>(kt) * IMG + 8 * (tid + 512 * i));
  };
  auto istore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4 *>(&KVs[buf][8 * (tid + 512 * i)]) = st[i];
  };
  iload(0);
  istore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * KT;
    if (kt + 1 < nkt) iload(kt + 1);   // in flight under this tile's work
    const uint16_t *Ks = KVs[kt & 1];
    const uint16_t *Vt = KVs[kt & 1] + KT * D;
    // ---- attention for this wave's 32 query rows (two blocks of 16) ----
    // Each K and V fragment is read from LDS once and feeds the MFMAs of
    // both query blocks. Swizzles depend on the row only through j (rows
    // 16 kk + j, d rows 16 x + j), so each (t) or (u, half) needs one base
    // and the key block / d block is a constant offset.
    f32x4 sc[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) sc[qb][kk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < HALF; ++t) {
      const uint16_t *kp = Ks + j * D + (((4 * t + grp) ^ (j & (CH - 1))) * 8);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 kf = *reinterpret_cast<const u32x4 *>(kp + 16 * kk * D);
        sc[0][kk] = mfma_bf16(kf, qf[0][t], sc[0][kk]);
        sc[1][kk] = mfma_bf16(kf, qf[1][t], sc[1][kk]);
      }
    }
    // lane (q = j, grp) holds S^T[k0 + 16kk + 4grp + r][q]. Only tiles that
    // reach past the wave's earliest query position (past + t0: its rows are
    // tokens t0 .. t0 + 31 of one head) need the causal mask.
    if (k0 + KT - 1 > past + t0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (k0 + 16 * kk + 4 * grp + r > qpos[qb]) sc[qb][kk][r] = -INFINITY;
    }
    float alpha[2];
    bool grew = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[qb][kk][r]);
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      const float m_new = fmaxf(m_run[qb], mx);
      grew |= m_new > m_run[qb];
      alpha[qb] = exp2_hw(m_run[qb] - m_new);
      float psum = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sc[qb][kk][r] = exp2_hw(sc[qb][kk][r] - m_new);
          psum += sc[qb][kk][r];
        }
      // per-lane partial sums: the four lanes of a row share alpha, so they
      // are added across lanes once, after the last tile
      l_run[qb] = l_run[qb] * alpha[qb] + psum;
      m_run[qb] = m_new;
    }
    // the output rescale only when some row's running maximum rose
    if (__builtin_amdgcn_ballot_w64(grew)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int x = 0; x < DB; ++x) accO[qb][x] *= alpha[qb];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const u32x4 pf0 = pack_acc(sc[0][2 * u], sc[0][2 * u + 1]);
      const u32x4 pf1 = pack_acc(sc[1][2 * u], sc[1][2 * u + 1]);
      // keys 32u + 4grp + r and 32u + 16 + 4grp + r of d row 16x + j: one
      // swizzled chunk of the image
      const uint16_t *vp = Vt + j * KT + 8 * ((4 * u + grp) ^ (j & 7));
#pragma unroll
      for (int x = 0; x < DB; ++x) {
        const u32x4 vf = *reinterpret_cast<const u32x4 *>(vp + 16 * x * KT);
        accO[0][x] = mfma_bf16(vf, pf0, accO[0][x]);
        accO[1][x] = mfma_bf16(vf, pf1, accO[1][x]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nkt) istore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- normalise and store: lane (q = j, grp) holds O^T[16x + 4grp + r][q] ----
  float lsum[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) lsum[qb] = wave_sum_xor(wave_sum_xor(l_run[qb], 16), 32);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (!qok[qb]) continue;
    const int rho = 32 * wave + 16 * qb + j;
    const int hl = rho / QT, tt = t0 + rho % QT;
    const float inv = 1.f / lsum[qb];
    // row b T + tt, columns (g G + hl) D + 16 x + 4 grp .. +3: four
    // contiguous elements row-major and in operand tiles alike
    const int orow = b * a.T + tt, ocol = (g * G + hl) * D + 4 * grp;
    const int ncol = a.n_q * D;
#pragma unroll
    for (int x = 0; x < DB; ++x) {
      const size_t o = a.out_tiled ? tile_off(orow, ocol + 16 * x, ncol)
                                   : static_cast<size_t>(orow) * ncol + ocol + 16 * x;
      *reinterpret_cast<u32x2 *>(a.out + o) =
          u32x2{pack2(accO[qb][x][0] * inv, accO[qb][x][1] * inv),
                pack2(accO[qb][x][2] * inv, accO[qb][x][3] * inv)};
    }
  }
}

}  // namespace

hipError_t launch_attn_prefill_bf16(const AttnPrefillArgs &a, hipStream_t s) {
  TraceGuard trace_guard(K_ATTN_PREFILL, s);
  const int G = a.n_q / a.n_kv;
  const int QT = 256 / G;
  // the kernel addresses the cache pools and each factor through 32-bit
  // buffer offsets
  const int64_t lim = INT32_MAX;
  if (a.pool_pages * kPage * std::max(a.r_k, a.r_v) * 2 > lim ||
      static_cast<int64_t>(a.n_kv) * a.d * std::max(a.r_k, a.r_v) * 2 > lim)
    return hipErrorInvalidValue;
  if (!a.kv) return hipErrorInvalidValue;
  dim3 rgrid(a.L_max / kPage, a.n_kv, a.Bsz);
  if (a.d == 128)
    attn_rebuild_kernel<8><<<rgrid, 512, 0, s>>>(a);
  else
    attn_rebuild_kernel<4><<<rgrid, 512, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((a.T + QT - 1) / QT, a.n_kv, a.Bsz);
  if (a.d == 128)
    attn_prefill_kernel<8><<<grid, 512, 0, s>>>(a);
  else
    attn_prefill_kernel<4><<<grid, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dl
