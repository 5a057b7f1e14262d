// Attention over the low-rank KV cache, bf16 MFMA (DeInfer section 4.2:
// rebuild K = C_k B_k and V = C_v B_v from the cached latents, rotate the
// rebuilt keys, attend).
//
// Neither K nor V is ever written to memory. Caches and factors are stored
// in 16 x 32 operand tiles (MFMA lane order): a key block of 16 positions x
// 32 ranks and an up-factor fragment are each one contiguous 1 KB read; the
// value cache is rank-major ([r_v, L_max] tiles per sequence) and gathered
// per key. The rebuilt tiles live in MFMA accumulators:
//
//  prefill  A workgroup owns one kv head and up to 256 (token, head) query
//           rows; per 64-key tile its eight waves rebuild K (rotated) and
//           V^T into swizzled LDS, then each wave runs an online-softmax
//           pass for its 32 query rows.
#include <math.h>

#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace dl {

namespace {

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// operand fragment (rank step rs, d block blk of kv head g) of an up factor
// stored [n_kv * d, r] in tiles: lane (c, grp) gets B[32rs + 8grp .. +8][16blk + c]
__device__ __forceinline__ u32x4 frag(const uint16_t *bt, int r, int gblk, int rs, int lane) {
  return ld16(bt + frag_off(gblk, rs, r, lane));
}

// ---------------------------------------------------------------------------
// Prefill
// ---------------------------------------------------------------------------
template <int DB>
__global__ __launch_bounds__(512) void attn_prefill_kernel(AttnPrefillArgs a) {
  constexpr int D = DB * 16, HALF = DB / 2, KT = 64;
  constexpr int CH = D / 8;  // 16-byte chunks per K row
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * KT];
  __shared__ double revs[D / 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int G = a.n_q / a.n_kv;
  const int QT = 256 / G;
  const int nqt = (a.T + QT - 1) / QT;
  const int qt = nqt - 1 - static_cast<int>(blockIdx.x);
  const int g = blockIdx.y, b = blockIdx.z;
  const int t0 = qt * QT;
  const int past = a.past_lens[b];
  const bool rope_on = a.theta != 0.f;

  for (int i = tid; i < D / 2; i += 512) revs[i] = rope_on ? rope_rev(i, D, a.theta) : 0.0;
  __syncthreads();

  // ---- query fragments: rows rho = 32*wave + 16*qb + (0..15) ----
  // B operand of S^T = K Q^T: lane (q = j, grp) holds Q[q][32t + 8grp + e].
  u32x4 qf[2][HALF];
  int qpos[2];
  bool qok[2];
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
  const int nkt = qmax_pos / KT + 1;
  const int rsk = a.r_k / 32, rsv = a.r_v / 32;
  const uint16_t *ck_b = a.ck + static_cast<size_t>(b) * a.L_max * a.r_k;
  const uint16_t *cv_b = a.cv + static_cast<size_t>(b) * a.r_v * a.L_max;
  const int kb = wave >> 1;  // key block rebuilt by this wave

  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * KT;
    const int keyrow = k0 + 16 * kb + j;
    const bool kvalid = keyrow <= qmax_pos;
    // ---- rebuild K (rotated) for key block kb, d blocks {x, x+HALF} ----
    {
      constexpr int NX = HALF / 2 > 0 ? HALF / 2 : 1;
      f32x4 acc[NX][2];
#pragma unroll
      for (int xi = 0; xi < NX; ++xi) acc[xi][0] = acc[xi][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int xbase = (wave & 1) * NX;
      // key tile of this 16-key block (lanes of keys past the last query
      // position do not load)
      const uint16_t *cp = ck_b + frag_off((k0 >> 4) + kb, 0, a.r_k, lane);
      for (int rs = 0; rs < rsk; ++rs) {
        const u32x4 c = kvalid ? ld16(cp + 512 * rs) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int xi = 0; xi < NX; ++xi) {
          acc[xi][0] = mfma_bf16(frag(a.bk, a.r_k, g * DB + xbase + xi, rs, lane), c, acc[xi][0]);
          acc[xi][1] = mfma_bf16(frag(a.bk, a.r_k, g * DB + xbase + xi + HALF, rs, lane), c, acc[xi][1]);
        }
      }
      // lane (key = j, grp) holds K^T[16blk + 4grp + r][keyrow]
#pragma unroll
      for (int xi = 0; xi < NX; ++xi) {
        const int blk = xbase + xi;
        if (rope_on) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float c, s;
            rope_cs(keyrow, revs[16 * blk + 4 * grp + r], c, s);
            const float u = acc[xi][0][r], v = acc[xi][1][r];
            acc[xi][0][r] = u * c - v * s;
            acc[xi][1][r] = u * s + v * c;
          }
        }
        const int krow = 16 * kb + j;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int dcol = 16 * (blk + hh * HALF) + 4 * grp;
          const int chunk = (dcol >> 3) ^ (krow & (CH - 1));
          *reinterpret_cast<u32x2 *>(&Ks[krow * D + chunk * 8 + (dcol & 7)]) =
              u32x2{pack2(acc[xi][hh][0], acc[xi][hh][1]), pack2(acc[xi][hh][2], acc[xi][hh][3])};
        }
      }
    }
    // ---- rebuild V^T for key block kb, d blocks (wave&1)*HALF .. +HALF ----
    {
      f32x4 acc[HALF];
#pragma unroll
      for (int x = 0; x < HALF; ++x) acc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int nb0 = (wave & 1) * HALF;
      // C_v[keyrow][32rs + 8grp + e], e = 0..7, gathered from the value tiles
      for (int rs = 0; rs < rsv; ++rs) {
        u32x4 c = {0u, 0u, 0u, 0u};
        if (kvalid) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            c[q] = static_cast<uint32_t>(cv_b[tile_off(32 * rs + 8 * grp + 2 * q, keyrow, a.L_max)]) |
                   (static_cast<uint32_t>(cv_b[tile_off(32 * rs + 8 * grp + 2 * q + 1, keyrow, a.L_max)]) << 16);
        }
#pragma unroll
        for (int x = 0; x < HALF; ++x) acc[x] = mfma_bf16(c, frag(a.bv, a.r_v, g * DB + nb0 + x, rs, lane), acc[x]);
      }
      // lane (d = j, grp) holds V[16kb + 4grp + r][16(nb0+x) + j]
#pragma unroll
      for (int x = 0; x < HALF; ++x) {
        const int dd = 16 * (nb0 + x) + j;
        const int unit = (4 * kb + grp) ^ (dd & 15);
        *reinterpret_cast<u32x2 *>(&Vt[dd * KT + unit * 4]) =
            u32x2{pack2(acc[x][0], acc[x][1]), pack2(acc[x][2], acc[x][3])};
      }
    }
    __syncthreads();

    // ---- attention for this wave's 32 query rows ----
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x4 s[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        s[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int krow = 16 * kk + j;
#pragma unroll
        for (int t = 0; t < HALF; ++t) {
          const int chunk = (4 * t + grp) ^ (krow & (CH - 1));
          s[kk] = mfma_bf16(*reinterpret_cast<const u32x4 *>(&Ks[krow * D + chunk * 8]), qf[qb][t],
                            s[kk]);
        }
      }
      // lane (q = j, grp) holds S^T[k0 + 16kk + 4grp + r][q]
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (k0 + 16 * kk + 4 * grp + r > qpos[qb]) s[kk][r] = -INFINITY;
          mx = fmaxf(mx, s[kk][r]);
        }
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      const float m_new = fmaxf(m_run[qb], mx);
      const float alpha = exp2f(m_run[qb] - m_new);
      float psum = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[kk][r] = exp2f(s[kk][r] - m_new);
          psum += s[kk][r];
        }
      psum = wave_sum_xor(psum, 16);
      psum = wave_sum_xor(psum, 32);
      l_run[qb] = l_run[qb] * alpha + psum;
      m_run[qb] = m_new;
#pragma unroll
      for (int x = 0; x < DB; ++x) accO[qb][x] *= alpha;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4 pf = pack_acc(s[2 * u], s[2 * u + 1]);
#pragma unroll
        for (int x = 0; x < DB; ++x) {
          const int dd = 16 * x + j;
          const int u0 = (4 * (2 * u) + grp) ^ (dd & 15);
          const int u1 = (4 * (2 * u + 1) + grp) ^ (dd & 15);
          const u32x2 lo = *reinterpret_cast<const u32x2 *>(&Vt[dd * KT + u0 * 4]);
          const u32x2 hi = *reinterpret_cast<const u32x2 *>(&Vt[dd * KT + u1 * 4]);
          accO[qb][x] = mfma_bf16(u32x4{lo.x, lo.y, hi.x, hi.y}, pf, accO[qb][x]);
        }
      }
    }
    __syncthreads();
  }

  // ---- normalise and store: lane (q = j, grp) holds O^T[16x + 4grp + r][q] ----
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (!qok[qb]) continue;
    const int rho = 32 * wave + 16 * qb + j;
    const int hl = rho / QT, tt = t0 + rho % QT;
    const float inv = 1.f / l_run[qb];
    uint16_t *dst = a.out + (static_cast<size_t>(b) * a.T + tt) * a.n_q * D +
                    static_cast<size_t>(g * G + hl) * D;
#pragma unroll
    for (int x = 0; x < DB; ++x)
      *reinterpret_cast<u32x2 *>(dst + 16 * x + 4 * grp) =
          u32x2{pack2(accO[qb][x][0] * inv, accO[qb][x][1] * inv),
                pack2(accO[qb][x][2] * inv, accO[qb][x][3] * inv)};
  }
}

}  // namespace

hipError_t launch_attn_prefill_bf16(const AttnPrefillArgs &a, hipStream_t s) {
  TraceGuard trace_guard(K_ATTN_PREFILL, s);
  const int G = a.n_q / a.n_kv;
  const int QT = 256 / G;
  dim3 grid((a.T + QT - 1) / QT, a.n_kv, a.Bsz);
  if (a.d == 128)
    attn_prefill_kernel<8><<<grid, 512, 0, s>>>(a);
  else
    attn_prefill_kernel<4><<<grid, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dl
