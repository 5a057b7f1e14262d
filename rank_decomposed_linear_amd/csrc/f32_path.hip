// float32 path: plain VALU kernels for every shape (used when the caller
// passes DL_F32). They compute the same operations as the bf16 MFMA kernels
// -- factor-pair GEMMs (DeInfer section 2.1, Eq. (1)) and attention that
// rebuilds each key and value from the low-rank cache on the fly (section
// 4.2) -- in full float32, for shapes too small or too irregular for the
// MFMA tiling. Storage follows the bf16 path: weights transposed (Wt[N, K]),
// up factors [n_kv * d, r], value cache rank-major [Bsz, r_v, L_max].
#include <math.h>

#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace dl {

namespace {

constexpr int TM = 64, TN = 64, TK = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Args a) {
  __shared__ float As[TK][TM + 1];
  __shared__ float Bs[TK][TN + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < a.K; k0 += TK) {
    for (int i = tid; i < TM * TK; i += 256) {
      const int r = i / TK, kk = i % TK;
      const int m = m0 + r, k = k0 + kk;
      float v = 0.f;
      if (m < a.M && k < a.K) {
        v = a.X[static_cast<size_t>(m) * a.ldx + k];
        if (a.X2) v = (v / (1.f + expf(-v))) * a.X2[static_cast<size_t>(m) * a.ldx + k];
      }
      As[kk][r] = v;
    }
    for (int i = tid; i < TK * TN; i += 256) {
      const int c = i / TK, kk = i % TK;
      const int k = k0 + kk, n = n0 + c;
      Bs[kk][c] = (k < a.K && n < a.N) ? a.W[static_cast<size_t>(n) * a.K + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[i] = Bs[kk][tx * 4 + i];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = fmaf(av[i], bv[jj], acc[i][jj]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= a.M) continue;
    if (a.omode == F32_OUT_CACHE_T) {
      const int b = m / a.T, t = m - b * a.T;
      const size_t col = static_cast<size_t>(a.past_lens[b]) + t;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int n = n0 + tx * 4 + jj;
        if (n < a.N) a.C[(static_cast<size_t>(b) * a.N + n) * a.L_max + col] = acc[i][jj];
      }
      continue;
    }
    size_t rowoff;
    if (a.omode == F32_OUT_CACHE) {
      const int b = m / a.T, t = m - b * a.T;
      rowoff = (static_cast<size_t>(b) * a.L_max + a.past_lens[b] + t) * a.ldc;
    } else {
      rowoff = static_cast<size_t>(m) * a.ldc;
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int n = n0 + tx * 4 + jj;
      if (n >= a.N) continue;
      float v = acc[i][jj];
      if (a.omode == F32_OUT_RESID) v += a.R[static_cast<size_t>(m) * a.ldr + n];
      if (a.omode == F32_OUT_RELU) v = fmaxf(v, 0.f);
      a.C[rowoff + n] = v;
    }
  }
}

// One wave per (sequence, token, query head). Lane u owns rotary pairs
// (i, i + d/2) for i = lane + 64u; every key and value row is rebuilt from
// the cache as it is visited, with an online softmax.
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnF32Args a) {
  const int lane = threadIdx.x;
  const int h = blockIdx.x % a.n_q;
  const int t = (blockIdx.x / a.n_q) % a.T;
  const int b = blockIdx.x / (a.n_q * a.T);
  const int D = a.d, H = D / 2, G = a.n_q / a.n_kv, g = h / G;
  const int pos = a.decode ? a.lens[b] - 1 : a.lens[b] + t;
  const bool rope_on = a.theta != 0.f;

  float qx[2] = {0.f, 0.f}, qy[2] = {0.f, 0.f};
  double rev[2] = {0.0, 0.0};
  bool ok[2];
  const float *qrow = a.q + (static_cast<size_t>(b) * a.T + t) * a.ldq + static_cast<size_t>(h) * D;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = lane + 64 * u;
    ok[u] = i < H;
    if (!ok[u]) continue;
    if (rope_on) rev[u] = rope_rev(i, D, a.theta);
    float x = qrow[i], y = qrow[i + H];
    if (rope_on) {
      float c, s;
      rope_cs(pos, rev[u], c, s);
      const float x2 = x * c - y * s;
      y = x * s + y * c;
      x = x2;
    }
    qx[u] = x;
    qy[u] = y;
  }
  float m = -INFINITY, l = 0.f;
  float ox[2] = {0.f, 0.f}, oy[2] = {0.f, 0.f};
  for (int key = 0; key <= pos; ++key) {
    const float *ckr = a.ck + (static_cast<size_t>(b) * a.L_max + key) * a.r_k;
    const float *cvc = a.cv + static_cast<size_t>(b) * a.r_v * a.L_max + key;
    float kx[2] = {0.f, 0.f}, ky[2] = {0.f, 0.f}, vx[2] = {0.f, 0.f}, vy[2] = {0.f, 0.f};
    // up-factor rows of this lane's dimensions (i, i + d/2)
    const float *bk = a.bk + static_cast<size_t>(g * D) * a.r_k;
    const float *bv = a.bv + static_cast<size_t>(g * D) * a.r_v;
    for (int r = 0; r < a.r_k; ++r) {
      const float c = ckr[r];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (ok[u]) {
          kx[u] = fmaf(c, bk[static_cast<size_t>(lane + 64 * u) * a.r_k + r], kx[u]);
          ky[u] = fmaf(c, bk[static_cast<size_t>(lane + 64 * u + H) * a.r_k + r], ky[u]);
        }
    }
    for (int r = 0; r < a.r_v; ++r) {
      const float c = cvc[static_cast<size_t>(r) * a.L_max];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (ok[u]) {
          vx[u] = fmaf(c, bv[static_cast<size_t>(lane + 64 * u) * a.r_v + r], vx[u]);
          vy[u] = fmaf(c, bv[static_cast<size_t>(lane + 64 * u + H) * a.r_v + r], vy[u]);
        }
    }
    float dot = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (ok[u]) {
        float x = kx[u], y = ky[u];
        if (rope_on) {
          float c, s;
          rope_cs(key, rev[u], c, s);
          const float x2 = x * c - y * s;
          y = x * s + y * c;
          x = x2;
        }
        dot = fmaf(qx[u], x, fmaf(qy[u], y, dot));
      }
    const float sc = wave_sum(dot) * a.sm_scale;
    const float m_new = fmaxf(m, sc);
    const float alpha = expf(m - m_new);
    const float p = expf(sc - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      ox[u] = ox[u] * alpha + p * vx[u];
      oy[u] = oy[u] * alpha + p * vy[u];
    }
    m = m_new;
  }
  float *orow = a.out + (static_cast<size_t>(b) * a.T + t) * a.n_q * D + static_cast<size_t>(h) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (ok[u]) {
      orow[lane + 64 * u] = ox[u] * inv;
      orow[lane + 64 * u + H] = oy[u] * inv;
    }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmF32Args &a, hipStream_t s) {
  TraceGuard trace_guard(K_GEMM_F32, s);
  dim3 grid((a.N + TN - 1) / TN, (a.M + TM - 1) / TM);
  gemm_f32_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnF32Args &a, hipStream_t s) {
  TraceGuard trace_guard(K_ATTN_F32, s);
  attn_f32_kernel<<<a.Bsz * a.T * a.n_q, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dl
