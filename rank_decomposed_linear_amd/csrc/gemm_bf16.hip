// bf16 MFMA GEMM for prefill-sized M: one factor of a decomposed projection
// (W ~ A B, DeInfer section 2.1, Eq. (1)), C = X W with f32 accumulation.
//
// Both factors are stored [in, out] row-major, so the reduction index of the
// weight operand is its row index: the 16x16x32 MFMA wants eight consecutive
// reduction values per lane. The weight tile is therefore transposed once
// per workgroup while it is staged into LDS: a thread loads eight rows x
// eight columns (eight 16-byte loads covering 4 rows x 256 contiguous bytes
// per instruction), transposes them in registers and writes eight operand
// fragments in lane order, so every MFMA operand read from LDS is one
// conflict-free 16-byte ds_read. The activation tile is staged as rows with
// an XOR swizzle of its 16-byte chunks.
//
// Tile 128 x 128 x 64, 4 waves (2 x 2), each wave 64 x 64 = 4 x 4 MFMA
// blocks; LDS double-buffered (64 KB).
#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace dl {

namespace {
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kAElems = BM * BK;          // bf16 elements of one A tile
constexpr int kBElems = BK * BN;          // bf16 elements of one B tile (fragments)

struct Stage {
  u32x4 v[8];
};

__device__ __forceinline__ u32x4 swiglu8(u32x4 g, u32x4 u) {
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float a0 = silu(bflo(g[q])) * bflo(u[q]);
    const float a1 = silu(bfhi(g[q])) * bfhi(u[q]);
    r[q] = pack2(a0, a1);
  }
  return r;
}

__device__ __forceinline__ void transpose8(const u32x4 (&r)[8], u32x4 (&b)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = r[2 * q][e >> 1], hi = r[2 * q + 1][e >> 1];
      b[e][q] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
  }
}

template <int XM, int OM>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][kAElems + kBElems];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;

  const int bx = blockIdx.x;
  int si = 0;
  if (a.nseg > 1 && bx >= a.seg[1].tile_begin) si = 1;
  if (a.nseg > 2 && bx >= a.seg[2].tile_begin) si = 2;
  const GemmSeg sg = a.seg[si];
  const int n0 = (bx - sg.tile_begin) * BN;
  const int m0 = blockIdx.y * BM;

  // Loader roles: threads 0..127 stage A (8 rows x 16 B each),
  // threads 128..255 stage B (8 k-rows x 8 columns each).
  const bool loads_a = tid < 128;
  const int t = tid & 127;
  // A: chunk kc = t % 8 of rows (t / 8) + 16 * it, it = 0..7
  const int a_kc = t & 7, a_r0 = t >> 3;
  // B: k-row group q = t / 16 (rows 8q..8q+7), column group p = t % 16
  const int b_q = t >> 4, b_p = t & 15;
  const int b_col = n0 + 8 * b_p;
  const bool b_ok = b_col < sg.N;

  auto gload = [&](Stage &st, int k0) {
    if (loads_a) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = m0 + a_r0 + 16 * it;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row < a.M) {
          const size_t off = static_cast<size_t>(row) * sg.ldx + k0 + 8 * a_kc;
          v = *reinterpret_cast<const u32x4 *>(sg.X + off);
          if constexpr (XM == GEMM_X_SWIGLU)
            v = swiglu8(v, *reinterpret_cast<const u32x4 *>(sg.X2 + off));
        }
        st.v[it] = v;
      }
    } else {
      const uint16_t *wp = sg.W + static_cast<size_t>(k0 + 8 * b_q) * sg.N + b_col;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        st.v[s] = b_ok ? *reinterpret_cast<const u32x4 *>(wp + static_cast<size_t>(s) * sg.N)
                       : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](const Stage &st, int buf) {
    uint16_t *base = lds[buf];
    if (loads_a) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = a_r0 + 16 * it;
        const int chunk = a_kc ^ (row & 7);
        *reinterpret_cast<u32x4 *>(base + row * BK + chunk * 8) = st.v[it];
      }
    } else {
      u32x4 f[8];
      transpose8(st.v, f);
      // k rows 8q..8q+7 -> kstep ks = q/4, lane group g = q%4;
      // column 8p + e -> block nb = p/2, lane column jj = 8(p%2) + e
      const int ks = b_q >> 2, g = b_q & 3, nb = b_p >> 1;
      uint16_t *fb = base + kAElems + ((ks * (BN / 16) + nb) * 64) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ln = g * 16 + 8 * (b_p & 1) + e;
        *reinterpret_cast<u32x4 *>(fb + ln * 8) = f[e];
      }
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ktiles = a.K / BK;
  Stage st;
  gload(st, 0);
  sstore(st, 0);
  __syncthreads();
  for (int kt = 0; kt < ktiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ktiles) gload(st, (kt + 1) * BK);
    const uint16_t *base = lds[buf];
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      u32x4 af[4], bfr[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int row = wm * 64 + mb * 16 + j;
        const int chunk = (ks * 4 + grp) ^ (row & 7);
        af[mb] = *reinterpret_cast<const u32x4 *>(base + row * BK + chunk * 8);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int gnb = wn * 4 + nb;
        bfr[nb] = *reinterpret_cast<const u32x4 *>(base + kAElems +
                                                   ((ks * (BN / 16) + gnb) * 64 + lane) * 8);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma_bf16(af[mb], bfr[nb], acc[mb][nb]);
    }
    if (kt + 1 < ktiles) sstore(st, buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane (j, grp) holds C[m0 + 64wm + 16mb + 4grp + r][n0 + 64wn + 16nb + j].
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + mb * 16 + 4 * grp + r;
      if (m >= a.M) continue;
      size_t rowoff;
      if constexpr (OM == GEMM_OUT_CACHE) {
        const int b = m / a.T, tt = m - b * a.T;
        rowoff = (static_cast<size_t>(b) * a.L_max + a.past_lens[b] + tt) * sg.ldc;
      } else {
        rowoff = static_cast<size_t>(m) * sg.ldc;
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int n = n0 + wn * 64 + nb * 16 + j;
        if (n >= sg.N) continue;
        float v = acc[mb][nb][r];
        if constexpr (OM == GEMM_OUT_BF16 || OM == GEMM_OUT_CACHE) {
          static_cast<uint16_t *>(sg.C)[rowoff + n] = f2bf(v);
        } else if constexpr (OM == GEMM_OUT_BF16_RES_F32) {
          v += static_cast<const float *>(sg.R)[static_cast<size_t>(m) * sg.ldr + n];
          static_cast<uint16_t *>(sg.C)[rowoff + n] = f2bf(v);
          if (sg.C32) sg.C32[rowoff + n] = v;
        } else {  // GEMM_OUT_F32_RES_BF16
          v += bf2f(static_cast<const uint16_t *>(sg.R)[static_cast<size_t>(m) * sg.ldr + n]);
          sg.C32[rowoff + n] = v;
        }
      }
    }
  }
}

template <int XM>
hipError_t launch_x(const GemmArgs &a, dim3 grid, hipStream_t s) {
  switch (a.omode) {
    case GEMM_OUT_BF16: gemm_bf16_kernel<XM, GEMM_OUT_BF16><<<grid, kThreads, 0, s>>>(a); break;
    case GEMM_OUT_BF16_RES_F32:
      gemm_bf16_kernel<XM, GEMM_OUT_BF16_RES_F32><<<grid, kThreads, 0, s>>>(a);
      break;
    case GEMM_OUT_F32_RES_BF16:
      gemm_bf16_kernel<XM, GEMM_OUT_F32_RES_BF16><<<grid, kThreads, 0, s>>>(a);
      break;
    default: gemm_bf16_kernel<XM, GEMM_OUT_CACHE><<<grid, kThreads, 0, s>>>(a); break;
  }
  return hipGetLastError();
}
}  // namespace

int gemm_ntiles(int N) { return (N + BN - 1) / BN; }

hipError_t launch_gemm_bf16(const GemmArgs &a, hipStream_t s) {
  TraceGuard trace_guard(K_GEMM_BF16, s);
  int tiles = 0;
  for (int i = 0; i < a.nseg; ++i) tiles += gemm_ntiles(a.seg[i].N);
  dim3 grid(tiles, (a.M + BM - 1) / BM);
  if (a.xmode == GEMM_X_SWIGLU) return launch_x<GEMM_X_SWIGLU>(a, grid, s);
  return launch_x<GEMM_X_BF16>(a, grid, s);
}

}  // namespace dl
