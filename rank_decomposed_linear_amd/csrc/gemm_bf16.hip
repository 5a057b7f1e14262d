// bf16 MFMA GEMM for prefill-sized M: one factor of a decomposed projection
// (W ~ A B, DeInfer section 2.1, Eq. (1)), C = X W with f32 accumulation.
//
// Both factors are stored transposed (Wt[N, K]) in 16 x 32 operand tiles
// (1 KB, MFMA lane order): the weight block of a workgroup's k step is
// sixteen such tiles, copied to LDS with contiguous 16-byte loads and read
// back one 16-byte ds_read per lane and fragment. The activation rows are
// staged as 16-byte chunks with an XOR swizzle, so their operand reads are
// conflict-free too.
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
constexpr int kBElems = BN * BK;          // bf16 elements of one weight tile

struct Stage {
  u32x4 a[4], b[4];
};

template <int OM>
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

  // Thread t stages 16-byte chunk (row (t + 256 it) / 8, column chunk t % 8)
  // of both tiles, it = 0..3.
  const int kc = tid & 7, r0 = tid >> 3;

  // weight unit u = tid + 256 it (16 bytes): tile T = u / 64 = 2 nb + ks,
  // lane u % 64; tiles (nb, 0) and (nb, 1) are adjacent in memory
  auto gload = [&](Stage &st, int k0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = m0 + r0 + 32 * it;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < a.M) {
        const size_t off = static_cast<size_t>(row) * sg.ldx + k0 + 8 * kc;
        v = *reinterpret_cast<const u32x4 *>(sg.X + off);
      }
      st.a[it] = v;
      const int u = tid + 256 * it, tt = u >> 6, nb = tt >> 1, ks = tt & 1;
      st.b[it] = n0 + 16 * nb < sg.N
                     ? *reinterpret_cast<const u32x4 *>(sg.W + frag_off((n0 >> 4) + nb, (k0 >> 5) + ks, a.K, u & 63))
                     : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](const Stage &st, int buf) {
    uint16_t *base = lds[buf];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = r0 + 32 * it;
      const int chunk = kc ^ (row & 7);
      *reinterpret_cast<u32x4 *>(base + row * BK + chunk * 8) = st.a[it];
      *reinterpret_cast<u32x4 *>(base + kAElems + (tid + 256 * it) * 8) = st.b[it];
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
      for (int nb = 0; nb < 4; ++nb)
        bfr[nb] = *reinterpret_cast<const u32x4 *>(base + kAElems + (((wn * 4 + nb) * 2 + ks) * 64 + lane) * 8);
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
      if constexpr (OM == GEMM_OUT_CACHE || OM == GEMM_OUT_CACHE_T) {
        // key cache tiled [L_max, N] / value cache tiled [N, L_max], per sequence
        const int b = m / a.T, pos = a.past_lens[b] + (m - b * a.T);
        uint16_t *seq = static_cast<uint16_t *>(sg.C) + static_cast<size_t>(b) * sg.N * a.L_max;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int n = n0 + wn * 64 + nb * 16 + j;
          if (n < sg.N)
            seq[OM == GEMM_OUT_CACHE ? tile_off(pos, n, sg.N) : tile_off(n, pos, a.L_max)] =
                f2bf(acc[mb][nb][r]);
        }
        continue;
      }
      const size_t rowoff = static_cast<size_t>(m) * sg.ldc;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int n = n0 + wn * 64 + nb * 16 + j;
        if (n >= sg.N) continue;
        float v = acc[mb][nb][r];
        if constexpr (OM == GEMM_OUT_BF16) {
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

hipError_t launch_o(const GemmArgs &a, dim3 grid, hipStream_t s) {
  switch (a.omode) {
    case GEMM_OUT_BF16: gemm_bf16_kernel<GEMM_OUT_BF16><<<grid, kThreads, 0, s>>>(a); break;
    case GEMM_OUT_BF16_RES_F32: gemm_bf16_kernel<GEMM_OUT_BF16_RES_F32><<<grid, kThreads, 0, s>>>(a); break;
    case GEMM_OUT_F32_RES_BF16: gemm_bf16_kernel<GEMM_OUT_F32_RES_BF16><<<grid, kThreads, 0, s>>>(a); break;
    case GEMM_OUT_CACHE: gemm_bf16_kernel<GEMM_OUT_CACHE><<<grid, kThreads, 0, s>>>(a); break;
    default: gemm_bf16_kernel<GEMM_OUT_CACHE_T><<<grid, kThreads, 0, s>>>(a); break;
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
  return launch_o(a, grid, s);
}

}  // namespace dl
