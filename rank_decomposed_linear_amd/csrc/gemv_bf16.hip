// Weight-streaming factor GEMV for decode-sized M (M <= 64), bf16 MFMA.
//
// One projection factor of a decomposed layer (W ~ A B, DeInfer section 2.1,
// Eq. (1)) applied to a handful of token rows reads every weight once and
// does M multiply-adds per weight: at M = 16 that is 16 flop/byte, above the
// float32 VALU ridge of MI355X (~10 flop/byte without packed math) and far
// below the bf16 MFMA ridge. So the product runs on MFMA with the token rows
// padded to 16, and the kernel is organised to keep HBM busy:
//
//  * A wave owns a strip of 128 output columns. Per 32-row step, lane
//    (c = lane%16, g = lane/16) issues eight 16-byte loads W[k0+8g+s][n0+8c ..
//    n0+8c+7], s = 0..7: each load instruction covers 4 rows x 256
//    contiguous bytes. The eight registers are transposed in-lane into eight
//    B operands (one per column offset 0..7), so no LDS staging is needed
//    for the weights; output column n0 + 8c + e comes out of operand e.
//  * The A operand (token rows, 16 per block) is a single 16-byte load per
//    lane, converted from f32 or passed through the SwiGLU prologue.
//  * Eight waves of a workgroup split the strip's K range; their results are
//    summed in LDS, and workgroups that split K further (grid.y) add their
//    sums into the f32 output with hardware float atomics.
#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace dl {

namespace {
constexpr int kCols = 128;   // output columns per strip
constexpr int kWaves = 8;    // waves per workgroup (all on one strip)
constexpr int kPitch = 132;  // LDS row pitch (floats) of the reduction tile

template <int XM>
__device__ __forceinline__ u32x4 load_x(const GemvSeg &sg, int M, int m, int k) {
  u32x4 r = {0u, 0u, 0u, 0u};
  if (m >= M) return r;
  if constexpr (XM == GEMV_X_BF16) {
    r = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(sg.X) +
                                          static_cast<size_t>(m) * sg.ldx + k);
  } else {
    const float *p = static_cast<const float *>(sg.X) + static_cast<size_t>(m) * sg.ldx + k;
    f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
    if constexpr (XM == GEMV_X_SWIGLU_F32) {
      const float *q = sg.X2 + static_cast<size_t>(m) * sg.ldx + k;
      f32x4 ua = *reinterpret_cast<const f32x4 *>(q);
      f32x4 ub = *reinterpret_cast<const f32x4 *>(q + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = silu(a[i]) * ua[i];
        b[i] = silu(b[i]) * ub[i];
      }
    }
    r.x = pack2(a[0], a[1]);
    r.y = pack2(a[2], a[3]);
    r.z = pack2(b[0], b[1]);
    r.w = pack2(b[2], b[3]);
  }
  return r;
}

// Transpose eight rows x eight bf16 columns held one row per register into
// eight operands holding one column (8 rows) each.
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

template <int MB, int XM>
__global__ __launch_bounds__(kWaves * 64) void gemv_bf16_kernel(GemvArgs a) {
  __shared__ float red[MB * 16 * kPitch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, grp = lane >> 4;

  const int bx = blockIdx.x;
  int si = 0;
  if (a.nseg > 1 && bx >= a.seg[1].strip_begin) si = 1;
  if (a.nseg > 2 && bx >= a.seg[2].strip_begin) si = 2;
  const GemvSeg sg = a.seg[si];
  const int n0 = (bx - sg.strip_begin) * kCols;
  const int col = n0 + 8 * c;
  const bool col_ok = col < sg.N;

  const int ksteps = a.K >> 5;
  const int c0 = static_cast<int>(static_cast<int64_t>(blockIdx.y) * ksteps / gridDim.y);
  const int c1 = static_cast<int>(static_cast<int64_t>(blockIdx.y + 1) * ksteps / gridDim.y);
  const int span = c1 - c0;
  const int s0 = c0 + wave * span / kWaves, s1 = c0 + (wave + 1) * span / kWaves;

  f32x4 acc[MB][8];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[mb][e] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t ldw = static_cast<size_t>(sg.N);
  const uint16_t *wcol = sg.W + col;
  u32x4 cur[8], nxt[8];
  auto load_w = [&](u32x4 (&r)[8], int st) {
    const uint16_t *wp = wcol + static_cast<size_t>(st * 32 + 8 * grp) * ldw;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      r[s] = col_ok ? *reinterpret_cast<const u32x4 *>(wp + s * ldw) : u32x4{0u, 0u, 0u, 0u};
  };
  auto compute = [&](const u32x4 (&r)[8], int st) {
    u32x4 b[8];
    transpose8(r, b);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const u32x4 x = load_x<XM>(sg, a.M, mb * 16 + c, st * 32 + 8 * grp);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[mb][e] = mfma_bf16(x, b[e], acc[mb][e]);
    }
  };

  if (s0 < s1) load_w(cur, s0);
  for (int st = s0; st < s1; st += 2) {
    if (st + 1 < s1) load_w(nxt, st + 1);
    compute(cur, st);
    if (st + 1 < s1) {
      if (st + 2 < s1) load_w(cur, st + 2);
      compute(nxt, st + 1);
    }
  }

  for (int i = threadIdx.x; i < MB * 16 * kPitch; i += blockDim.x) red[i] = 0.f;
  __syncthreads();
  // lane (c, grp) holds D[4*grp + r][c] of operand e = global column 8c + e;
  // LDS column index e*16 + c keeps the 64 lanes on distinct banks.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        atomicAdd(&red[(mb * 16 + 4 * grp + r) * kPitch + e * 16 + c], acc[mb][e][r]);
  __syncthreads();
  for (int i = threadIdx.x; i < MB * 16 * kCols; i += blockDim.x) {
    const int m = i / kCols, cc = i % kCols;
    if (m < a.M && n0 + cc < sg.N)
      unsafeAtomicAdd(sg.out + static_cast<size_t>(m) * sg.ldo + n0 + cc,
                      red[m * kPitch + (cc & 7) * 16 + (cc >> 3)]);
  }
}

template <int MB>
hipError_t launch_mb(const GemvArgs &a, dim3 grid, hipStream_t s) {
  switch (a.xmode) {
    case GEMV_X_BF16: gemv_bf16_kernel<MB, GEMV_X_BF16><<<grid, kWaves * 64, 0, s>>>(a); break;
    case GEMV_X_F32: gemv_bf16_kernel<MB, GEMV_X_F32><<<grid, kWaves * 64, 0, s>>>(a); break;
    default: gemv_bf16_kernel<MB, GEMV_X_SWIGLU_F32><<<grid, kWaves * 64, 0, s>>>(a); break;
  }
  return hipGetLastError();
}
}  // namespace

int gemv_strips(int N) { return (N + kCols - 1) / kCols; }

hipError_t launch_gemv_bf16(const GemvArgs &a, int ksplit, hipStream_t s) {
  TraceGuard trace_guard(K_GEMV_BF16, s);
  int strips = 0;
  for (int i = 0; i < a.nseg; ++i) strips += gemv_strips(a.seg[i].N);
  dim3 grid(strips, ksplit);
  const int mb = (a.M + 15) / 16;
  switch (mb) {
    case 1: return launch_mb<1>(a, grid, s);
    case 2: return launch_mb<2>(a, grid, s);
    case 3: return launch_mb<3>(a, grid, s);
    default: return launch_mb<4>(a, grid, s);
  }
}

}  // namespace dl
