// Small memory-bound helpers of the layer: RMSNorm, accumulator
// initialisation (fills and copies) and float32 -> storage conversion.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace dl {

namespace {

__device__ __forceinline__ float load_elem(const void *p, int is_f32, size_t i) {
  return is_f32 ? static_cast<const float *>(p)[i] : bf2f(static_cast<const uint16_t *>(p)[i]);
}

// One workgroup per row: y = x / sqrt(mean(x^2) + eps) * gamma.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void *x, int x_f32, const void *gamma,
                                                      int gamma_f32, void *y, int y_f32, int n,
                                                      float eps) {
  __shared__ float part[4];
  const size_t row = blockIdx.x;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) {
    const float v = load_elem(x, x_f32, row * n + i);
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float rstd = 1.0f / sqrtf(tot / n + eps);
  for (int i = threadIdx.x; i < n; i += 256) {
    float v = load_elem(x, x_f32, row * n + i) * rstd;
    if (gamma) v *= load_elem(gamma, gamma_f32, i);
    if (y_f32)
      static_cast<float *>(y)[row * n + i] = v;
    else
      static_cast<uint16_t *>(y)[row * n + i] = f2bf(v);
  }
}

// Same result for rows of n % 8 == 0 with 16-byte aligned bases: 16-byte
// accesses, the first kNormCache chunks of 8 per thread kept in registers
// (one read of x for rows up to 256 * 8 * kNormCache elements).
constexpr int kNormCache = 8;

__device__ __forceinline__ void load8(const void *p, int f32, size_t i, float v[8]) {
  if (f32) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(p) + i);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(p) + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p) + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bflo(w[q]);
      v[2 * q + 1] = bfhi(w[q]);
    }
  }
}

// Row of workgroup `bid` among M: the hardware deals workgroups to the
// eight XCDs round-robin; XCD x takes a contiguous range of rows, so the 16
// rows of an operand tile are written through one L2 (a bijection).
__device__ __forceinline__ int xcd_row(int bid, int M) {
  const int xcd = bid & 7, local = bid >> 3, q = M >> 3, rem = M & 7;
  return xcd < rem ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
}

__global__ __launch_bounds__(256) void rmsnorm_vec_kernel(const void *x, int x_f32, const void *gamma,
                                                          int gamma_f32, void *y, int y_mode, int n,
                                                          float eps) {
  __shared__ float part[4];
  const int row = xcd_row(blockIdx.x, gridDim.x);
  const size_t base = static_cast<size_t>(row) * n;
  const int nc = n >> 3;
  float v[kNormCache][8];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kNormCache; ++k) {
    const int c = threadIdx.x + 256 * k;
    if (c < nc) {
      load8(x, x_f32, base + 8 * c, v[k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(v[k][e], v[k][e], ss);
    }
  }
  for (int c = threadIdx.x + 256 * kNormCache; c < nc; c += 256) {
    float t[8];
    load8(x, x_f32, base + 8 * c, t);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(t[e], t[e], ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float rstd = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / n + eps);
  auto emit = [&](int c, float *t) {
    float gm[8];
    if (gamma) load8(gamma, gamma_f32, 8 * static_cast<size_t>(c), gm);
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = t[e] * rstd * (gamma ? gm[e] : 1.f);
    if (y_mode == RMS_Y_F32) {
      float *o = static_cast<float *>(y) + base + 8 * c;
      *reinterpret_cast<f32x4 *>(o) = f32x4{t[0], t[1], t[2], t[3]};
      *reinterpret_cast<f32x4 *>(o + 4) = f32x4{t[4], t[5], t[6], t[7]};
    } else if (y_mode == RMS_Y_TILED) {
      // the eight columns 8c .. 8c + 7 of this row are contiguous in its tile
      *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(y) + tile_off(row, 8 * c, n)) =
          u32x4{pack2(t[0], t[1]), pack2(t[2], t[3]), pack2(t[4], t[5]), pack2(t[6], t[7])};
    } else {
      *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(y) + base + 8 * c) =
          u32x4{pack2(t[0], t[1]), pack2(t[2], t[3]), pack2(t[4], t[5]), pack2(t[6], t[7])};
    }
  };
#pragma unroll
  for (int k = 0; k < kNormCache; ++k) {
    const int c = threadIdx.x + 256 * k;
    if (c < nc) emit(c, v[k]);
  }
  for (int c = threadIdx.x + 256 * kNormCache; c < nc; c += 256) {
    float t[8];
    load8(x, x_f32, base + 8 * c, t);
    emit(c, t);
  }
}

struct FillPack {
  FillRegion r[4];
  int nreg;
};

__global__ void fill_kernel(FillPack p) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int k = 0; k < p.nreg; ++k) {
    const FillRegion &rg = p.r[k];
    if (rg.tile_cols > 0) {
      // chunk i = 8 bf16 of tile i / 64, lane i % 64
      const int cs_n = rg.tile_cols >> 5;
      for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < rg.n;
           i += stride) {
        const int64_t t = i >> 6;
        const int ln = static_cast<int>(i & 63);
        const int r = static_cast<int>(t / cs_n) * 16 + (ln & 15);
        const int c = static_cast<int>(t % cs_n) * 32 + (ln >> 4) * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < rg.tile_rows)
          v = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(rg.src) +
                                               static_cast<size_t>(r) * rg.tile_cols + c);
        reinterpret_cast<u32x4 *>(rg.dst)[i] = v;
      }
      continue;
    }
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < rg.n;
         i += stride) {
      float v = 0.f;
      if (rg.src) v = load_elem(rg.src, !rg.src_bf16, static_cast<size_t>(i));
      rg.dst[i] = v;
    }
  }
}

// Zero the fill regions (src NULL) with the workgroups [b0, gridDim.x).
__device__ void zero_regions(const FillPack &p, int b0) {
  const int64_t stride = static_cast<int64_t>(gridDim.x - b0) * blockDim.x;
  for (int k = 0; k < p.nreg; ++k)
    for (int64_t i = static_cast<int64_t>(blockIdx.x - b0) * blockDim.x + threadIdx.x; i < p.r[k].n;
         i += stride)
      p.r[k].dst[i] = 0.f;
}

// RMSNorm of row m = blockIdx.x < Mp into bf16 operand tiles (rows >= M
// zero); workgroups past Mp zero the fill regions. Eight columns per chunk:
// one 16-byte read of x, one 16-byte write of the tile (columns c .. c + 7
// of a row are contiguous in a tile when c % 8 == 0).
__global__ __launch_bounds__(256) void norm_tiles_kernel(const uint16_t *x, const void *gamma,
                                                         int gamma_f32, float eps, uint16_t *xt,
                                                         int M, int Mp, int n, FillPack z) {
  const int m = blockIdx.x;
  if (m >= Mp) {
    zero_regions(z, Mp);
    return;
  }
  __shared__ float part[4];
  const int nch = n >> 3;
  const uint16_t *row = x + static_cast<size_t>(m) * n;
  // chunks i = threadIdx.x + 256 c stay in registers between the sum of
  // squares and the store (up to kCh per thread; longer rows reread the rest)
  constexpr int kCh = 8;
  u32x4 v[kCh];
  float ss = 0.f;
  auto sumsq = [&](const u32x4 &w) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = bflo(w[q]), hi = bfhi(w[q]);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
  };
#pragma unroll
  for (int c = 0; c < kCh; ++c) {
    const int i = threadIdx.x + 256 * c;
    v[c] = u32x4{0u, 0u, 0u, 0u};
    if (m < M && i < nch) v[c] = *reinterpret_cast<const u32x4 *>(row + 8 * i);
  }
#pragma unroll
  for (int c = 0; c < kCh; ++c) sumsq(v[c]);
  if (m < M)
    for (int i = threadIdx.x + 256 * kCh; i < nch; i += 256) sumsq(*reinterpret_cast<const u32x4 *>(row + 8 * i));
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float rstd = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / n + eps);
  auto store = [&](int i, const u32x4 &w) {
    u32x4 o = {0u, 0u, 0u, 0u};
    if (m < M) {
      float f[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[2 * q] = bflo(w[q]) * rstd;
        f[2 * q + 1] = bfhi(w[q]) * rstd;
      }
      if (gamma) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] *= load_elem(gamma, gamma_f32, 8 * i + e);
      }
      o = u32x4{pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
    }
    *reinterpret_cast<u32x4 *>(xt + tile_off(m, 8 * i, n)) = o;
  };
#pragma unroll
  for (int c = 0; c < kCh; ++c) {
    const int i = threadIdx.x + 256 * c;
    if (i < nch) store(i, v[c]);
  }
  for (int i = threadIdx.x + 256 * kCh; i < nch; i += 256)
    store(i, m < M ? *reinterpret_cast<const u32x4 *>(row + 8 * i) : u32x4{0u, 0u, 0u, 0u});
}

__global__ void convert_kernel(const float *src, void *dst, int dst_bf16, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    if (dst_bf16)
      static_cast<uint16_t *>(dst)[i] = f2bf(src[i]);
    else
      static_cast<float *>(dst)[i] = src[i];
  }
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

}  // namespace

hipError_t launch_rmsnorm(const void *x, int x_f32, const void *gamma, int gamma_f32, void *y,
                          int y_mode, int M, int n, float eps, hipStream_t s) {
  TraceGuard trace_guard(K_RMSNORM, s);
  const auto a16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec = n % 8 == 0 && a16(x) && a16(y) && (!gamma || a16(gamma));
  if (y_mode == RMS_Y_TILED && (!vec || n % 32 != 0)) return hipErrorInvalidValue;
  if (vec)
    rmsnorm_vec_kernel<<<M, 256, 0, s>>>(x, x_f32, gamma, gamma_f32, y, y_mode, n, eps);
  else
    rmsnorm_kernel<<<M, 256, 0, s>>>(x, x_f32, gamma, gamma_f32, y, y_mode, n, eps);
  return hipGetLastError();
}

hipError_t launch_fill(const FillRegion *r, int nreg, hipStream_t s) {
  TraceGuard trace_guard(K_FILL, s);
  FillPack p{};
  int64_t mx = 0;
  for (int i = 0; i < nreg && i < 4; ++i) {
    p.r[i] = r[i];
    if (r[i].n > mx) mx = r[i].n;
  }
  p.nreg = nreg < 4 ? nreg : 4;
  fill_kernel<<<grid_for(mx), 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_norm_tiles(const uint16_t *x, const void *gamma, int gamma_f32, float eps,
                             uint16_t *xt, int M, int Mp, int n, const FillRegion *zero, int nzero,
                             hipStream_t s) {
  TraceGuard trace_guard(K_RMSNORM, s);
  FillPack p{};
  int64_t mx = 0;
  for (int i = 0; i < nzero && i < 4; ++i) {
    p.r[i] = zero[i];
    if (zero[i].n > mx) mx = zero[i].n;
  }
  p.nreg = nzero < 4 ? nzero : 4;
  const int zgrid = p.nreg ? static_cast<int>(std::min<int64_t>((mx + 255) / 256, 64)) : 0;
  norm_tiles_kernel<<<Mp + zgrid, 256, 0, s>>>(x, gamma, gamma_f32, eps, xt, M, Mp, n, p);
  return hipGetLastError();
}

hipError_t launch_convert_f32(const float *src, void *dst, int dst_bf16, int64_t n, hipStream_t s) {
  TraceGuard trace_guard(K_CONVERT, s);
  convert_kernel<<<grid_for(n), 256, 0, s>>>(src, dst, dst_bf16, n);
  return hipGetLastError();
}

}  // namespace dl
