// Matrix-pipe issue-rate probe: the measured denominator next to the
// published bf16 MFMA peak in roofline reports. Every wave issues rounds of
// eight independent v_mfma_f32_16x16x32_bf16 (16 x 16 x 32, 16384 flops
// each), so no instruction waits on an earlier result. The operands are
// random bf16 values (hashed from the lane and register index, magnitudes
// near one): constant operands let the matrix pipe run at a higher clock
// than real data does (1.47 against 1.30 PFLOP/s measured on MI355X).
#include "common.h"
#include "kernels.h"

namespace dl {

namespace {
__global__ __launch_bounds__(256) void mfma_probe_kernel(float *sink, int iters) {
  const uint32_t lane = threadIdx.x & 63;
  // bf16 pairs with random mantissas and signs and exponents of 0.5 .. 1
  auto rnd = [&](uint32_t k) {
    uint32_t h = (lane + 64u * k) * 0x9E3779B1u;
    h ^= h >> 15;
    h *= 0x85EBCA77u;
    h ^= h >> 13;
    return (h & 0x807f807fu) | 0x3f003f00u;
  };
  u32x4 a[2], b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a[i] = u32x4{rnd(8 * i), rnd(8 * i + 1), rnd(8 * i + 2), rnd(8 * i + 3)};
    b[i] = u32x4{rnd(8 * i + 4), rnd(8 * i + 5), rnd(8 * i + 6), rnd(8 * i + 7)};
  }
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = mfma_bf16(a[k & 1], b[(k >> 1) & 1], acc[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  sink[static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x] = s;
}
}  // namespace

hipError_t launch_mfma_probe(float *sink, int blocks, int iters, hipStream_t s) {
  mfma_probe_kernel<<<blocks, 256, 0, s>>>(sink, iters);
  return hipGetLastError();
}

}  // namespace dl
