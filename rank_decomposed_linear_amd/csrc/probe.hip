// Matrix-pipe rate probe: the measured denominator next to the published
// bf16 MFMA peak in roofline reports. Workgroups of eight waves (two per
// SIMD, as the GEMM runs); every round, each wave reads twelve 1 KB operand
// fragments from LDS (eight A, four B; the fragments rotate from round to
// round, so the operand data keeps changing) and issues 32 independent
// v_mfma_f32_16x16x32_bf16 into an 8 x 4 block of accumulators, the GEMM's
// own mix. The LDS holds random bf16 values (hashed from the index,
// magnitudes near one): constant operands let the matrix pipe run at a
// higher clock than real data does. Fewer accumulator chains per wave
// (eight instead of 32) measured about a third lower on MI355X, so the rate
// depends on the mix; this one is the GEMM's.
#include "common.h"
#include "kernels.h"

namespace dl {

namespace {
constexpr int kProbeThreads = 512;
constexpr int kProbeFrags = 32;   // 1 KB fragments in LDS

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float *sink, int iters) {
  __shared__ u32x4 lds[kProbeFrags * 64];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // bf16 pairs with random mantissas and signs and exponents of 0.5 .. 1
  auto rnd = [](uint32_t k) {
    uint32_t h = k * 0x9E3779B1u;
    h ^= h >> 15;
    h *= 0x85EBCA77u;
    h ^= h >> 13;
    return (h & 0x807f807fu) | 0x3f003f00u;
  };
  for (uint32_t i = tid; i < kProbeFrags * 64; i += kProbeThreads)
    lds[i] = u32x4{rnd(4 * i), rnd(4 * i + 1), rnd(4 * i + 2), rnd(4 * i + 3)};
  __syncthreads();
  f32x4 acc[8][4];
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
    const uint32_t fb = (it + wave) & 15;
    u32x4 ar[8], bq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) bq[q] = lds[((fb + 16 + q) & 31) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) ar[i] = lds[((fb + i) & 31) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][q] = mfma_bf16(ar[i], bq[q], acc[i][q]);
  }
  float s = 0.f;
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) s += acc[x][y][0] + acc[x][y][1] + acc[x][y][2] + acc[x][y][3];
  sink[static_cast<size_t>(blockIdx.x) * kProbeThreads + tid] = s;
}
}  // namespace

hipError_t launch_mfma_probe(float *sink, int blocks, int iters, hipStream_t s) {
  mfma_probe_kernel<<<blocks, kProbeThreads, 0, s>>>(sink, iters);
  return hipGetLastError();
}

}  // namespace dl
