// Matrix-pipe issue-rate probe: the measured denominator next to the
// published bf16 MFMA peak in roofline reports. Every wave issues rounds of
// eight independent v_mfma_f32_16x16x32_bf16 (16 x 16 x 32, 16384 flops
// each), so no instruction waits on an earlier result.
#include "common.h"
#include "kernels.h"

namespace dl {

namespace {
__global__ __launch_bounds__(256) void mfma_probe_kernel(float *sink, int iters) {
  const uint32_t lane = threadIdx.x & 63;
  // small bf16 operands (0x3c00.. ~ 0.0078): accumulators stay finite
  const u32x4 a = {0x3c003c00u + lane, 0x3c013c01u, 0x3c023c02u, 0x3c033c03u};
  const u32x4 b = {0x3c043c04u, 0x3c053c05u + lane, 0x3c063c06u, 0x3c073c07u};
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = mfma_bf16(a, b, acc[k]);
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
