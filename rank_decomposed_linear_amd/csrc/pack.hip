// Storage conversion between the row-major form of the factors and caches
// (W ~ A B with A [m, k], B [k, n]; latent caches [Bsz, L_max, r]) and the
// library's layouts: transposed factors and cache pages, in 16 x 32 operand
// tiles for bf16 (tile_off in common.h). One-time data movement: every
// thread handles one 16-byte chunk (eight bf16) of the tiled side, whose
// lanes read or write 16 consecutive rows of one column, so each of the
// eight element accesses is coalesced over 16 lanes.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace dl {

namespace {

// chunk u of an operand-tiled [R, C] matrix -> its row and first column
// (the chunk holds columns c .. c + 7 of row r)
__device__ __forceinline__ void chunk_rc(size_t u, int C, int &r, int &c) {
  const size_t tile = u >> 6;
  const int l = static_cast<int>(u & 63);
  const int tr = static_cast<int>(tile / (C >> 5)), tc = static_cast<int>(tile % (C >> 5));
  r = 16 * tr + (l & 15);
  c = 32 * tc + 8 * (l >> 4);
}

// out = F^T in operand tiles: F [rows, cols] row-major bf16, F^T [cols, rows]
__global__ __launch_bounds__(256) void pack_factor_kernel(const uint16_t *F, int rows, int cols,
                                                         uint16_t *out) {
  const size_t n = static_cast<size_t>(rows) * cols / 8;
  for (size_t u = blockIdx.x * 256ull + threadIdx.x; u < n; u += gridDim.x * 256ull) {
    int r, c;   // row r of F^T = column r of F; columns c .. c + 7 of F^T = rows of F
    chunk_rc(u, rows, r, c);
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = F[static_cast<size_t>(c + e) * cols + r];
    *reinterpret_cast<u32x4 *>(out + 8 * u) =
        u32x4{v[0] | (uint32_t(v[1]) << 16), v[2] | (uint32_t(v[3]) << 16),
              v[4] | (uint32_t(v[5]) << 16), v[6] | (uint32_t(v[7]) << 16)};
  }
}

// One sequence-major cache [Bsz, L_max, r] (row-major) <-> library pages.
// Key pages hold [kPage, r] tiles (positions are rows), value pages hold
// [r, kPage] tiles (rank components are rows). unpack = 1 copies the other
// way. Chunk u runs over every page of every sequence.
__global__ __launch_bounds__(256) void pack_cache_kernel(const uint16_t *src, uint16_t *dst, int Bsz,
                                                        int L_max, int r, int value, int unpack) {
  const size_t page_elems = static_cast<size_t>(kPage) * r;
  const size_t n = static_cast<size_t>(Bsz) * L_max * r / 8;
  for (size_t u = blockIdx.x * 256ull + threadIdx.x; u < n; u += gridDim.x * 256ull) {
    const size_t page = (8 * u) / page_elems;          // = b * (L_max / kPage) + p
    const size_t in_page = u - page * (page_elems / 8);
    int tr, tc;
    chunk_rc(in_page, value ? kPage : r, tr, tc);
    // row-major element (position, rank) of sequence-major storage; pages
    // of one sequence are consecutive, so page * kPage is b * L_max + 64 p
    const size_t pos0 = page * kPage;
    uint16_t *tiled = (unpack ? const_cast<uint16_t *>(src) : dst) + 8 * u;
    if (!value) {
      // chunk = key latents (position pos0 + tr, ranks tc .. tc + 7): contiguous in both
      const size_t rm = (pos0 + tr) * r + tc;
      if (unpack)
        *reinterpret_cast<u32x4 *>(dst + rm) = *reinterpret_cast<const u32x4 *>(tiled);
      else
        *reinterpret_cast<u32x4 *>(dst + 8 * u) = *reinterpret_cast<const u32x4 *>(src + rm);
    } else {
      // chunk = value latents (rank tr, positions pos0 + tc .. + 7): strided rows
      if (unpack) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(tiled);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          dst[(pos0 + tc + e) * r + tr] = static_cast<uint16_t>((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
      } else {
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = src[(pos0 + tc + e) * r + tr];
        *reinterpret_cast<u32x4 *>(dst + 8 * u) =
            u32x4{v[0] | (uint32_t(v[1]) << 16), v[2] | (uint32_t(v[3]) << 16),
                  v[4] | (uint32_t(v[5]) << 16), v[6] | (uint32_t(v[7]) << 16)};
      }
    }
  }
}

// float32 [batch][R][C] -> [batch][C][R] (out[b][c][r] = in[b][r][c]); with
// R = 0 a plain copy of batch * C elements
__global__ __launch_bounds__(256) void transpose_f32_kernel(const float *in, float *out, int batch,
                                                           int R, int C) {
  const size_t n = static_cast<size_t>(batch) * (R ? R : 1) * C;
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += gridDim.x * 256ull) {
    if (!R) {
      out[i] = in[i];
      continue;
    }
    // i indexes the output [b][c][r]
    const size_t rc = static_cast<size_t>(R) * C;
    const size_t b = i / rc, rem = i - b * rc;
    const size_t c = rem / R, r = rem - c * R;
    out[i] = in[b * rc + r * C + c];
  }
}

int grid_for(size_t work) {
  return static_cast<int>(std::min<size_t>((work + 255) / 256, 8192));
}

}  // namespace

hipError_t launch_pack_factor(const void *F, int rows, int cols, int bf16, void *out, hipStream_t s) {
  TraceGuard trace_guard(K_CONVERT, s);
  if (bf16)
    pack_factor_kernel<<<grid_for(static_cast<size_t>(rows) * cols / 8), 256, 0, s>>>(
        static_cast<const uint16_t *>(F), rows, cols, static_cast<uint16_t *>(out));
  else
    transpose_f32_kernel<<<grid_for(static_cast<size_t>(rows) * cols), 256, 0, s>>>(
        static_cast<const float *>(F), static_cast<float *>(out), 1, rows, cols);
  return hipGetLastError();
}

hipError_t launch_pack_cache(const void *src, void *dst, int Bsz, int L_max, int r, int value,
                             int unpack, int bf16, hipStream_t s) {
  TraceGuard trace_guard(K_CONVERT, s);
  if (bf16) {
    pack_cache_kernel<<<grid_for(static_cast<size_t>(Bsz) * L_max * r / 8), 256, 0, s>>>(
        static_cast<const uint16_t *>(src), static_cast<uint16_t *>(dst), Bsz, L_max, r, value, unpack);
  } else if (!value) {
    transpose_f32_kernel<<<grid_for(static_cast<size_t>(Bsz) * L_max * r), 256, 0, s>>>(
        static_cast<const float *>(src), static_cast<float *>(dst), Bsz * L_max, 0, r);
  } else {
    // row-major [Bsz, L_max, r] <-> rank-major [Bsz, r, L_max]
    transpose_f32_kernel<<<grid_for(static_cast<size_t>(Bsz) * L_max * r), 256, 0, s>>>(
        static_cast<const float *>(src), static_cast<float *>(dst), Bsz, unpack ? r : L_max,
        unpack ? L_max : r);
  }
  return hipGetLastError();
}

}  // namespace dl
