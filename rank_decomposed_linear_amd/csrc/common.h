// Shared device helpers for the gfx950 kernels: bf16 conversion, MFMA
// operand types, warp-level reductions, rotary-angle evaluation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest even, hardware v_cvt_pk_bf16_f32) and
// pack them: `lo` in bits 0..15, `hi` in bits 16..31.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  bf16x2_t v;
  v.x = static_cast<__bf16>(lo);
  v.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).
// Operand registers: lane l holds 8 consecutive-slot values of row/column
// (l % 16) for reduction slots 8*(l/16) .. 8*(l/16)+7. The accumulator lane
// l holds D[4*(l/16) + r][l % 16], r = 0..3.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Operand-tile storage of a bf16 matrix [R][C] (R % 16 == 0, C % 32 == 0):
// 16 x 32 tiles of 1 KB, row-tile major, each in MFMA operand lane order --
// lane l = (r % 16) + 16 * ((c % 32) / 8) holds columns 8 * ((c % 32) / 8)
// .. +7 of row r, at byte 16 * l of the tile. One operand fragment is one
// contiguous 1 KB read.
__device__ __forceinline__ size_t tile_off(int r, int c, int C) {
  return (static_cast<size_t>(r >> 4) * (C >> 5) + (c >> 5)) * 512 +
         ((((c & 31) >> 3) << 4) + (r & 15)) * 8 + (c & 7);
}
// float32 variant (2 KB tiles): the eight columns of a lane are split into
// two 1 KB halves, columns 0..3 of every lane first, so each half of a
// fragment is again one contiguous 1 KB read.
__device__ __forceinline__ size_t tile_off_f32(int r, int c, int C) {
  return (static_cast<size_t>(r >> 4) * (C >> 5) + (c >> 5)) * 512 +
         ((((c & 7) >> 2) << 6) + (((c & 31) >> 3) << 4) + (r & 15)) * 4 + (c & 3);
}
// first element of operand fragment (row block rb, column step cs) of lane l
__device__ __forceinline__ size_t frag_off(int rb, int cs, int C, int lane) {
  return (static_cast<size_t>(rb) * (C >> 5) + cs) * 512 + lane * 8;
}

// Latent caches (bf16) are stored in pages of kPage positions. A key page
// holds [kPage, r_k] in operand tiles (kPage * r_k elements, rows =
// positions); a value page holds [r_v, kPage] in operand tiles (kPage * r_v
// elements, rows = rank components). Logical page p of sequence b is pool
// page table[b * stride + p]; without a table (a contiguous cache) it is
// page b * stride + p.
constexpr int kPage = 64;
__device__ __forceinline__ int cache_page(const int32_t *table, int stride, int b, int p) {
  return table ? table[b * stride + p] : b * stride + p;
}
// The same lookup for a (b, p) that is uniform across the wave, through the
// scalar cache: a vector load here would make the compiler wait for every
// vector load in flight (vmcnt counts in issue order) before the page is
// known, draining any prefetch ring around it; a scalar load waits on
// lgkmcnt instead. The table is read-only while a kernel runs.
__device__ __forceinline__ int cache_page_uniform(const int32_t *table, int stride, int b, int p) {
  const int idx = __builtin_amdgcn_readfirstlane(b * stride + p);
  if (!table) return idx;
  typedef const int32_t __attribute__((address_space(4))) *cptr;
  return __builtin_amdgcn_readfirstlane(((cptr)table)[idx]);
}
// element offsets of key latent (pos, r) and value latent (pos, n) in a pool
// whose position pos lies on pool page `page`
__device__ __forceinline__ size_t key_off(int page, int pos, int r, int r_k) {
  return static_cast<size_t>(page) * (kPage * r_k) + tile_off(pos & (kPage - 1), r, r_k);
}
__device__ __forceinline__ size_t val_off(int page, int pos, int n, int r_v) {
  return static_cast<size_t>(page) * (kPage * r_v) + tile_off(n, pos & (kPage - 1), kPage);
}

// Pack the four accumulator values of two 16x16 blocks into one operand
// register set: slots 0..3 from `x`, 4..7 from `y`.
__device__ __forceinline__ u32x4 pack_acc(f32x4 x, f32x4 y) {
  u32x4 r;
  r.x = pack2(x[0], x[1]);
  r.y = pack2(x[2], x[3]);
  r.z = pack2(y[0], y[1]);
  r.w = pack2(y[2], y[3]);
  return r;
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ __forceinline__ float wave_sum_xor(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Rotary angle pos * w, returned as (cos, sin). `rev` is w / (2*pi) in
// float64; the product is reduced to a fraction of a turn in float64 so the
// float32 evaluation sees an argument in [-pi, pi] regardless of pos.
__device__ __forceinline__ void rope_cs(int pos, double rev, float &c, float &s) {
  double t = static_cast<double>(pos) * rev;
  t -= rint(t);
  const float a = static_cast<float>(t * 6.283185307179586);
  __sincosf(a, &s, &c);
}

__device__ __forceinline__ double rope_rev(int i, int d, float theta) {
  // theta^(-2i/d) / (2*pi)
  return exp(-2.0 * i / d * log(static_cast<double>(theta))) * 0.15915494309189535;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// 2^x by the hardware instruction alone (v_exp_f32): results below the
// normal range flush to zero, which softmax weights may do; exp2f adds a
// range reduction for them (four more instructions per call).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Compile-time loop: f(IntC<0>{}), ..., f(IntC<N - 1>{}), so the index can
// select register arrays and scheduling groups statically.
template <int V>
struct IntC {
  static constexpr int value = V;
};
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(IntC<I>{});
    static_for<N, I + 1>(f);
  }
}

}  // namespace dl
