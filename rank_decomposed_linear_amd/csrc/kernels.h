// Launchers of the gfx950 kernels (internal to the library; the public
// surface is include/dl.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dl {

// ---------------------------------------------------------------------------
// Weight-streaming bf16 GEMV for small M (decode): out_s[M, N_s] += X_s W_s.
// Up to three segments share M and K; each has its own activations, weight
// and fp32 output. Outputs are accumulated with atomics, so they must hold
// their initial value (zero or a residual) before the launch.
// ---------------------------------------------------------------------------
enum GemvX : int {
  GEMV_X_BF16 = 0,       // X: bf16 [M, K]
  GEMV_X_F32 = 1,        // X: f32 [M, K]
  GEMV_X_SWIGLU_F32 = 2  // X = silu(X) * X2, both f32 [M, K]
};

struct GemvSeg {
  const uint16_t *W;  // [K, N] bf16
  const void *X;      // [M, ldx]
  const float *X2;    // second operand of the SwiGLU prologue
  float *out;         // [M, ldo] f32
  int N, ldx, ldo;
  int strip_begin;    // index of this segment's first 128-column strip
};

struct GemvArgs {
  GemvSeg seg[3];
  int nseg;
  int M, K;
  int xmode;
};

hipError_t launch_gemv_bf16(const GemvArgs &a, int ksplit, hipStream_t s);
int gemv_strips(int N);

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM for large M (prefill): C_s[M, N_s] = X_s[M, K] W_s[K, N_s]
// with a per-launch epilogue. Up to three segments.
// ---------------------------------------------------------------------------
enum GemmX : int {
  GEMM_X_BF16 = 0,     // X bf16 [M, ldx]
  GEMM_X_SWIGLU = 1    // X = silu(X) * X2, both bf16
};
enum GemmOut : int {
  GEMM_OUT_BF16 = 0,        // C bf16 [M, ldc]
  GEMM_OUT_BF16_RES_F32 = 1,// C bf16 = acc + R (f32 [M, ldr]); also C32 (f32) if non-null
  GEMM_OUT_F32_RES_BF16 = 2,// C32 f32 = acc + R (bf16 [M, ldr])
  GEMM_OUT_CACHE = 3        // C bf16 rows scattered: row b*T+t -> cache[b, past[b]+t]
};

struct GemmSeg {
  const uint16_t *W;  // [K, N]
  const uint16_t *X;  // [M, ldx]
  const uint16_t *X2; // SwiGLU partner
  void *C;            // output
  float *C32;         // optional f32 output
  const void *R;      // residual
  int N, ldx, ldc, ldr;
  int tile_begin;     // first N tile of this segment
};

struct GemmArgs {
  GemmSeg seg[3];
  int nseg;
  int M, K;
  int xmode, omode;
  // cache scatter
  const int32_t *past_lens;
  int T, L_max;
};

hipError_t launch_gemm_bf16(const GemmArgs &a, hipStream_t s);
int gemm_ntiles(int N);

// ---------------------------------------------------------------------------
// Attention over the low-rank cache (bf16 MFMA).
// ---------------------------------------------------------------------------
// Rearranges an up factor B[r, n_kv*d] into MFMA operand order:
// packed[g][r/32][d/16][lane][8], lane = 16*grp + c holds
// B[32*rs + 8*grp + e][g*d + 16*blk + c], e = 0..7.
hipError_t launch_pack_up_factor(const uint16_t *B, uint16_t *packed, int r, int n_kv, int d,
                                 hipStream_t s);

struct AttnDecodeArgs {
  const void *q;       // [Bsz, n_q, d] bf16 or f32 (q_f32)
  const uint16_t *ck, *cv;
  const uint16_t *bk_packed, *bv_packed;
  const int32_t *ctx_lens;
  float *part;         // [Bsz, n_q, nsplit, d + 2]
  int Bsz, n_q, n_kv, d, r_k, r_v, L_max;
  int ctx_offset;      // context of sequence b = ctx_lens[b] + ctx_offset
  int nsplit, tiles_per_split;
  float scale_log2;    // sm_scale * log2(e)
  float theta;
  int q_f32;
};
hipError_t launch_attn_decode_bf16(const AttnDecodeArgs &a, hipStream_t s);
// out[b, h, :] from the split partials; out is bf16 (out_f32 = 0) or f32.
hipError_t launch_attn_combine(const float *part, void *out, int Bsz, int n_q, int nsplit, int d,
                               int out_f32, hipStream_t s);

struct AttnPrefillArgs {
  const void *q;       // [Bsz, T, n_q, d] bf16 or f32
  const uint16_t *ck, *cv;
  const uint16_t *bk_packed, *bv_packed;
  const int32_t *past_lens;
  uint16_t *out;       // [Bsz, T, n_q*d]
  int Bsz, T, n_q, n_kv, d, r_k, r_v, L_max;
  int ldq;             // elements between consecutive tokens of q
  int q_f32;           // q is f32 instead of bf16
  float scale_log2;
  float theta;
};
hipError_t launch_attn_prefill_bf16(const AttnPrefillArgs &a, hipStream_t s);

// ---------------------------------------------------------------------------
// fp32 path (plain VALU kernels; every shape).
// ---------------------------------------------------------------------------
enum F32Out : int {
  F32_OUT_STORE = 0,     // C = acc
  F32_OUT_RESID = 1,     // C = acc + R
  F32_OUT_CACHE = 2      // row b*T+t -> cache[b, past[b]+t]
};
struct GemmF32Args {
  const float *X, *X2;   // X2 non-null: X = silu(X) * X2
  const float *W;
  float *C;
  const float *R;
  int M, N, K, ldx, ldc, ldr;
  int omode;
  const int32_t *past_lens;
  int T, L_max;
};
hipError_t launch_gemm_f32(const GemmF32Args &a, hipStream_t s);

struct AttnF32Args {
  const float *q;      // [Bsz, T, n_q, d], token stride ldq
  const float *ck, *cv, *bk, *bv;
  const int32_t *lens; // decode: ctx_lens; prefill: past_lens
  float *out;          // [Bsz, T, n_q*d]
  int decode;          // 1: query position lens[b]-1 (T == 1)
  int Bsz, T, n_q, n_kv, d, r_k, r_v, L_max, ldq;
  float sm_scale, theta;
};
hipError_t launch_attn_f32(const AttnF32Args &a, hipStream_t s);

// ---------------------------------------------------------------------------
// Elementwise helpers.
// ---------------------------------------------------------------------------
// y[M, n] = x / rms(x) * gamma; x and y are bf16 or f32 (flags), gamma is
// in the storage dtype of the layer (gamma_f32) or NULL.
hipError_t launch_rmsnorm(const void *x, int x_f32, const void *gamma, int gamma_f32, void *y,
                          int y_f32, int M, int n, float eps, hipStream_t s);
// Up to four f32 regions: region i gets zero (src == NULL) or a copy of a
// bf16 source (src_bf16 != NULL) or an f32 source.
struct FillRegion {
  float *dst;
  const void *src;
  int src_bf16;
  int64_t n;
};
hipError_t launch_fill(const FillRegion *r, int nreg, hipStream_t s);
// dst (bf16 or f32) = src f32
hipError_t launch_convert_f32(const float *src, void *dst, int dst_bf16, int64_t n, hipStream_t s);
// cache[b, past[b] + t, :] = row b*T + t of an f32 [Bsz*T, ld] matrix
// (columns [0, r)), converted to the cache dtype.
hipError_t launch_store_cache_rows(const float *src, int ld, void *cache, int cache_bf16,
                                   const int32_t *past, int Bsz, int T, int r, int L_max,
                                   hipStream_t s);

}  // namespace dl
