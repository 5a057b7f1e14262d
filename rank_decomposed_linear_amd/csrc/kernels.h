// Launchers of the gfx950 kernels (internal to the library; the public
// surface is include/dl.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dl {

// ---------------------------------------------------------------------------
// Weight-streaming bf16 GEMV for small M (decode), M <= 64:
// out_s = epilogue(X_s[M, K] W_s) for up to three segments that share M
// and K. Every weight is stored transposed, Wt[N, K], in 16 x 32 operand
// tiles (tile_off in common.h). X is row-major bf16 / f32 or operand-tiled
// bf16 ([Mpad, K] with Mpad = M rounded up to 16). Paired launches
// (K2 > 0) have one segment whose two halves (X, W, K) and (X2, W2, K2)
// produce two results for the same output columns, combined by the SwiGLU
// epilogue.
// ---------------------------------------------------------------------------
enum GvOut : int {
  GV_OUT_BF16 = 0,      // out bf16 [m * ldo + n] = v
  GV_OUT_F32 = 1,       // out f32 [m * ldo + n] = v
  GV_OUT_CACHE = 2,     // key cache page of sequence b = m / T, position past[b] + t
  GV_OUT_CACHE_T = 6,   // value cache page of sequence b, position past[b] + t
  GV_OUT_TILED = 7,     // out bf16 operand tiles [Mpad, N]
  GV_OUT_RES_F32 = 3,   // out f32 = v + R (R f32 if res_f32, else bf16); out2 gets a copy
  GV_OUT_RES_BF16 = 4,  // out bf16 = v + R (R f32)
  GV_OUT_SWIGLU = 5,    // paired: out bf16 = silu(v_first) * v_second
  GV_OUT_SWIGLU_TILED = 8, // paired, stored as operand tiles [Mpad, N]
  GV_OUT_RELU_TILED = 9    // out bf16 operand tiles [Mpad, N] = max(v, 0)
};

struct GvSeg {
  const uint16_t *W;   // Wt [N, K] bf16, operand tiles
  const uint16_t *W2;  // paired: second half Wt2 [N, K2]
  const void *X;       // bf16 [M, ldx]; tiled: [Mpad, K] operand tiles, ldx = K
  const void *X2;      // paired: second-half activations, like X with K2
  void *out;
  float *out2;         // optional copy (GV_OUT_RES_F32)
  // GV_OUT_RES_F32, optional: the next RMSNorm's input, gamma * out as bf16
  // operand tiles [Mpad, N] (gamma [N] or NULL = 1), and the sum of squares
  // of out over each 16-column tile, ssq_out[m * (N / 16) + n / 16]
  uint16_t *out_nt;
  const void *gamma;
  int gamma_f32;
  float *ssq_out;
  const void *R;       // residual [M, ldr]
  int N, ldx, ldx2, ldo, ldr;
  int omode, res_f32;
  int tile_begin;      // first work item of the segment, set by gemv_plan
};

struct GvArgs {
  GvSeg seg[3];
  int nseg;
  int M, K, K2;           // K2 > 0 only for paired launches (then nseg == 1)
  int x_tiled;            // X (and X2) are operand-tiled
  // optional RMSNorm row scale: rows of the result are multiplied by
  // 1 / sqrt(sum_c rs_part[m * rs_cols + c] / K + eps) (X holds gamma * x;
  // rs_part the per-tile row sums of squares of x, from GV_OUT_RES_F32)
  const float *rs_part;
  int rs_cols;
  float eps;
  const int32_t *past;    // cache scatter (GV_OUT_CACHE / _T)
  int T;
  const int32_t *block_table;  // cache pages (cache_page in common.h); NULL: contiguous
  int page_stride;             // table row length (contiguous: L_max / kPage)
  // set by gemv_plan / the caller
  int ntiles, ksplit, split_steps;   // ntiles: work items (groups of rtiles tiles) per split
  int rtiles;             // 16-row tiles per work item (1, 2 or 4)
  int waves;              // waves per workgroup (4 or 8)
  float *part;            // gemv_plan's return value in floats
  int *counters;          // ntiles ints, zero before the launch (left zero after it)
};

// Chooses the K split and tile numbering; returns the partial-sum floats
// the launch needs (0 when there is no split).
size_t gemv_plan(GvArgs &a);
hipError_t launch_gemv(const GvArgs &a, hipStream_t s);

// A chain of GEMV stages in one persistent launch (stage s + 1 reads what
// stage s writes): every stage planned by gemv_plan, with its own part /
// counters; stages after the first read operand-tiled activations; all
// stages share M. sync points to kChainSyncInts ints that must be zero on
// entry, one counter per 256-byte line: the work is dealt to kChainQueues
// queues (workgroup b serves queue b % kChainQueues), each with its own
// ticket counter [kSyncStride * q] and done counter per stage
// [kSyncStride * (kChainQueues + s * kChainQueues + q)], so no counter is
// hit by more than a queue's workgroups; [kSyncStride * (kChainQueues * (1 +
// kMaxChain))] is set if a wait timed out (the affected outputs are NaN).
constexpr int kMaxChain = 6;
constexpr int kChainQueues = 32;
constexpr int kSyncStride = 64;
constexpr int kChainSyncInts = kSyncStride * (kChainQueues * (1 + kMaxChain) + 1);
struct GvChain {
  GvArgs st[kMaxChain];
  int nst;
  int *sync;
};
hipError_t launch_gemv_chain(const GvChain &c, hipStream_t s);

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM for large M (prefill): C_s[M, N_s] = X_s[M, K] W_s with
// W_s stored transposed, Wt[N_s, K] row-major; per-launch epilogue. Up to
// three segments.
// ---------------------------------------------------------------------------
enum GemmX : int {
  GEMM_X_BF16 = 0,     // X bf16 [M, ldx]
  GEMM_X_TILED = 1     // X bf16 operand tiles [M rounded up to 16, ldx = K]: each 16-row, 32-k
                       // fragment is one contiguous 1 KB (rows past M are read, never stored)
};
enum GemmOut : int {
  GEMM_OUT_BF16 = 0,        // C bf16 [M, ldc]
  GEMM_OUT_BF16_RES_F32 = 1,// C bf16 = acc + R (f32 [M, ldr]); also C32 (f32) if non-null
  GEMM_OUT_F32_RES_BF16 = 2,// C32 f32 = acc + R (bf16 [M, ldr])
  GEMM_OUT_CACHE = 3,       // key cache: row b*T+t -> sequence b, position past[b]+t
  GEMM_OUT_CACHE_T = 4,     // value cache: row b*T+t, column n -> sequence b, (position past[b]+t, rank n)
  GEMM_OUT_SWIGLU = 5,      // C bf16 = silu(R) * acc, R bf16 [M, ldr] (the gate values; C may be R)
  GEMM_OUT_RELU = 6         // C bf16 = max(acc, 0)
};

struct GemmSeg {
  const uint16_t *W;  // Wt [N, K], operand tiles
  const uint16_t *X;  // [M, ldx]
  void *C;            // output
  float *C32;         // optional f32 output
  const void *R;      // residual
  int N, ldx, ldc, ldr;
  int omode;          // GemmOut of this segment
  int tile_begin;     // first N tile of this segment (set by the launcher)
  int c_tiled;        // bf16 C stored as operand tiles [M rounded up to 16, ldc]
  int r_tiled;        // bf16 R read from operand tiles [M rounded up to 16, ldr]
};

struct GemmArgs {
  GemmSeg seg[3];
  int nseg;
  int M, K;           // K % 64 == 0; every segment's N % 16 == 0
  int xmode, omode;   // omode: default for segments whose own omode is < 0
  // cache scatter
  const int32_t *past_lens;
  int T;
  const int32_t *block_table;  // cache pages; NULL: contiguous
  int page_stride;
  int tiles_m, tiles_n;  // set by the launcher
  // Remainder split: f32 partial tiles of the split units (NULL: no split).
  // The launcher splits the k range of the tiles of an underfilled last
  // round when gemm_part_bytes() of the shape is nonzero and fits.
  float *part;
  size_t part_bytes;
  int full, split;       // set by the launcher: tiles run whole, parts per split tile
};

// Sets the segments' tile_begin and the tile counts, then launches (the
// GEMM, and the fixup that sums split tiles' partials when it splits).
hipError_t launch_gemm_bf16(GemmArgs &a, hipStream_t s);
int gemm_ntiles(int N);
// Partial-tile bytes the launcher needs to split a GEMM of M rows,
// ntiles_n column tiles (the sum over segments of gemm_ntiles) and depth K
// on the current device; 0 when it runs unsplit.
size_t gemm_part_bytes(int M, int ntiles_n, int K);

// ---------------------------------------------------------------------------
// Attention over the low-rank cache (bf16 MFMA).
// ---------------------------------------------------------------------------
struct AttnDecodeArgs {
  const void *q;       // [Bsz, n_q, d] bf16 or f32 (q_f32)
  const uint16_t *ck;  // key cache pool (pages of [kPage, r_k] operand tiles)
  const uint16_t *cv;  // value cache pool (pages of [r_v, kPage] operand tiles)
  const int32_t *block_table;  // NULL: contiguous, page_stride pages per sequence
  int page_stride;
  const uint16_t *bk, *bv;  // up factors, [n_kv * d, r] in operand tiles
  const int32_t *ctx_lens;
  void *out;           // [Bsz, n_q, d] bf16 (or f32 with out_f32); out_tiled: bf16
                       // operand tiles of the [Bsz (padded to 16), n_q * d] matrix
  float *part;         // [Bsz, n_kv, nsplit, 16, d + 2] split partials (nsplit > 1)
  int *counters;       // [Bsz * n_kv], zero on entry, left zero
  int Bsz, n_q, n_kv, d, r_k, r_v, L_max;
  int ctx_offset;      // context of sequence b = ctx_lens[b] + ctx_offset
  int nsplit, split_len;  // context positions per split (multiple of attn_decode_split_granule())
  // set by the launcher (LDS plan)
  int rs_cap, rs_tail;    // rank steps resident for the whole item; steps per restaged tail chunk (0: none)
  int pitch, lds_bs, lds_s;
  int vpasses;         // value-side passes (set by the launcher)
  float *uglob;        // [Bsz, n_kv, nsplit, 16, r_v] f32 when passes > 1
  float scale_log2;    // sm_scale * log2(e)
  float theta;
  int q_f32, out_f32, out_tiled;
};
// Decode attention in the latent space (rotary embedding off): Q~ = B_k q,
// S = C_k Q~, U = softmax(S) C_v, o = U B_v (three launches).
struct LatentAttnArgs {
  const void *q;       // [Bsz, n_q, d] bf16 or f32 (q_f32)
  const uint16_t *ck, *cv;        // cache pools (pages, as AttnDecodeArgs)
  const int32_t *block_table;     // NULL: contiguous, page_stride pages per sequence
  int page_stride;
  const uint16_t *bk, *bv;        // up factors, [n_kv * d, r] in operand tiles
  const int32_t *ctx_lens;
  void *out;           // [Bsz, n_q, d] bf16 (f32 with out_f32; operand tiles with out_tiled)
  uint16_t *qt;        // workspace [Bsz, ngroups, 16, r_k] bf16 operand tiles (Q~, scaled)
  uint16_t *u;         // workspace [Bsz, n_q, r_v] bf16 (U / l)
  float *part;         // workspace [Bsz, ngroups, nsplit, 16, r_v + 2] (nsplit > 1)
  int *counters;       // [Bsz * ngroups], zero on entry, left zero
  int Bsz, n_q, n_kv, d, r_k, r_v, L_max;
  int ctx_offset;
  int ngroups, nsplit, split_len;
  int pitch, lds_q, lds_s;   // set by the launcher
  float scale_log2;
  int q_f32, out_f32, out_tiled;
};
// longest context split one latent-attention workgroup holds (0: r_k too large)
int latent_attn_max_split(int r_k);
hipError_t launch_latent_attn_bf16(LatentAttnArgs a, hipStream_t s);

int attn_decode_split_granule();
// value-side passes of the decode kernel for r_v (more than one keeps U in
// the workspace between context chunks)
int attn_decode_value_passes(int r_v);
hipError_t launch_attn_decode_bf16(const AttnDecodeArgs &a, hipStream_t s);

struct AttnPrefillArgs {
  const void *q;       // [Bsz, T, n_q, d] bf16 or f32
  const uint16_t *ck;  // key cache pool (pages of [kPage, r_k] operand tiles)
  const uint16_t *cv;  // value cache pool (pages of [r_v, kPage] operand tiles)
  const int32_t *block_table;  // NULL: contiguous, page_stride pages per sequence
  int page_stride;
  int64_t pool_pages;  // pages in each pool (bounds the 32-bit buffer offsets)
  const uint16_t *bk, *bv;  // [n_kv * d, r] in operand tiles
  const int32_t *past_lens;
  uint16_t *out;       // [Bsz, T, n_q*d]; out_tiled: operand tiles [Bsz*T rounded up to 16, n_q*d]
  int out_tiled;
  uint16_t *kv;        // workspace: rebuilt key tiles, [Bsz, n_kv, L_max / 64, 2 * 64 * d]
                       // (per 64-key tile: K rows rotated and swizzled, then V^T rows)
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
  F32_OUT_CACHE = 2,     // row b*T+t -> cache[b, past[b]+t]
  F32_OUT_CACHE_T = 3,   // row b*T+t, column n -> cache[b, n, past[b]+t]
  F32_OUT_RELU = 4       // C = max(acc, 0)
};
struct GemmF32Args {
  const float *X, *X2;   // X2 non-null: X = silu(X) * X2
  const float *W;        // Wt [N, K]
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
  const float *ck;     // [Bsz, L_max, r_k]
  const float *cv;     // [Bsz, r_v, L_max]
  const float *bk, *bv;  // [n_kv * d, r]
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
// y[M, n] = x / rms(x) * gamma; x is bf16 or f32 (flag); y is bf16 (y_mode
// RMS_Y_BF16), f32 (RMS_Y_F32) or bf16 operand tiles [M rounded up to 16, n]
// (RMS_Y_TILED, n % 8 == 0); gamma is in the storage dtype of the layer
// (gamma_f32) or NULL.
enum RmsY : int { RMS_Y_BF16 = 0, RMS_Y_F32 = 1, RMS_Y_TILED = 2 };
hipError_t launch_rmsnorm(const void *x, int x_f32, const void *gamma, int gamma_f32, void *y,
                          int y_mode, int M, int n, float eps, hipStream_t s);
// Up to four f32 regions: region i gets zero (src == NULL) or a copy of a
// bf16 source (src_bf16 != NULL) or an f32 source. With tile_cols > 0 the
// region is instead a bf16 operand-tile copy: src bf16 row-major
// [tile_rows, tile_cols] -> dst bf16 tiles [tile_rows rounded up to 16,
// tile_cols], padding rows zero; n counts 16-byte chunks of dst.
struct FillRegion {
  float *dst;
  const void *src;
  int src_bf16;
  int64_t n;
  int tile_rows = 0, tile_cols = 0;
};
hipError_t launch_fill(const FillRegion *r, int nreg, hipStream_t s);
// RMSNorm into operand tiles: xt [Mp, n] bf16 tiles, row m < M =
// x[m] / sqrt(mean(x[m]^2) + eps) * gamma (x bf16 [M, n], gamma [n] or NULL),
// rows M .. Mp - 1 zero; the same launch zeroes up to four fill regions.
hipError_t launch_norm_tiles(const uint16_t *x, const void *gamma, int gamma_f32, float eps,
                             uint16_t *xt, int M, int Mp, int n, const FillRegion *zero, int nzero,
                             hipStream_t s);
// Matrix-pipe issue-rate probe (dl_probe_mfma_bf16)
hipError_t launch_mfma_probe(float *sink, int blocks, int iters, hipStream_t s);

// Storage conversion (pack.hip). Factor: F [rows, cols] row-major -> F^T
// (bf16 operand tiles: rows % 32 == 0, cols % 16 == 0). Cache: one cache
// [Bsz, L_max, r] row-major <-> library pages (bf16: L_max % kPage == 0,
// r % 32 == 0); value = 1 for the value cache, unpack = 1 for the inverse.
hipError_t launch_pack_factor(const void *F, int rows, int cols, int bf16, void *out, hipStream_t s);
hipError_t launch_pack_cache(const void *src, void *dst, int Bsz, int L_max, int r, int value,
                             int unpack, int bf16, hipStream_t s);

// dst (bf16 or f32) = src f32
hipError_t launch_convert_f32(const float *src, void *dst, int dst_bf16, int64_t n, hipStream_t s);

}  // namespace dl
