/*
 * dl.h -- C ABI of the decomposed-layer forward pass on one MI355X (gfx950).
 *
 * The method is the one of "DeInfer: Efficient Parallel Inferencing for
 * Decomposed Large Language Models" (Huang, Huang, Liao, Wen; DAC '26):
 *   - section 2.1, Eq. (1): every projection W (m x n) is replaced by a factor
 *     pair A (m x k), B (k x n), W ~ A B, so a row vector maps as
 *     y = (x A) B;
 *   - section 2.1: the low-rank intermediates x A_k and x A_v of the key and
 *     value pairs are stored as the KV cache ("low-rank cache");
 *   - section 4.2: attention rebuilds K = C_k B_k and V = C_v B_v from the
 *     cache, applies rotary position embedding to the rebuilt keys, then
 *     attends;
 *   - Table 2: MHA / MQA / GQA attention, GLU-based and non-GLU MLPs,
 *     rotary embedding (section 5.1: OPT-30B is the non-GLU model).
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major, contiguous. Every pointer argument is a
 *     device pointer owned by the caller, 16-byte aligned.
 *   - Factor storage: every factor is passed transposed, so that its rows
 *     run along the reduction index: A (m x k) as At = A^T [k, m] and
 *     B (k x n) as Bt = B^T [n, k] (the [out, in] layout of the two maps
 *     x -> x A and t -> t B). The up factors of attention are B_k^T and
 *     B_v^T, [n_kv * d, r].
 *   - DL_BF16 operand tiles: with DL_BF16 every factor matrix above (At, Bt,
 *     B_k^T, B_v^T) and every cache page below is stored in 16 x 32 tiles of
 *     1 KB, in MFMA operand order: element (r, c) of an [R, C] matrix sits
 *     at element offset
 *       ((r / 16) * (C / 32) + c / 32) * 512
 *         + (((c % 32) / 8) * 16 + r % 16) * 8 + c % 8
 *     (R % 16 == 0, C % 32 == 0). Every operand fragment the kernels read is
 *     then one contiguous 1 KB block. DL_F32 tensors are plain row-major.
 *     dl_pack_factor / dl_pack_kv_cache convert the pages' row-major
 *     A [m, k], B [k, n] and caches [Bsz, L_max, r] into these layouts.
 *   - Latent caches, DL_BF16: in pages of DL_PAGE = 64 positions. A key page
 *     holds the 64 positions' k latents as an operand-tiled [64, r_k] matrix
 *     (64 * r_k elements); a value page holds the same positions' v latents
 *     rank-major, as an operand-tiled [r_v, 64] matrix (64 * r_v elements),
 *     because attention reduces the value latents over positions. A
 *     contiguous cache (Ck, Cv with L_max rows per sequence, L_max % 64 ==
 *     0) is sequence b's L_max / 64 pages back to back: Ck and Cv are
 *     [Bsz, L_max / 64, 64 * r] in pages. A paged cache (dl_kv_cache) reaches
 *     each sequence's pages through a block table.
 *   - Latent caches, DL_F32: Ck is [Bsz, L_max, r_k] row-major and Cv is
 *     rank-major [Bsz, r_v, L_max]; no paged form.
 *   - dtype DL_F32: every tensor is float32 and arithmetic is float32.
 *     dtype DL_BF16: activations, factors, caches and outputs are bfloat16,
 *     products accumulate in float32; intermediates may be rounded to bf16.
 *   - Outputs have the dtype of the inputs (bf16 stores round to nearest
 *     even), except x2_out of dl_decomposed_layer_fwd which is float32.
 *   - Projection outputs are head-major: head j owns columns [j*d, (j+1)*d).
 *     Query head h reads kv head h / (n_q / n_kv).
 *   - Rotary embedding rotates the pair (v_i, v_{i+d/2}) by the angle
 *     pos * theta^(-2i/d). It is applied to the query and to rebuilt keys,
 *     never to the cache. rope_theta == 0 disables it.
 *   - sm_scale == 0 selects 1/sqrt(d).
 *   - `stream` is a hipStream_t (NULL = the null stream). Every call only
 *     enqueues work on it and returns without synchronising. The library
 *     never allocates, frees or synchronises device memory.
 *   - `ws` is a caller-owned device workspace of at least the size the
 *     matching *_workspace() query returns; its contents on entry are
 *     ignored and on return are unspecified. Calls that overlap in time
 *     must not share a workspace.
 *   - Host-side validation runs before any launch. On failure nothing is
 *     enqueued and a status is returned; dl_last_error() then describes it.
 *   - Tuning switches, read from the environment at each call (results are
 *     the same whatever they are set to; only timing changes):
 *       DL_FUSED_CHAIN      "all" (default): decode-sized factor pairs and
 *                           the dependent GEMV stages of a decode step run
 *                           as persistent fused launches; "pair": only
 *                           dl_lowrank_linear's pair; "none": one launch
 *                           per factor.
 *       DL_CHAIN_WGS_PER_CU persistent workgroups per compute unit of a
 *                           fused launch (default 1).
 *       DL_GEMV_R           force 1, 2 or 4 16-row weight tiles per GEMV
 *                           work item (default: chosen per launch).
 *       DL_GEMV_KS, DL_GEMV_MIN_STEPS, DL_GEMV_CUS, DL_GEMV_WAVES
 *                           GEMV K-split cap, minimum steps per split,
 *                           compute units assumed, waves per workgroup.
 *       DL_ATTN_TARGET_WGS  decode-attention workgroups aimed for when
 *                           choosing the context splits (default 256).
 *   - Device-resident lengths (past_lens, ctx_lens) are not checked (that
 *     would need a synchronisation); their stated ranges are preconditions.
 */
#ifndef DL_H
#define DL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DL_OK = 0,
  DL_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, n_q % n_kv != 0, bad dtype */
  DL_ERR_UNSUPPORTED = 2,  /* a shape the library does not implement (see each call) */
  DL_ERR_ALIGNMENT = 3,    /* a tensor pointer is not 16-byte aligned */
  DL_ERR_WORKSPACE = 4,    /* ws is NULL or ws_bytes is below the required size */
  DL_ERR_HIP = 5           /* a HIP launch failed; dl_last_error() has the text */
} dl_status;

typedef enum { DL_F32 = 0, DL_BF16 = 1 } dl_dtype;

#define DL_PAGE 64   /* positions per cache page (DL_BF16) */

/* A paged low-rank KV cache (DL_BF16) -- section 4.2, Fig. 4(b): the
 * latents live in fixed-size pages of a pool, and a block table maps each
 * sequence's logical pages to pool pages, so the cache grows a page at a
 * time and one captured HIP graph can replay every decode step (the
 * kernels read lengths and tables from device memory).
 *   k, v        : key and value page pools, num_pages pages each (layout
 *                 above), caller-owned device memory
 *   block_table : device int32 [Bsz, pages_per_seq]; entry [b, p] is the
 *                 pool page holding positions 64 p .. 64 p + 63 of
 *                 sequence b. Preconditions (not checked, device data):
 *                 every entry a call reaches -- pages 0 .. (len - 1) / 64 of
 *                 a sequence of len positions -- lies in [0, num_pages),
 *                 and no two sequences share a page a call writes.
 *   pages_per_seq: row length of block_table; a sequence holds at most
 *                 64 * pages_per_seq positions (the L_max of the paged form).
 *   num_pages   : pages in each pool. */
typedef struct {
  void *k;
  void *v;
  const int32_t *block_table;
  int64_t pages_per_seq;
  int64_t num_pages;
} dl_kv_cache;

/* Description of the last non-OK status returned on the calling thread. */
const char *dl_last_error(void);

/* ------------------------------------------------------------------------
 * Factor-pair projection -- section 2.1, Eq. (1).
 *   y[M, n] = (x[M, m] A[m, k]) B[k, n]      A passed as At [k, m], B as Bt [n, k]
 * For M <= 64 the pair is one fused launch: a persistent grid streams A,
 * hands the rank-k intermediate x A to the B stage through the
 * device-coherent cache level, and streams B (MFMA GEMV passes on 16-row
 * tiles); for larger M it runs as two MFMA GEMMs with the intermediate in
 * the workspace.
 * DL_BF16 requires m, k, n to be multiples of 64 (else UNSUPPORTED).
 * ------------------------------------------------------------------------ */
size_t dl_lowrank_linear_workspace(int64_t M, int64_t m, int64_t k, int64_t n,
                                   dl_dtype dt);
dl_status dl_lowrank_linear(const void *x, const void *A, const void *B, void *y,
                            int64_t M, int64_t m, int64_t k, int64_t n,
                            dl_dtype dt, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Allocation-free factor-pair projection.
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, result and kernels as dl_lowrank_linear, but
 * the workspace is a static device array inside the library (one per GPU,
 * held from library load until the process ends) of DL_STATIC_SCRATCH_BYTES
 * (16 MiB). A product whose
 * dl_lowrank_linear_workspace() exceeds that is rejected with
 * DL_ERR_WORKSPACE before any device work. The call allocates and frees
 * nothing. Every call on one GPU uses the same scratch array, and each call
 * re-initialises what it needs, so sequential calls (any stream order that
 * serialises them) are safe; calls that overlap in time on one GPU (other
 * streams, other threads) race on the scratch and give undefined results.
 * ------------------------------------------------------------------------ */
#define DL_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
dl_status dl_lowrank_linear_static(const void *x, const void *A, const void *B,
                                   void *y, int64_t M, int64_t m, int64_t k,
                                   int64_t n, dl_dtype dt, void *stream);

/* ------------------------------------------------------------------------
 * Low-rank KV-cache append -- section 2.1 (the k/v latents are the cache)
 * and section 4.1 (they are stored as KV cache).
 *   key latent   (b, past_lens[b] + t) = x[b, t, :] A_k     x : [Bsz, T, m]
 *   value latent (b, past_lens[b] + t) = x[b, t, :] A_v     A_k, A_v passed
 *                                                           as [r_k, m], [r_v, m]
 * into the cache (layouts above). past_lens: device int32 [Bsz];
 * precondition past_lens[b] + T <= L_max. No other cache position is
 * written. DL_BF16 requires m, r_k, r_v multiples of 64 and L_max % 64 == 0.
 * The _paged form writes through the block table (L_max = 64 *
 * pages_per_seq).
 * ------------------------------------------------------------------------ */
size_t dl_kv_append_workspace(int64_t Bsz, int64_t T, int64_t m, int64_t r_k,
                              int64_t r_v, dl_dtype dt);
dl_status dl_lowrank_kv_append(const void *x, const void *A_k, const void *A_v,
                               void *Ck, void *Cv, const int32_t *past_lens,
                               int64_t Bsz, int64_t T, int64_t m, int64_t r_k,
                               int64_t r_v, int64_t L_max, dl_dtype dt,
                               void *ws, size_t ws_bytes, void *stream);
dl_status dl_lowrank_kv_append_paged(const void *x, const void *A_k,
                                     const void *A_v, const dl_kv_cache *cache,
                                     const int32_t *past_lens, int64_t Bsz,
                                     int64_t T, int64_t m, int64_t r_k,
                                     int64_t r_v, dl_dtype dt, void *ws,
                                     size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Decode attention over the low-rank cache -- section 4.2.
 *   q   : [Bsz, n_q, d] un-rotated queries
 *   Ck, Cv: latent caches of L_max positions per sequence (layouts above)
 *   B_k : [r_k, n_kv*d], B_v: [r_v, n_kv*d] up factors of the k and v pairs,
 *         passed transposed ([n_kv*d, r_k], [n_kv*d, r_v])
 *   ctx_lens: device int32 [Bsz], 1 <= ctx_lens[b] <= L_max
 *   out : [Bsz, n_q, d]
 * Sequence b attends rows 0 .. ctx_lens[b]-1 and its query sits at position
 * ctx_lens[b]-1. Keys are rebuilt on chip (never written to memory) and
 * rotated by their row index; the value factor is applied once to the
 * probability-weighted value latents (softmax(s) C_v B_v, the same product
 * in another association). Softmax is computed online.
 * DL_BF16 requires d in {64, 128}, r_k and r_v multiples of 64, r_v <= 1024,
 * L_max % 64 == 0 and n_q / n_kv <= 16. DL_F32 requires even d <= 256.
 * The _paged form reads the cache through its block table (L_max = 64 *
 * pages_per_seq for the workspace query).
 * ------------------------------------------------------------------------ */
size_t dl_attn_decode_workspace(int64_t Bsz, int64_t n_q, int64_t n_kv,
                                int64_t d, int64_t r_k, int64_t r_v,
                                int64_t L_max, dl_dtype dt);
dl_status dl_lowrank_attn_decode(const void *q, const void *Ck, const void *Cv,
                                 const void *B_k, const void *B_v,
                                 const int32_t *ctx_lens, void *out,
                                 int64_t Bsz, int64_t n_q, int64_t n_kv,
                                 int64_t d, int64_t r_k, int64_t r_v,
                                 int64_t L_max, float sm_scale,
                                 float rope_theta, dl_dtype dt, void *ws,
                                 size_t ws_bytes, void *stream);
dl_status dl_lowrank_attn_decode_paged(const void *q, const dl_kv_cache *cache,
                                       const void *B_k, const void *B_v,
                                       const int32_t *ctx_lens, void *out,
                                       int64_t Bsz, int64_t n_q, int64_t n_kv,
                                       int64_t d, int64_t r_k, int64_t r_v,
                                       float sm_scale, float rope_theta,
                                       dl_dtype dt, void *ws, size_t ws_bytes,
                                       void *stream);

/* ------------------------------------------------------------------------
 * Causal prefill attention over the low-rank cache -- section 4.2.
 *   q   : [Bsz, T, n_q, d] un-rotated; out: [Bsz, T, n_q, d]
 * Query t of sequence b sits at position past_lens[b] + t and attends rows
 * 0 .. past_lens[b] + t, which must already hold the latents (append
 * first). Precondition past_lens[b] + T <= L_max. Same shape rules as
 * decode; DL_BF16 also needs each cache pool (all pages of Ck, or of Cv)
 * below 2 GiB. DL_BF16 runs in the section's order, rebuild then attend:
 * every cached key up to past_lens[b] + T - 1 is rebuilt once (K rotated,
 * and V) into the workspace, Bsz * n_kv * L_max * d * 4 bytes of it, then
 * the causal pass reads those tiles.
 * ------------------------------------------------------------------------ */
size_t dl_attn_prefill_workspace(int64_t Bsz, int64_t T, int64_t n_q,
                                 int64_t n_kv, int64_t d, int64_t r_k,
                                 int64_t r_v, int64_t L_max, dl_dtype dt);
dl_status dl_lowrank_attn_prefill(const void *q, const void *Ck, const void *Cv,
                                  const void *B_k, const void *B_v,
                                  const int32_t *past_lens, void *out,
                                  int64_t Bsz, int64_t T, int64_t n_q,
                                  int64_t n_kv, int64_t d, int64_t r_k,
                                  int64_t r_v, int64_t L_max, float sm_scale,
                                  float rope_theta, dl_dtype dt, void *ws,
                                  size_t ws_bytes, void *stream);
dl_status dl_lowrank_attn_prefill_paged(const void *q, const dl_kv_cache *cache,
                                        const void *B_k, const void *B_v,
                                        const int32_t *past_lens, void *out,
                                        int64_t Bsz, int64_t T, int64_t n_q,
                                        int64_t n_kv, int64_t d, int64_t r_k,
                                        int64_t r_v, float sm_scale,
                                        float rope_theta, dl_dtype dt, void *ws,
                                        size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * One decomposed pre-norm transformer layer (LLaMA block; the paper names
 * no norm or residual, this is the plain reading of Fig. 3 on a LLaMA
 * model):
 *   a   = RMSNorm(x) * attn_norm
 *   Ck/Cv rows past..past+T-1 = a A_k, a A_v            (append)
 *   q   = (a A_q) B_q ; o = attention(q, Ck, Cv, B_k, B_v)
 *   x2  = x + (o A_o) B_o
 *   b   = RMSNorm(x2) * mlp_norm
 *   y   = x2 + ((silu((b A_gate) B_gate) * ((b A_up) B_up)) A_down) B_down
 *                                                   (mlp == DL_MLP_GLU)
 *   y   = x2 + (relu((b A_up) B_up) A_down) B_down  (mlp == DL_MLP_RELU)
 * x, y: [Bsz, T, hidden]. T == 1 uses decode attention (query at position
 * past_lens[b]), T > 1 causal prefill attention. past_lens is not advanced
 * (the caller does). x2_out (optional, float32 [Bsz, T, hidden]) receives
 * x2. Factor shapes follow dl_factor; norm gains may be NULL (= 1).
 * DL_MLP_RELU is the non-GLU MLP of Table 2, OPT's fc1 -> ReLU -> fc2 with
 * fc1 = the up pair and fc2 = the down pair (section 5.1); its gate factor
 * is not read and may be {NULL, NULL, 0}. OPT's LayerNorm, biases and
 * learned positions are outside this block (rope_theta = 0 turns the rotary
 * embedding off).
 * ------------------------------------------------------------------------ */
typedef struct {
  const void *A;   /* A^T, [k, m] */
  const void *B;   /* B^T, [n, k] */
  int64_t k;
} dl_factor;

typedef enum { DL_MLP_GLU = 0, DL_MLP_RELU = 1 } dl_mlp;

typedef struct {
  int64_t hidden, n_q, n_kv, head_dim, ffn;
  dl_factor q, k, v, o, gate, up, down;
  const void *attn_norm;  /* [hidden] or NULL */
  const void *mlp_norm;   /* [hidden] or NULL */
  float rms_eps;
  float rope_theta;
  dl_dtype dt;
  dl_mlp mlp;             /* DL_MLP_GLU (SwiGLU) or DL_MLP_RELU (non-GLU) */
} dl_layer;

size_t dl_layer_workspace(const dl_layer *L, int64_t Bsz, int64_t T,
                          int64_t L_max);
/* The same upper bound under its plain name (L_max = 64 * pages_per_seq for
 * the paged form); 0 for an invalid layer description. */
size_t dl_workspace_size(const dl_layer *L, int64_t Bsz, int64_t T,
                         int64_t L_max);
dl_status dl_decomposed_layer_fwd(const dl_layer *L, const void *x, void *y,
                                  void *x2_out, void *Ck, void *Cv,
                                  const int32_t *past_lens, int64_t Bsz,
                                  int64_t T, int64_t L_max, void *ws,
                                  size_t ws_bytes, void *stream);
/* The layer over a paged cache (DL_BF16): appends through the block table,
 * then attends through it. */
dl_status dl_decomposed_layer_fwd_paged(const dl_layer *L, const void *x,
                                        void *y, void *x2_out,
                                        const dl_kv_cache *cache,
                                        const int32_t *past_lens, int64_t Bsz,
                                        int64_t T, void *ws, size_t ws_bytes,
                                        void *stream);

/* ------------------------------------------------------------------------
 * Storage conversion from the pages' row-major form (section 2.1, Eq. (1):
 * A [m, k], B [k, n]; caches [Bsz, L_max, r]) into the library's layouts,
 * on the GPU, asynchronous on `stream`, into caller-owned buffers (nothing
 * is allocated). Source and destination must not overlap.
 *
 * dl_pack_factor: F [rows, cols] row-major (A: rows = m, cols = k; B: rows =
 *   k, cols = n) -> its library storage F^T [cols, rows] (operand tiles for
 *   DL_BF16, plain for DL_F32), dl_factor_bytes(rows, cols, dt) bytes.
 *   DL_BF16 needs rows % 32 == 0 and cols % 16 == 0 (every factor of a
 *   DL_BF16 layer or pair, whose sizes are multiples of 64, qualifies).
 * dl_pack_kv_cache / dl_unpack_kv_cache: Ck [Bsz, L_max, r_k] and
 *   Cv [Bsz, L_max, r_v], row-major, <-> the contiguous library caches of
 *   the same shape (layouts above). DL_BF16 needs L_max % 64 == 0 and
 *   r_k, r_v multiples of 32.
 * Errors: INVALID_ARG (null pointer, non-positive size, bad dtype),
 * UNSUPPORTED (sizes above), ALIGNMENT (pointers not 16-byte aligned),
 * HIP (launch failure).
 * ------------------------------------------------------------------------ */
size_t dl_factor_bytes(int64_t rows, int64_t cols, dl_dtype dt);
dl_status dl_pack_factor(const void *F, int64_t rows, int64_t cols,
                         dl_dtype dt, void *out, void *stream);
dl_status dl_pack_kv_cache(const void *Ck, const void *Cv, int64_t Bsz,
                           int64_t L_max, int64_t r_k, int64_t r_v,
                           dl_dtype dt, void *Ck_lib, void *Cv_lib,
                           void *stream);
dl_status dl_unpack_kv_cache(const void *Ck_lib, const void *Cv_lib,
                             int64_t Bsz, int64_t L_max, int64_t r_k,
                             int64_t r_v, dl_dtype dt, void *Ck, void *Cv,
                             void *stream);

/* ------------------------------------------------------------------------
 * Kernel timing hook (instrumentation; not part of the method).
 * While a trace is installed, every kernel the library enqueues is
 * bracketed by hipEventRecord(events[2i]) and hipEventRecord(events[2i+1])
 * on the call's stream, where i counts traced launches; kinds[i] names the
 * kernel (dl_kernel_kind_name) and roles[i] the step of the layer it serves
 * (dl_role_name). Launches beyond `capacity` run untraced. The events are
 * hipEvent_t created by the caller; the library only records them.
 * Installation is process-wide and not thread-safe; NULL uninstalls.
 * ------------------------------------------------------------------------ */
typedef struct {
  void **events;     /* 2 * capacity hipEvent_t */
  int32_t *kinds;    /* capacity entries */
  int32_t *roles;    /* capacity entries */
  int32_t capacity;
  int32_t count;     /* traced launches so far (advanced by the library) */
} dl_trace;

void dl_trace_install(dl_trace *t);
const char *dl_kernel_kind_name(int32_t kind);
const char *dl_role_name(int32_t role);

/* ------------------------------------------------------------------------
 * Matrix-pipe probe (measurement aid; not part of the method).
 * Launches `blocks` workgroups of eight waves; every wave runs `iters`
 * rounds of twelve 1 KB operand reads from LDS and 32 independent
 * v_mfma_f32_16x16x32_bf16 (16384 flops each) into an 8 x 4 block of
 * accumulators, the prefill GEMM's mix, on random operands that change from
 * round to round. The work is blocks * 8 * iters * 32 * 16384 flops: timing
 * it gives the bf16 MFMA rate this GPU sustains for such a mix, the measured
 * denominator reported next to the published peak.
 * sink: caller-owned device float[blocks * 512], overwritten (the values
 * only keep the products live). Asynchronous on `stream`.
 * Errors: DL_ERR_INVALID_ARG for a null sink or blocks / iters outside
 * [1, 2^31); DL_ERR_HIP on a launch failure.
 * ------------------------------------------------------------------------ */
dl_status dl_probe_mfma_bf16(float *sink, int64_t blocks, int64_t iters,
                             void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DL_H */
