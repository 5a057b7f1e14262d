// C ABI of the decomposed-layer library: host-side validation, workspace
// carving and the launch sequences of the five entry points declared in
// include/dl.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "dl.h"
#include "common.h"
#include "kernels.h"
#include "trace.h"

using namespace dl;

// ---------------------------------------------------------------------------
// Launch tracing (dl_trace)
// ---------------------------------------------------------------------------
namespace {
dl_trace *g_trace = nullptr;
int g_role = R_OTHER;
bool g_open = false;

const char *const kKindNames[K_NUM_KINDS] = {
    "rmsnorm",       "fill",        "convert",      "store_cache_rows",
    "gemv_bf16",     "gemm_bf16",   "gemm_f32",     "pack_up_factor",
    "attn_decode_bf16", "attn_combine", "attn_prefill_bf16", "attn_f32", "gemv_chain",
    "attn_latent"};
const char *const kRoleNames[R_NUM_ROLES] = {
    "other",        "attn_norm",    "qkv_down", "kv_store",  "q_up",
    "attention",    "o_down",       "o_up",     "mlp_norm",  "gate_up_down",
    "gate_up_up",   "down_down",    "down_up",  "output",    "init",
    "qkv_chain",    "o_mlp_chain",  "pair_chain"};
}  // namespace

namespace dl {
void set_role(int role) { g_role = role; }
void trace_begin(int kind, hipStream_t s) {
  g_open = g_trace && g_trace->count < g_trace->capacity;
  if (!g_open) return;
  g_trace->kinds[g_trace->count] = kind;
  (void)hipEventRecord(static_cast<hipEvent_t>(g_trace->events[2 * g_trace->count]), s);
}
void trace_end(hipStream_t s) {
  if (!g_open) return;
  (void)hipEventRecord(static_cast<hipEvent_t>(g_trace->events[2 * g_trace->count + 1]), s);
  g_trace->roles[g_trace->count] = g_role;
  g_trace->count++;
  g_open = false;
}
}  // namespace dl

namespace {

thread_local std::string g_last_error;

dl_status fail(dl_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

#define DL_CHECK(cond, st, ...) \
  do {                          \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define DL_HIP(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(DL_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bump allocator over the caller's workspace. With base == nullptr it only
// measures.
struct Carver {
  char *base;
  size_t off = 0;
  explicit Carver(void *b) : base(static_cast<char *>(b)) {}
  template <typename T>
  T *take(size_t count) {
    T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
    off = align_up(off + count * sizeof(T));
    return p;
  }
};

int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

bool valid_dtype(dl_dtype dt) { return dt == DL_F32 || dt == DL_BF16; }

// ---------------------------------------------------------------------------
// GEMV / GEMM helpers
// ---------------------------------------------------------------------------
GvSeg gvseg(const void *W, const void *X, int ldx, void *out, int ldo, int N, int omode) {
  GvSeg g{};
  g.W = static_cast<const uint16_t *>(W);
  g.X = X;
  g.ldx = ldx;
  g.out = out;
  g.ldo = ldo;
  g.N = N;
  g.omode = omode;
  return g;
}

// Segment whose activations are operand-tiled bf16 ([Mpad, K], ldx = K).
GvSeg gvseg_t(const void *W, const void *X, int K, void *out, int ldo, int N, int omode) {
  return gvseg(W, X, K, out, ldo, N, omode);
}

// rows of an operand-tiled activation buffer
size_t mpad(int64_t M) { return static_cast<size_t>((M + 15) / 16 * 16); }

GvArgs gvargs(int M, int K, int nseg) {
  GvArgs a{};
  a.M = M;
  a.K = K;
  a.nseg = nseg;
  a.T = 1;
  return a;
}

// Sizes of the shared split-K scratch of a sequence of GEMV launches: the
// launches run one after another on one stream, so they share one partial
// buffer and one counter array (each launch leaves its counters at zero).
struct GvScratch {
  size_t part_floats = 0;
  int counters = 0;
  void add(GvArgs &a) {
    part_floats = std::max(part_floats, gemv_plan(a));
    counters = std::max(counters, a.ntiles);
  }
};

hipError_t gemv_run(GvArgs &a, float *part, int *counters, hipStream_t s) {
  gemv_plan(a);
  a.part = part;
  a.counters = counters;
  return launch_gemv(a, s);
}

// Runs GEMV stages in order, each reading the previous one's output: as
// one persistent chain launch per maximal run of stages whose inputs after
// the first are operand-tiled (a stage reading row-major activations starts
// a new run). Stages share `part` / `counters` (a stage's merges finish
// before the next stage passes its wait). sync: kChainSyncInts zero ints per
// run (runs <= max_runs).
hipError_t gemv_sequence(GvArgs *g, int n, float *part, int *counters, int *sync, int max_runs,
                         bool fuse, const int *roles, int chain_role, hipStream_t s) {
  int i = 0, run = 0;
  while (i < n) {
    int j = i + 1;
    while (fuse && j < n && j - i < kMaxChain && g[j].x_tiled) ++j;
    if (j - i > 1 && run >= max_runs) return hipErrorInvalidValue;
    GvChain c{};
    c.nst = j - i;
    c.sync = sync + run * kChainSyncInts;
    for (int k = i; k < j; ++k) {
      gemv_plan(g[k]);
      g[k].part = part;
      g[k].counters = counters;
      c.st[k - i] = g[k];
    }
    set_role(c.nst == 1 ? roles[i] : chain_role);
    const hipError_t e = c.nst == 1 ? launch_gemv(c.st[0], s) : launch_gemv_chain(c, s);
    if (e != hipSuccess) return e;
    if (c.nst > 1) ++run;
    i = j;
  }
  return hipSuccess;
}

// Where decode-sized factor pairs run fused (one persistent launch per chain
// of dependent GEMV stages) instead of one launch per stage:
// DL_FUSED_CHAIN = "all" (default: the pair of dl_lowrank_linear and the
// stages of a decode step) | "pair" (dl_lowrank_linear only) | "none".
enum FuseMode { FUSE_NONE = 0, FUSE_PAIR = 1, FUSE_ALL = 2 };
int fuse_mode() {
  const char *v = getenv("DL_FUSED_CHAIN");
  if (!v || !*v) return FUSE_ALL;
  if (!strcmp(v, "none")) return FUSE_NONE;
  if (!strcmp(v, "pair")) return FUSE_PAIR;
  return FUSE_ALL;
}

// `part`: f32 scratch for the remainder split (NULL: the GEMM runs unsplit)
hipError_t gemm(GemmArgs &a, hipStream_t s, float *part = nullptr, size_t part_bytes = 0) {
  for (int i = 0; i < a.nseg; ++i)
    if (a.seg[i].omode < 0) a.seg[i].omode = a.omode;
  a.part = part;
  a.part_bytes = part_bytes;
  return launch_gemm_bf16(a, s);
}

// Partial bytes of the two GEMMs of a factor pair at prefill-sized M.
size_t pair_part_bytes(int64_t M, int64_t m, int64_t k, int64_t n) {
  return std::max(gemm_part_bytes((int)M, gemm_ntiles((int)k), (int)m),
                  gemm_part_bytes((int)M, gemm_ntiles((int)n), (int)k));
}

GemmSeg mseg(const void *W, const void *X, void *C, int N, int ldx, int ldc) {
  GemmSeg g{};
  g.W = static_cast<const uint16_t *>(W);
  g.X = static_cast<const uint16_t *>(X);
  g.C = C;
  g.N = N;
  g.ldx = ldx;
  g.ldc = ldc;
  g.omode = -1;
  return g;
}

hipError_t gemm_f32(const float *X, const float *X2, const void *W, float *C, int M, int N, int K,
                    int ldx, int ldc, int omode, const float *R, int ldr, const int32_t *past,
                    int T, int L_max, hipStream_t s) {
  GemmF32Args a{};
  a.X = X;
  a.X2 = X2;
  a.W = static_cast<const float *>(W);
  a.C = C;
  a.R = R;
  a.M = M;
  a.N = N;
  a.K = K;
  a.ldx = ldx;
  a.ldc = ldc;
  a.ldr = ldr;
  a.omode = omode;
  a.past_lens = past;
  a.T = T;
  a.L_max = L_max;
  return launch_gemm_f32(a, s);
}

// ---------------------------------------------------------------------------
// Attention planning
// ---------------------------------------------------------------------------
struct DecodePlan {
  int nsplit, split_len;
};
// Context splits of decode attention: one workgroup per CU for the
// (sequence, kv head) work items, splits balanced to the position granule,
// at most 64 splits.
DecodePlan plan_decode(int64_t Bsz, int64_t n_kv, int64_t L_max) {
  const int gran = attn_decode_split_granule();
  const int target = env_int("DL_ATTN_TARGET_WGS", 256);
  int ns = static_cast<int>((target + Bsz * n_kv - 1) / (Bsz * n_kv));
  ns = std::max(1, std::min(ns, 64));
  ns = std::min<int64_t>(ns, (L_max + gran - 1) / gran);
  int len = static_cast<int>((L_max + ns - 1) / ns);
  len = (len + gran - 1) / gran * gran;
  ns = static_cast<int>((L_max + len - 1) / len);
  return {ns, len};
}

// Latent-space decode attention (rotary embedding off): groups of 16 query
// heads; splits no longer than one workgroup's LDS holds, enough of them
// for about one workgroup per CU.
constexpr int kLatentHeads = 16;
struct LatentPlan {
  int ngroups = 0, nsplit = 0, split_len = 0;   // nsplit == 0: not available
};
LatentPlan plan_latent(int64_t Bsz, int64_t n_q, int64_t r_k, int64_t L_max) {
  LatentPlan p;
  const int maxs = latent_attn_max_split(static_cast<int>(r_k));
  if (maxs < 64) return p;
  p.ngroups = static_cast<int>((n_q + kLatentHeads - 1) / kLatentHeads);
  const int target = env_int("DL_ATTN_TARGET_WGS", 256);
  int ns = static_cast<int>((target + Bsz * p.ngroups - 1) / (Bsz * p.ngroups));
  ns = std::max<int64_t>(ns, (L_max + maxs - 1) / maxs);
  ns = std::min<int64_t>(ns, (L_max + 63) / 64);
  int len = static_cast<int>((L_max + ns - 1) / ns);
  len = std::min((len + 63) / 64 * 64, maxs);
  p.nsplit = static_cast<int>((L_max + len - 1) / len);
  p.split_len = len;
  return p;
}

// Attention scratch: split partials and merge counters (decode; the
// counters must be zero before the launch), plus the latent path's
// absorbed queries, normalised U rows and partials.
struct AttnWS {
  float *part = nullptr;
  float *uglob = nullptr;   // rebuilding decode kernel's U between chunks (r_v > 512)
  int *counters = nullptr;
  int n_counters = 0;
  uint16_t *lat_q = nullptr, *lat_u = nullptr;
  float *lat_part = nullptr;
  int *lat_counters = nullptr;
  uint16_t *kv_tiles = nullptr;   // prefill: rebuilt K / V^T tile images
};

AttnWS carve_attn(Carver &c, int64_t Bsz, int64_t n_q, int64_t n_kv, int64_t d, int64_t r_k,
                  int64_t r_v, int64_t L_max, bool decode) {
  AttnWS w;
  if (decode) {
    const DecodePlan p = plan_decode(Bsz, n_kv, L_max);
    const LatentPlan lp = plan_latent(Bsz, n_q, r_k, L_max);
    w.part = c.take<float>(static_cast<size_t>(Bsz * n_q * p.nsplit * (d + 2)));
    if (attn_decode_value_passes(static_cast<int>(r_v)) > 1)
      w.uglob = c.take<float>(static_cast<size_t>(Bsz * n_kv * p.nsplit) * 16 * r_v);
    w.n_counters = static_cast<int>(Bsz * n_kv + (lp.nsplit ? Bsz * lp.ngroups : 0));
    w.counters = c.take<int>(static_cast<size_t>(w.n_counters));
    if (lp.nsplit) {
      w.lat_counters = w.counters + Bsz * n_kv;
      w.lat_q = c.take<uint16_t>(static_cast<size_t>(Bsz * lp.ngroups * kLatentHeads * r_k));
      w.lat_u = c.take<uint16_t>(static_cast<size_t>(Bsz * n_q * r_v));
      if (lp.nsplit > 1)
        w.lat_part = c.take<float>(static_cast<size_t>(Bsz * lp.ngroups) * lp.nsplit * kLatentHeads *
                                   (r_v + 2));
    }
  } else {
    w.kv_tiles = c.take<uint16_t>(static_cast<size_t>(Bsz * n_kv * (L_max / kPage)) * 2 * kPage * d);
  }
  return w;
}

size_t attn_bf16_ws(int64_t Bsz, int64_t n_q, int64_t n_kv, int64_t d, int64_t r_k, int64_t r_v,
                    int64_t L_max, bool decode) {
  Carver c(nullptr);
  carve_attn(c, Bsz, n_q, n_kv, d, r_k, r_v, L_max, decode);
  return c.off;
}

// Decode attention without the rotary embedding runs in the latent space
// when one workgroup's LDS holds the group's absorbed queries.
bool use_latent_decode(float theta, int64_t r_k) {
  return theta == 0.f && latent_attn_max_split(static_cast<int>(r_k)) >= 64;
}

dl_status check_attn_shape(int64_t n_q, int64_t n_kv, int64_t d, int64_t r_k, int64_t r_v,
                           int64_t L_max, dl_dtype dt, bool prefill, float theta) {
  DL_CHECK(n_q > 0 && n_kv > 0 && d > 0 && r_k > 0 && r_v > 0, DL_ERR_INVALID_ARG,
           "attention dims must be positive");
  DL_CHECK(n_q % n_kv == 0, DL_ERR_INVALID_ARG, "n_q (%lld) must be a multiple of n_kv (%lld)",
           (long long)n_q, (long long)n_kv);
  if (dt == DL_BF16) {
    DL_CHECK(d == 64 || d == 128, DL_ERR_UNSUPPORTED, "bf16 attention needs head_dim 64 or 128");
    DL_CHECK(r_k % 64 == 0 && r_v % 64 == 0, DL_ERR_UNSUPPORTED,
             "bf16 attention needs r_k, r_v multiples of 64");
    DL_CHECK(r_k <= 8192 && r_v <= 8192, DL_ERR_UNSUPPORTED, "bf16 attention needs r_k, r_v <= 8192");
    DL_CHECK(L_max % kPage == 0, DL_ERR_UNSUPPORTED,
             "bf16 caches need L_max to be a multiple of %d (cache pages)", kPage);
    const int64_t G = n_q / n_kv;
    DL_CHECK(G <= 16, DL_ERR_UNSUPPORTED, "bf16 attention needs n_q / n_kv <= 16");
    if (prefill)
      DL_CHECK(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, DL_ERR_UNSUPPORTED,
               "bf16 prefill attention needs n_q / n_kv in {1, 2, 4, 8, 16}");
  } else {
    DL_CHECK(d % 2 == 0 && d <= 256, DL_ERR_UNSUPPORTED, "f32 attention needs even head_dim <= 256");
  }
  return DL_OK;
}

// A latent cache as the kernels see it: two page pools, an optional block
// table and the pages per sequence (see cache_page in common.h). A contiguous
// bf16 cache of L_max rows per sequence is the same thing with the identity
// table: L_max / kPage pages per sequence, sequence b's pages consecutive.
struct CacheRef {
  void *k = nullptr, *v = nullptr;
  const int32_t *table = nullptr;
  int stride = 0;           // pages per sequence (table row length)
  int64_t pool_pages = 0;   // pages in each pool
  int64_t L_max = 0;        // positions per sequence = stride * kPage (bf16)
};

CacheRef contiguous_cache(void *Ck, void *Cv, int64_t Bsz, int64_t L_max) {
  CacheRef c;
  c.k = Ck;
  c.v = Cv;
  c.stride = static_cast<int>(L_max / kPage);
  c.pool_pages = Bsz * (L_max / kPage);
  c.L_max = L_max;
  return c;
}

// Checks a paged cache descriptor and converts it (bf16 only).
dl_status paged_cache(const dl_kv_cache *pc, dl_dtype dt, CacheRef *out) {
  DL_CHECK(pc, DL_ERR_INVALID_ARG, "null cache descriptor");
  DL_CHECK(dt == DL_BF16, DL_ERR_UNSUPPORTED, "paged caches are bf16 only");
  DL_CHECK(pc->k && pc->v && pc->block_table, DL_ERR_INVALID_ARG, "null cache pointer");
  DL_CHECK(pc->pages_per_seq > 0 && pc->num_pages > 0, DL_ERR_INVALID_ARG,
           "pages_per_seq and num_pages must be positive");
  DL_CHECK(pc->pages_per_seq <= (1 << 24) && pc->num_pages <= INT32_MAX, DL_ERR_UNSUPPORTED,
           "page counts too large");
  DL_CHECK(aligned16(pc->k) && aligned16(pc->v) && aligned16(pc->block_table), DL_ERR_ALIGNMENT,
           "cache pointers must be 16-byte aligned");
  out->k = pc->k;
  out->v = pc->v;
  out->table = pc->block_table;
  out->stride = static_cast<int>(pc->pages_per_seq);
  out->pool_pages = pc->num_pages;
  out->L_max = pc->pages_per_seq * kPage;
  return DL_OK;
}

// Prefill attention addresses each pool with 32-bit byte offsets.
dl_status check_prefill_pools(const CacheRef &c, int64_t r_k, int64_t r_v) {
  DL_CHECK(c.pool_pages * kPage * std::max(r_k, r_v) * 2 <= INT32_MAX, DL_ERR_UNSUPPORTED,
           "bf16 prefill attention needs each cache pool below 2 GiB");
  return DL_OK;
}

// Runs the bf16 attention kernels; q is bf16 (q_f32 = 0) or f32. For
// decode, w.counters must be zero.
hipError_t run_attn_bf16(const void *q, int q_f32, int ldq, const CacheRef &c,
                         const void *B_k, const void *B_v, const int32_t *lens, int ctx_offset,
                         bool decode, void *out, int out_f32, int out_tiled, int Bsz, int T,
                         int n_q, int n_kv, int d, int r_k, int r_v, float sm_scale,
                         float theta, const AttnWS &w, hipStream_t s) {
  const float scale = (sm_scale != 0.f ? sm_scale : 1.0f / sqrtf(static_cast<float>(d))) * kLog2e;
  const int L_max = static_cast<int>(c.L_max);
  if (decode && use_latent_decode(theta, r_k)) {
    const LatentPlan p = plan_latent(Bsz, n_q, r_k, L_max);
    LatentAttnArgs a{};
    a.q = q;
    a.q_f32 = q_f32;
    a.ck = static_cast<const uint16_t *>(c.k);
    a.cv = static_cast<const uint16_t *>(c.v);
    a.block_table = c.table;
    a.page_stride = c.stride;
    a.bk = static_cast<const uint16_t *>(B_k);
    a.bv = static_cast<const uint16_t *>(B_v);
    a.ctx_lens = lens;
    a.ctx_offset = ctx_offset;
    a.out = out;
    a.out_f32 = out_f32;
    a.out_tiled = out_tiled;
    a.qt = w.lat_q;
    a.u = w.lat_u;
    a.part = w.lat_part;
    a.counters = w.lat_counters;
    a.Bsz = Bsz;
    a.n_q = n_q;
    a.n_kv = n_kv;
    a.d = d;
    a.r_k = r_k;
    a.r_v = r_v;
    a.L_max = L_max;
    a.ngroups = p.ngroups;
    a.nsplit = p.nsplit;
    a.split_len = p.split_len;
    a.scale_log2 = scale;
    return launch_latent_attn_bf16(a, s);
  }
  if (decode) {
    const DecodePlan p = plan_decode(Bsz, n_kv, L_max);
    AttnDecodeArgs a{};
    a.q = q;
    a.q_f32 = q_f32;
    a.ck = static_cast<const uint16_t *>(c.k);
    a.cv = static_cast<const uint16_t *>(c.v);
    a.block_table = c.table;
    a.page_stride = c.stride;
    a.bk = static_cast<const uint16_t *>(B_k);
    a.bv = static_cast<const uint16_t *>(B_v);
    a.ctx_lens = lens;
    a.ctx_offset = ctx_offset;
    a.out = out;
    a.out_f32 = out_f32;
    a.out_tiled = out_tiled;
    a.part = w.part;
    a.uglob = w.uglob;
    a.counters = w.counters;
    a.Bsz = Bsz;
    a.n_q = n_q;
    a.n_kv = n_kv;
    a.d = d;
    a.r_k = r_k;
    a.r_v = r_v;
    a.L_max = L_max;
    a.nsplit = p.nsplit;
    a.split_len = p.split_len;
    a.scale_log2 = scale;
    a.theta = theta;
    return launch_attn_decode_bf16(a, s);
  }
  AttnPrefillArgs a{};
  a.q = q;
  a.q_f32 = q_f32;
  a.ldq = ldq;
  a.ck = static_cast<const uint16_t *>(c.k);
  a.cv = static_cast<const uint16_t *>(c.v);
  a.block_table = c.table;
  a.page_stride = c.stride;
  a.pool_pages = c.pool_pages;
  a.bk = static_cast<const uint16_t *>(B_k);
  a.bv = static_cast<const uint16_t *>(B_v);
  a.past_lens = lens;
  a.out = static_cast<uint16_t *>(out);
  a.out_tiled = out_tiled;
  a.kv = w.kv_tiles;
  a.Bsz = Bsz;
  a.T = T;
  a.n_q = n_q;
  a.n_kv = n_kv;
  a.d = d;
  a.r_k = r_k;
  a.r_v = r_v;
  a.L_max = L_max;
  a.scale_log2 = scale;
  a.theta = theta;
  return launch_attn_prefill_bf16(a, s);
}

// ---------------------------------------------------------------------------
// Layer workspace layout
// ---------------------------------------------------------------------------
struct LayerDims {
  int M, T, Bsz, h, nq, nkv, d, f, rq, rk, rv, ro, rg, ru, rd, L_max;
  bool relu;   // non-GLU MLP: relu(up), no gate pair
  int qd() const { return nq * d; }
};

// The factor pairs a layer reads (the gate pair only with the GLU MLP).
int layer_factors(const dl_layer *L, const dl_factor *(&fs)[7]) {
  int n = 0;
  fs[n++] = &L->q;
  fs[n++] = &L->k;
  fs[n++] = &L->v;
  fs[n++] = &L->o;
  if (L->mlp != DL_MLP_RELU) fs[n++] = &L->gate;
  fs[n++] = &L->up;
  fs[n++] = &L->down;
  return n;
}

bool use_gemv(int M) { return M <= 64; }

}  // namespace

extern "C" {

const char *dl_last_error(void) { return g_last_error.c_str(); }

void dl_trace_install(dl_trace *t) {
  g_trace = t;
  g_open = false;
}
const char *dl_kernel_kind_name(int32_t kind) {
  return (kind >= 0 && kind < K_NUM_KINDS) ? kKindNames[kind] : "unknown";
}
const char *dl_role_name(int32_t role) {
  return (role >= 0 && role < R_NUM_ROLES) ? kRoleNames[role] : "unknown";
}

dl_status dl_probe_mfma_bf16(float *sink, int64_t blocks, int64_t iters, void *stream) {
  set_role(R_OTHER);
  DL_CHECK(sink, DL_ERR_INVALID_ARG, "null sink");
  DL_CHECK(blocks > 0 && blocks <= INT32_MAX && iters > 0 && iters <= INT32_MAX,
           DL_ERR_INVALID_ARG, "blocks and iters must lie in [1, 2^31)");
  DL_HIP(launch_mfma_probe(sink, static_cast<int>(blocks), static_cast<int>(iters),
                           as_stream(stream)));
  return DL_OK;
}

// ===========================================================================
// dl_lowrank_linear
// ===========================================================================
// GEMV-path plan of the factor pair (shapes only; pointers are filled in later).
static void linear_gemvs(int M, int m, int k, int n, const void *x, const void *A, const void *B,
                         void *t, void *y, GvArgs &g1, GvArgs &g2) {
  // the rank-k intermediate stays in operand tiles between the two passes
  g1 = gvargs(M, m, 1);
  g1.seg[0] = gvseg(A, x, m, t, k, k, GV_OUT_TILED);
  g2 = gvargs(M, k, 1);
  g2.x_tiled = 1;
  g2.seg[0] = gvseg_t(B, t, k, y, n, n, GV_OUT_BF16);
}

size_t dl_lowrank_linear_workspace(int64_t M, int64_t m, int64_t k, int64_t n, dl_dtype dt) {
  if (M <= 0 || m <= 0 || k <= 0 || n <= 0) return 0;
  Carver c(nullptr);
  if (dt == DL_F32) {
    c.take<float>(static_cast<size_t>(M * k));
  } else if (use_gemv(static_cast<int>(M))) {
    GvArgs g1, g2;
    linear_gemvs((int)M, (int)m, (int)k, (int)n, nullptr, nullptr, nullptr, nullptr, nullptr, g1, g2);
    GvScratch sc;
    sc.add(g1);
    sc.add(g2);
    c.take<int>(sc.counters + kChainSyncInts);
    c.take<float>(sc.part_floats);
    c.take<uint16_t>(mpad(M) * k);
  } else {
    c.take<uint16_t>(mpad(M) * k);
    c.take<float>(pair_part_bytes(M, m, k, n) / sizeof(float));
  }
  return c.off;
}

dl_status dl_lowrank_linear(const void *x, const void *A, const void *B, void *y, int64_t M,
                            int64_t m, int64_t k, int64_t n, dl_dtype dt, void *ws,
                            size_t ws_bytes, void *stream) {
  set_role(R_OTHER);
  DL_CHECK(valid_dtype(dt), DL_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  DL_CHECK(x && A && B && y, DL_ERR_INVALID_ARG, "null tensor pointer");
  DL_CHECK(M > 0 && m > 0 && k > 0 && n > 0, DL_ERR_INVALID_ARG, "dims must be positive");
  DL_CHECK(M <= INT32_MAX / 2 && m * k <= INT32_MAX && k * n <= INT32_MAX, DL_ERR_UNSUPPORTED,
           "dims too large");
  if (dt == DL_BF16)
    DL_CHECK(m % 64 == 0 && k % 64 == 0 && n % 64 == 0, DL_ERR_UNSUPPORTED,
             "bf16 factor pairs need m, k, n multiples of 64");
  DL_CHECK(aligned16(x) && aligned16(A) && aligned16(B) && aligned16(y), DL_ERR_ALIGNMENT,
           "tensor pointers must be 16-byte aligned");
  const size_t need = dl_lowrank_linear_workspace(M, m, k, n, dt);
  DL_CHECK(ws && aligned16(ws) && ws_bytes >= need, DL_ERR_WORKSPACE,
           "workspace of %zu bytes required, %zu given", need, ws_bytes);
  hipStream_t s = as_stream(stream);
  Carver c(ws);
  const int Mi = static_cast<int>(M), mi = static_cast<int>(m), ki = static_cast<int>(k),
            ni = static_cast<int>(n);
  if (dt == DL_F32) {
    float *t = c.take<float>(static_cast<size_t>(M * k));
    DL_HIP(gemm_f32(static_cast<const float *>(x), nullptr, A, t, Mi, ki, mi, mi, ki,
                    F32_OUT_STORE, nullptr, 0, nullptr, 1, 0, s));
    DL_HIP(gemm_f32(t, nullptr, B, static_cast<float *>(y), Mi, ni, ki, ki, ni, F32_OUT_STORE,
                    nullptr, 0, nullptr, 1, 0, s));
    return DL_OK;
  }
  if (use_gemv(Mi)) {
    GvArgs g1, g2;
    linear_gemvs(Mi, mi, ki, ni, nullptr, nullptr, nullptr, nullptr, nullptr, g1, g2);
    GvScratch sc;
    sc.add(g1);
    sc.add(g2);
    int *counters = c.take<int>(sc.counters + kChainSyncInts);
    float *part = c.take<float>(sc.part_floats);
    uint16_t *t = c.take<uint16_t>(mpad(M) * k);
    linear_gemvs(Mi, mi, ki, ni, x, A, B, t, y, g1, g2);
    // the fused pair: x A and then t B in one persistent launch, the rank-k
    // intermediate t handed over on chip (split counters and the chain's
    // ticket / done counters zeroed first)
    FillRegion z[1] = {{reinterpret_cast<float *>(counters), nullptr, 0, sc.counters + kChainSyncInts}};
    DL_HIP(launch_fill(z, 1, s));
    GvArgs g[2] = {g1, g2};
    const int roles[2] = {R_OTHER, R_OTHER};
    DL_HIP(gemv_sequence(g, 2, part, counters, counters + sc.counters, 1, fuse_mode() >= FUSE_PAIR,
                         roles, R_PAIR_CHAIN, s));
    return DL_OK;
  }
  // the rank-k intermediate in operand tiles (M rounded up to 16 rows)
  uint16_t *t = c.take<uint16_t>(mpad(M) * k);
  const size_t pb = pair_part_bytes(M, m, k, n);
  float *part = c.take<float>(pb / sizeof(float));
  GemmArgs a{};
  a.nseg = 1;
  a.M = Mi;
  a.K = mi;
  a.xmode = GEMM_X_BF16;
  a.omode = GEMM_OUT_BF16;
  a.seg[0] = mseg(A, x, t, ki, mi, ki);
  a.seg[0].c_tiled = 1;
  DL_HIP(gemm(a, s, part, pb));
  GemmArgs b{};
  b.nseg = 1;
  b.M = Mi;
  b.K = ki;
  b.xmode = GEMM_X_TILED;
  b.omode = GEMM_OUT_BF16;
  b.seg[0] = mseg(B, t, y, ni, ki, ni);
  DL_HIP(gemm(b, s, part, pb));
  return DL_OK;
}

// ===========================================================================
// dl_lowrank_linear_static: the same product with the workspace in a
// file-scope device array instead of a caller buffer
// ===========================================================================
namespace {
// Scratch of the allocation-free variant. Each device that runs the library
// holds its own copy from code-object load until the process ends. In host
// code `scratch` only names the symbol: its device address is looked up once
// per device with hipGetSymbolAddress and only that address is ever passed
// to kernels or copies.
constexpr size_t kScratchBytes = DL_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call per device, with that device current).
dl_status scratch_on_current_device(void **out) {
  int dev = -1;
  DL_HIP(hipGetDevice(&dev));
  DL_CHECK(dev >= 0 && dev < kMaxDevices, DL_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    DL_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    DL_CHECK(p != nullptr, DL_ERR_HIP, "hipGetSymbolAddress returned a null scratch address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DL_OK;
}
}  // namespace

dl_status dl_lowrank_linear_static(const void *x, const void *A, const void *B, void *y,
                                   int64_t M, int64_t m, int64_t k, int64_t n, dl_dtype dt,
                                   void *stream) {
  set_role(R_OTHER);
  DL_CHECK(valid_dtype(dt), DL_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  DL_CHECK(M > 0 && m > 0 && k > 0 && n > 0, DL_ERR_INVALID_ARG, "dims must be positive");
  const size_t need = dl_lowrank_linear_workspace(M, m, k, n, dt);
  DL_CHECK(need <= kScratchBytes, DL_ERR_WORKSPACE,
           "this product needs %zu bytes of scratch; the static scratch holds %zu "
           "(use dl_lowrank_linear with a caller workspace)",
           need, kScratchBytes);
  void *ws = nullptr;
  const dl_status st = scratch_on_current_device(&ws);
  if (st != DL_OK) return st;
  return dl_lowrank_linear(x, A, B, y, M, m, k, n, dt, ws, kScratchBytes, stream);
}

// ===========================================================================
// dl_lowrank_kv_append
// ===========================================================================
static GvArgs append_gemv(int M, int m, int rk, int rv, int T, const CacheRef &cache,
                          const void *x, const void *A_k, const void *A_v, const int32_t *past) {
  GvArgs a = gvargs(M, m, 2);
  a.past = past;
  a.T = T;
  a.block_table = cache.table;
  a.page_stride = cache.stride;
  a.seg[0] = gvseg(A_k, x, m, cache.k, rk, rk, GV_OUT_CACHE);
  a.seg[1] = gvseg(A_v, x, m, cache.v, rv, rv, GV_OUT_CACHE_T);
  return a;
}

size_t dl_kv_append_workspace(int64_t Bsz, int64_t T, int64_t m, int64_t r_k, int64_t r_v,
                              dl_dtype dt) {
  if (Bsz <= 0 || T <= 0 || m <= 0 || r_k <= 0 || r_v <= 0) return 0;
  const int64_t M = Bsz * T;
  if (dt == DL_BF16 && use_gemv(static_cast<int>(M))) {
    GvArgs a = append_gemv((int)M, (int)m, (int)r_k, (int)r_v, (int)T, CacheRef{}, nullptr,
                           nullptr, nullptr, nullptr);
    GvScratch sc;
    sc.add(a);
    Carver c(nullptr);
    c.take<int>(sc.counters);
    c.take<float>(sc.part_floats);
    return c.off;
  }
  return 0;
}

static dl_status kv_append_impl(const void *x, const void *A_k, const void *A_v,
                                const CacheRef &cache, const int32_t *past_lens, int64_t Bsz,
                                int64_t T, int64_t m, int64_t r_k, int64_t r_v, dl_dtype dt,
                                void *ws, size_t ws_bytes, void *stream) {
  const int64_t L_max = cache.L_max;
  DL_CHECK(x && A_k && A_v && cache.k && cache.v && past_lens, DL_ERR_INVALID_ARG, "null pointer");
  DL_CHECK(Bsz > 0 && T > 0 && m > 0 && r_k > 0 && r_v > 0 && L_max > 0, DL_ERR_INVALID_ARG,
           "dims must be positive");
  DL_CHECK(T <= L_max, DL_ERR_INVALID_ARG, "T exceeds L_max");
  DL_CHECK(Bsz * T <= INT32_MAX / 2 && Bsz * L_max * std::max(r_k, r_v) <= ((int64_t)1 << 40),
           DL_ERR_UNSUPPORTED, "dims too large");
  if (dt == DL_BF16) {
    DL_CHECK(m % 64 == 0 && r_k % 64 == 0 && r_v % 64 == 0, DL_ERR_UNSUPPORTED,
             "bf16 append needs m, r_k, r_v multiples of 64");
    DL_CHECK(L_max % kPage == 0, DL_ERR_UNSUPPORTED,
             "bf16 caches need L_max to be a multiple of %d (cache pages)", kPage);
  }
  DL_CHECK(aligned16(x) && aligned16(A_k) && aligned16(A_v) && aligned16(cache.k) &&
               aligned16(cache.v) && aligned16(past_lens),
           DL_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
  const size_t need = dl_kv_append_workspace(Bsz, T, m, r_k, r_v, dt);
  DL_CHECK(need == 0 || (ws && aligned16(ws) && ws_bytes >= need), DL_ERR_WORKSPACE,
           "workspace of %zu bytes required, %zu given", need, ws_bytes);
  hipStream_t s = as_stream(stream);
  const int M = static_cast<int>(Bsz * T), mi = static_cast<int>(m), rk = static_cast<int>(r_k),
            rv = static_cast<int>(r_v), Ti = static_cast<int>(T), Lm = static_cast<int>(L_max);
  if (dt == DL_F32) {
    DL_HIP(gemm_f32(static_cast<const float *>(x), nullptr, A_k, static_cast<float *>(cache.k), M,
                    rk, mi, mi, rk, F32_OUT_CACHE, nullptr, 0, past_lens, Ti, Lm, s));
    DL_HIP(gemm_f32(static_cast<const float *>(x), nullptr, A_v, static_cast<float *>(cache.v), M,
                    rv, mi, mi, rv, F32_OUT_CACHE_T, nullptr, 0, past_lens, Ti, Lm, s));
    return DL_OK;
  }
  if (use_gemv(M)) {
    GvArgs a = append_gemv(M, mi, rk, rv, Ti, cache, x, A_k, A_v, past_lens);
    GvScratch sc;
    sc.add(a);
    Carver c(ws);
    int *counters = c.take<int>(sc.counters);
    float *part = c.take<float>(sc.part_floats);
    FillRegion z[1] = {{reinterpret_cast<float *>(counters), nullptr, 0, sc.counters}};
    DL_HIP(launch_fill(z, 1, s));
    DL_HIP(gemv_run(a, part, counters, s));
    return DL_OK;
  }
  GemmArgs a{};
  a.nseg = 2;
  a.M = M;
  a.K = mi;
  a.xmode = GEMM_X_BF16;
  a.omode = GEMM_OUT_CACHE;
  a.past_lens = past_lens;
  a.T = Ti;
  a.block_table = cache.table;
  a.page_stride = cache.stride;
  a.seg[0] = mseg(A_k, x, cache.k, rk, mi, rk);
  a.seg[1] = mseg(A_v, x, cache.v, rv, mi, rv);
  a.seg[1].omode = GEMM_OUT_CACHE_T;
  DL_HIP(gemm(a, s));
  return DL_OK;
}

dl_status dl_lowrank_kv_append(const void *x, const void *A_k, const void *A_v, void *Ck,
                               void *Cv, const int32_t *past_lens, int64_t Bsz, int64_t T,
                               int64_t m, int64_t r_k, int64_t r_v, int64_t L_max, dl_dtype dt,
                               void *ws, size_t ws_bytes, void *stream) {
  set_role(R_OTHER);
  DL_CHECK(valid_dtype(dt), DL_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  DL_CHECK(Bsz > 0 && L_max > 0, DL_ERR_INVALID_ARG, "dims must be positive");
  return kv_append_impl(x, A_k, A_v, contiguous_cache(Ck, Cv, Bsz, L_max), past_lens, Bsz, T, m,
                        r_k, r_v, dt, ws, ws_bytes, stream);
}

dl_status dl_lowrank_kv_append_paged(const void *x, const void *A_k, const void *A_v,
                                     const dl_kv_cache *cache, const int32_t *past_lens,
                                     int64_t Bsz, int64_t T, int64_t m, int64_t r_k, int64_t r_v,
                                     dl_dtype dt, void *ws, size_t ws_bytes, void *stream) {
  set_role(R_OTHER);
  DL_CHECK(valid_dtype(dt), DL_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  CacheRef c;
  const dl_status st = paged_cache(cache, dt, &c);
  if (st != DL_OK) return st;
  return kv_append_impl(x, A_k, A_v, c, past_lens, Bsz, T, m, r_k, r_v, dt, ws, ws_bytes, stream);
}

// ===========================================================================
// Attention entry points
// ===========================================================================
size_t dl_attn_decode_workspace(int64_t Bsz, int64_t n_q, int64_t n_kv, int64_t d, int64_t r_k,
                                int64_t r_v, int64_t L_max, dl_dtype dt) {
  if (dt != DL_BF16 || Bsz <= 0 || n_kv <= 0 || L_max <= 0) return 0;
  return attn_bf16_ws(Bsz, n_q, n_kv, d, r_k, r_v, L_max, true);
}

size_t dl_attn_prefill_workspace(int64_t Bsz, int64_t T, int64_t n_q, int64_t n_kv, int64_t d,
                                 int64_t r_k, int64_t r_v, int64_t L_max, dl_dtype dt) {
  (void)T;
  if (dt != DL_BF16 || Bsz <= 0 || n_kv <= 0 || L_max <= 0) return 0;
  return attn_bf16_ws(Bsz, n_q, n_kv, d, r_k, r_v, L_max, false);
}

static dl_status attn_common(const void *q, const CacheRef &cache, const void *B_k,
                             const void *B_v, const int32_t *lens, void *out, int64_t Bsz,
                             int64_t T, int64_t n_q, int64_t n_kv, int64_t d, int64_t r_k,
                             int64_t r_v, float sm_scale, float rope_theta,
                             dl_dtype dt, void *ws, size_t ws_bytes, void *stream, bool decode) {
  const int64_t L_max = cache.L_max;
  DL_CHECK(q && cache.k && cache.v && B_k && B_v && lens && out, DL_ERR_INVALID_ARG, "null pointer");
  DL_CHECK(Bsz > 0 && T > 0 && L_max > 0, DL_ERR_INVALID_ARG, "dims must be positive");
  DL_CHECK(T <= L_max, DL_ERR_INVALID_ARG, "T exceeds L_max");
  dl_status st = check_attn_shape(n_q, n_kv, d, r_k, r_v, L_max, dt, !decode, rope_theta);
  if (st != DL_OK) return st;
  DL_CHECK(Bsz * L_max * std::max(r_k, r_v) <= ((int64_t)1 << 40) && Bsz * T * n_q * d <= INT32_MAX &&
               L_max <= INT32_MAX / 2,
           DL_ERR_UNSUPPORTED, "dims too large");
  DL_CHECK(isfinite(sm_scale) && sm_scale >= 0.f && isfinite(rope_theta) && rope_theta >= 0.f,
           DL_ERR_INVALID_ARG, "sm_scale and rope_theta must be finite and non-negative");
  DL_CHECK(aligned16(q) && aligned16(cache.k) && aligned16(cache.v) && aligned16(B_k) &&
               aligned16(B_v) && aligned16(lens) && aligned16(out),
           DL_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
  if (dt == DL_BF16 && !decode) {
    st = check_prefill_pools(cache, r_k, r_v);
    if (st != DL_OK) return st;
  }
  const size_t need = decode ? dl_attn_decode_workspace(Bsz, n_q, n_kv, d, r_k, r_v, L_max, dt)
                             : dl_attn_prefill_workspace(Bsz, T, n_q, n_kv, d, r_k, r_v, L_max, dt);
  DL_CHECK(need == 0 || (ws && aligned16(ws) && ws_bytes >= need), DL_ERR_WORKSPACE,
           "workspace of %zu bytes required, %zu given", need, ws_bytes);
  hipStream_t s = as_stream(stream);
  if (dt == DL_F32) {
    AttnF32Args a{};
    a.q = static_cast<const float *>(q);
    a.ck = static_cast<const float *>(cache.k);
    a.cv = static_cast<const float *>(cache.v);
    a.bk = static_cast<const float *>(B_k);
    a.bv = static_cast<const float *>(B_v);
    a.lens = lens;
    a.out = static_cast<float *>(out);
    a.decode = decode ? 1 : 0;
    a.Bsz = static_cast<int>(Bsz);
    a.T = static_cast<int>(T);
    a.n_q = static_cast<int>(n_q);
    a.n_kv = static_cast<int>(n_kv);
    a.d = static_cast<int>(d);
    a.r_k = static_cast<int>(r_k);
    a.r_v = static_cast<int>(r_v);
    a.L_max = static_cast<int>(L_max);
    a.ldq = static_cast<int>(n_q * d);
    a.sm_scale = sm_scale != 0.f ? sm_scale : 1.0f / sqrtf(static_cast<float>(d));
    a.theta = rope_theta;
    DL_HIP(launch_attn_f32(a, s));
    return DL_OK;
  }
  Carver c(ws);
  const AttnWS aw = carve_attn(c, Bsz, n_q, n_kv, d, r_k, r_v, L_max, decode);
  if (aw.counters) {
    FillRegion z[1] = {{reinterpret_cast<float *>(aw.counters), nullptr, 0, aw.n_counters}};
    DL_HIP(launch_fill(z, 1, s));
  }
  DL_HIP(run_attn_bf16(q, 0, static_cast<int>(n_q * d), cache, B_k, B_v, lens, 0, decode, out, 0, 0,
                       static_cast<int>(Bsz), static_cast<int>(T), static_cast<int>(n_q),
                       static_cast<int>(n_kv), static_cast<int>(d), static_cast<int>(r_k),
                       static_cast<int>(r_v), sm_scale, rope_theta, aw, s));
  return DL_OK;
}

dl_status dl_lowrank_attn_decode(const void *q, const void *Ck, const void *Cv, const void *B_k,
                                 const void *B_v, const int32_t *ctx_lens, void *out, int64_t Bsz,
                                 int64_t n_q, int64_t n_kv, int64_t d, int64_t r_k, int64_t r_v,
                                 int64_t L_max, float sm_scale, float rope_theta, dl_dtype dt,
                                 void *ws, size_t ws_bytes, void *stream) {
  set_role(R_OTHER);
  DL_CHECK(valid_dtype(dt), DL_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  DL_CHECK(Bsz > 0 && L_max > 0, DL_ERR_INVALID_ARG, "dims must be positive");
  return attn_common(q, contiguous_cache(const_cast<void *>(Ck), const_cast<void *>(Cv), Bsz, L_max),
                     B_k, B_v, ctx_lens, out, Bsz, 1, n_q, n_kv, d, r_k, r_v, sm_scale,
                     rope_theta, dt, ws, ws_bytes, stream, true);
}

dl_status dl_lowrank_attn_prefill(const void *q, const void *Ck, const void *Cv, const void *B_k,
                                  const void *B_v, const int32_t *past_lens, void *out,
                                  int64_t Bsz, int64_t T, int64_t n_q, int64_t n_kv, int64_t d,
                                  int64_t r_k, int64_t r_v, int64_t L_max, float sm_scale,
                                  float rope_theta, dl_dtype dt, void *ws, size_t ws_bytes,
                                  void *stream) {
  set_role(R_OTHER);
  DL_CHECK(valid_dtype(dt), DL_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  DL_CHECK(Bsz > 0 && L_max > 0, DL_ERR_INVALID_ARG, "dims must be positive");
  return attn_common(q, contiguous_cache(const_cast<void *>(Ck), const_cast<void *>(Cv), Bsz, L_max),
                     B_k, B_v, past_lens, out, Bsz, T, n_q, n_kv, d, r_k, r_v, sm_scale,
                     rope_theta, dt, ws, ws_bytes, stream, false);
}

dl_status dl_lowrank_attn_decode_paged(const void *q, const dl_kv_cache *cache, const void *B_k,
                                       const void *B_v, const int32_t *ctx_lens, void *out,
                                       int64_t Bsz, int64_t n_q, int64_t n_kv, int64_t d,
                                       int64_t r_k, int64_t r_v, float sm_scale,
                                       float rope_theta, dl_dtype dt, void *ws, size_t ws_bytes,
                                       void *stream) {
  set_role(R_OTHER);
  DL_CHECK(valid_dtype(dt), DL_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  CacheRef c;
  const dl_status st = paged_cache(cache, dt, &c);
  if (st != DL_OK) return st;
  return attn_common(q, c, B_k, B_v, ctx_lens, out, Bsz, 1, n_q, n_kv, d, r_k, r_v, sm_scale,
                     rope_theta, dt, ws, ws_bytes, stream, true);
}

dl_status dl_lowrank_attn_prefill_paged(const void *q, const dl_kv_cache *cache, const void *B_k,
                                        const void *B_v, const int32_t *past_lens, void *out,
                                        int64_t Bsz, int64_t T, int64_t n_q, int64_t n_kv,
                                        int64_t d, int64_t r_k, int64_t r_v, float sm_scale,
                                        float rope_theta, dl_dtype dt, void *ws, size_t ws_bytes,
                                        void *stream) {
  set_role(R_OTHER);
  DL_CHECK(valid_dtype(dt), DL_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  CacheRef c;
  const dl_status st = paged_cache(cache, dt, &c);
  if (st != DL_OK) return st;
  return attn_common(q, c, B_k, B_v, past_lens, out, Bsz, T, n_q, n_kv, d, r_k, r_v, sm_scale,
                     rope_theta, dt, ws, ws_bytes, stream, false);
}

// ===========================================================================
// dl_decomposed_layer_fwd
// ===========================================================================
static dl_status layer_dims(const dl_layer *L, int64_t Bsz, int64_t T, int64_t L_max,
                            LayerDims *o) {
  DL_CHECK(L, DL_ERR_INVALID_ARG, "null layer");
  DL_CHECK(valid_dtype(L->dt), DL_ERR_INVALID_ARG, "unknown dtype %d", (int)L->dt);
  DL_CHECK(Bsz > 0 && T > 0 && L_max > 0, DL_ERR_INVALID_ARG, "Bsz, T, L_max must be positive");
  DL_CHECK(T <= L_max, DL_ERR_INVALID_ARG, "T exceeds L_max");
  DL_CHECK(L->hidden > 0 && L->n_q > 0 && L->n_kv > 0 && L->head_dim > 0 && L->ffn > 0,
           DL_ERR_INVALID_ARG, "layer dims must be positive");
  DL_CHECK(L->mlp == DL_MLP_GLU || L->mlp == DL_MLP_RELU, DL_ERR_INVALID_ARG, "unknown MLP kind %d",
           (int)L->mlp);
  const dl_factor *fs[7];
  const int nf = layer_factors(L, fs);
  for (int i = 0; i < nf; ++i) {
    DL_CHECK(fs[i]->A && fs[i]->B, DL_ERR_INVALID_ARG, "null factor pointer");
    DL_CHECK(fs[i]->k > 0, DL_ERR_INVALID_ARG, "factor rank must be positive");
  }
  dl_status st = check_attn_shape(L->n_q, L->n_kv, L->head_dim, L->k.k, L->v.k, L_max, L->dt, T > 1,
                                  L->rope_theta);
  if (st != DL_OK) return st;
  if (L->dt == DL_BF16) {
    bool ok = L->hidden % 64 == 0 && L->ffn % 64 == 0;
    for (int i = 0; i < nf; ++i) ok = ok && fs[i]->k % 64 == 0;
    DL_CHECK(ok, DL_ERR_UNSUPPORTED, "bf16 layer needs hidden, ffn and every rank multiples of 64");
  }
  DL_CHECK(Bsz * T <= (1 << 24) && L->hidden <= (1 << 20) && L->ffn <= (1 << 20) &&
               Bsz * L_max * std::max(L->k.k, L->v.k) <= ((int64_t)1 << 40),
           DL_ERR_UNSUPPORTED, "dims too large");
  DL_CHECK(isfinite(L->rms_eps) && L->rms_eps >= 0.f && isfinite(L->rope_theta) &&
               L->rope_theta >= 0.f,
           DL_ERR_INVALID_ARG, "rms_eps and rope_theta must be finite and non-negative");
  o->M = static_cast<int>(Bsz * T);
  o->T = static_cast<int>(T);
  o->Bsz = static_cast<int>(Bsz);
  o->h = static_cast<int>(L->hidden);
  o->nq = static_cast<int>(L->n_q);
  o->nkv = static_cast<int>(L->n_kv);
  o->d = static_cast<int>(L->head_dim);
  o->f = static_cast<int>(L->ffn);
  o->rq = static_cast<int>(L->q.k);
  o->rk = static_cast<int>(L->k.k);
  o->rv = static_cast<int>(L->v.k);
  o->ro = static_cast<int>(L->o.k);
  o->relu = L->mlp == DL_MLP_RELU;
  o->rg = o->relu ? 0 : static_cast<int>(L->gate.k);
  o->ru = static_cast<int>(L->up.k);
  o->rd = static_cast<int>(L->down.k);
  o->L_max = static_cast<int>(L_max);
  return DL_OK;
}

// Workspace regions, in carve order (measuring and running use the same code).
struct LayerWS {
  // f32 path
  float *a, *tq, *qf, *att, *to, *x2, *b, *tg, *tu, *G, *U, *td;
  // bf16 small-M path: split-K scratch, bf16 latents, f32 query and residual stream
  int *counters;
  int n_counters;
  int *chain_sync;
  float *part, *q32, *x2f, *ssq;
  uint16_t *att16, *H16, *a16t, *x2g;
  // bf16 large-M (MFMA GEMM) path
  uint16_t *a16, *b16, *tq16, *q16, *to16, *tg16, *tu16, *G16, *td16;
  float *gpart;         // f32 partials of the GEMMs' remainder split
  size_t gpart_bytes;
};

enum { G_QKV, G_QUP, G_ODOWN, G_OUP, G_GUD, G_GUU, G_DD, G_DU, G_NUM };

// The eight GEMV launches of a small-M layer step:
//   (init)    RMSNorm(x) into operand tiles; split-K counters zeroed
//   qkv_down  x_n [A_q A_k A_v]; k, v latents scattered into the cache
//   q_up      t_q B_q -> f32 query
//   o_down    o A_o
//   o_up      x2 = x + t_o B_o (f32 residual stream; copy to x2_out), plus
//             g_mlp * x2 as bf16 tiles and its row sums of squares per tile
//   gate_up   (g_mlp * x2) [A_gate A_up], rows scaled by 1 / rms(x2)
//   gu_up     H = silu(t_g B_gate) * (t_u B_up)   (one paired launch)
//   down_down H A_down
//   down_up   y = x2 + t_d B_down
static void layer_gemvs(const dl_layer *L, const LayerDims &D, const LayerWS &w, const void *x,
                        void *y, void *x2_out, const CacheRef &cache, const int32_t *past,
                        GvArgs (&g)[G_NUM]) {
  const int M = D.M, h = D.h, qd = D.qd();
  const int gf32 = L->dt == DL_F32;
  g[G_QKV] = gvargs(M, h, 3);
  g[G_QKV].past = past;
  g[G_QKV].T = D.T;
  g[G_QKV].block_table = cache.table;
  g[G_QKV].page_stride = cache.stride;
  // x arrives row-major; the step's init launch normalises it into operand tiles
  (void)x;
  g[G_QKV].x_tiled = 1;
  g[G_QKV].seg[0] = gvseg_t(L->q.A, w.a16t, h, w.tq16, D.rq, D.rq, GV_OUT_TILED);
  g[G_QKV].seg[1] = gvseg_t(L->k.A, w.a16t, h, cache.k, D.rk, D.rk, GV_OUT_CACHE);
  g[G_QKV].seg[2] = gvseg_t(L->v.A, w.a16t, h, cache.v, D.rv, D.rv, GV_OUT_CACHE_T);

  g[G_QUP] = gvargs(M, D.rq, 1);
  g[G_QUP].x_tiled = 1;
  g[G_QUP].seg[0] = gvseg_t(L->q.B, w.tq16, D.rq, w.q32, qd, qd, GV_OUT_F32);

  g[G_ODOWN] = gvargs(M, qd, 1);
  g[G_ODOWN].x_tiled = D.T == 1;   // decode attention writes operand tiles, prefill rows
  g[G_ODOWN].seg[0] = gvseg_t(L->o.A, w.att16, qd, w.to16, D.ro, D.ro, GV_OUT_TILED);

  g[G_OUP] = gvargs(M, D.ro, 1);
  g[G_OUP].x_tiled = 1;
  g[G_OUP].seg[0] = gvseg_t(L->o.B, w.to16, D.ro, w.x2f, h, h, GV_OUT_RES_F32);
  g[G_OUP].seg[0].R = x;
  g[G_OUP].seg[0].ldr = h;
  g[G_OUP].seg[0].out2 = static_cast<float *>(x2_out);
  g[G_OUP].seg[0].out_nt = w.x2g;   // the MLP norm's input for the down halves
  g[G_OUP].seg[0].gamma = L->mlp_norm;
  g[G_OUP].seg[0].gamma_f32 = gf32;
  g[G_OUP].seg[0].ssq_out = w.ssq;

  g[G_GUD] = gvargs(M, h, D.relu ? 1 : 2);
  g[G_GUD].x_tiled = 1;
  g[G_GUD].rs_part = w.ssq;
  g[G_GUD].rs_cols = h / 16;
  g[G_GUD].eps = L->rms_eps;
  if (D.relu) {
    // non-GLU MLP: H = relu(t_u B_up)
    g[G_GUD].seg[0] = gvseg_t(L->up.A, w.x2g, h, w.tu16, D.ru, D.ru, GV_OUT_TILED);
    g[G_GUU] = gvargs(M, D.ru, 1);
    g[G_GUU].x_tiled = 1;
    g[G_GUU].seg[0] = gvseg_t(L->up.B, w.tu16, D.ru, w.H16, D.f, D.f, GV_OUT_RELU_TILED);
  } else {
    g[G_GUD].seg[0] = gvseg_t(L->gate.A, w.x2g, h, w.tg16, D.rg, D.rg, GV_OUT_TILED);
    g[G_GUD].seg[1] = gvseg_t(L->up.A, w.x2g, h, w.tu16, D.ru, D.ru, GV_OUT_TILED);
    g[G_GUU] = gvargs(M, D.rg, 1);
    g[G_GUU].K2 = D.ru;
    g[G_GUU].x_tiled = 1;
    g[G_GUU].seg[0] = gvseg_t(L->gate.B, w.tg16, D.rg, w.H16, D.f, D.f, GV_OUT_SWIGLU_TILED);
    g[G_GUU].seg[0].W2 = static_cast<const uint16_t *>(L->up.B);
    g[G_GUU].seg[0].X2 = w.tu16;
    g[G_GUU].seg[0].ldx2 = D.ru;
  }

  g[G_DD] = gvargs(M, D.f, 1);
  g[G_DD].x_tiled = 1;
  g[G_DD].seg[0] = gvseg_t(L->down.A, w.H16, D.f, w.td16, D.rd, D.rd, GV_OUT_TILED);

  g[G_DU] = gvargs(M, D.rd, 1);
  g[G_DU].x_tiled = 1;
  g[G_DU].seg[0] = gvseg_t(L->down.B, w.td16, D.rd, y, h, h, GV_OUT_RES_BF16);
  g[G_DU].seg[0].R = w.x2f;
  g[G_DU].seg[0].ldr = h;
}

static void carve_layer(Carver &c, const LayerDims &D, const dl_layer *L, LayerWS &w) {
  const size_t M = D.M;
  if (L->dt == DL_F32) {
    w.a = c.take<float>(M * D.h);
    w.tq = c.take<float>(M * D.rq);
    w.qf = c.take<float>(M * D.qd());
    w.att = c.take<float>(M * D.qd());
    w.to = c.take<float>(M * D.ro);
    w.x2 = c.take<float>(M * D.h);
    w.b = c.take<float>(M * D.h);
    w.tg = c.take<float>(M * D.rg);
    w.tu = c.take<float>(M * D.ru);
    w.G = c.take<float>(M * D.f);
    w.U = c.take<float>(M * D.f);
    w.td = c.take<float>(M * D.rd);
    return;
  }
  if (use_gemv(D.M)) {
    GvArgs g[G_NUM];
    LayerWS none{};
    layer_gemvs(L, D, none, nullptr, nullptr, nullptr, CacheRef{}, nullptr, g);
    GvScratch sc;
    for (GvArgs &a : g) sc.add(a);
    // split counters, then the sync ints of up to three chain runs; all
    // zeroed by the step's first kernel
    w.n_counters = sc.counters + 3 * kChainSyncInts;
    w.counters = c.take<int>(w.n_counters);
    w.chain_sync = w.counters + sc.counters;
    w.part = c.take<float>(sc.part_floats);
    // operand-tiled intermediates ([Mpad, cols], Mpad = M rounded up to 16)
    const size_t Mp = mpad(D.M);
    w.a16t = c.take<uint16_t>(Mp * D.h);
    w.x2g = c.take<uint16_t>(Mp * D.h);
    w.ssq = c.take<float>(static_cast<size_t>(D.M) * (D.h / 16));
    w.tq16 = c.take<uint16_t>(Mp * D.rq);
    w.q32 = c.take<float>(M * D.qd());
    w.att16 = c.take<uint16_t>(Mp * D.qd());
    w.to16 = c.take<uint16_t>(Mp * D.ro);
    w.x2f = c.take<float>(M * D.h);
    w.tg16 = c.take<uint16_t>(Mp * D.rg);
    w.tu16 = c.take<uint16_t>(Mp * D.ru);
    w.H16 = c.take<uint16_t>(Mp * D.f);
    w.td16 = c.take<uint16_t>(Mp * D.rd);
    return;
  }
  // operand-tiled activations: M rounded up to 16 rows
  const size_t Mt = mpad(D.M);
  w.a16 = c.take<uint16_t>(Mt * D.h);
  w.tq16 = c.take<uint16_t>(Mt * D.rq);
  w.q16 = c.take<uint16_t>(M * D.qd());
  w.att16 = c.take<uint16_t>(Mt * D.qd());
  w.to16 = c.take<uint16_t>(Mt * D.ro);
  w.x2f = c.take<float>(M * D.h);
  w.b16 = c.take<uint16_t>(Mt * D.h);
  w.tg16 = c.take<uint16_t>(Mt * D.rg);
  w.tu16 = c.take<uint16_t>(Mt * D.ru);
  w.G16 = c.take<uint16_t>(Mt * D.f);
  w.td16 = c.take<uint16_t>(Mt * D.rd);
  // one partial buffer for the step's GEMMs (they run in order on one
  // stream): the largest need over their shapes, (column tiles, depth)
  const int nt = gemm_ntiles(D.rq) + gemm_ntiles(D.rk) + gemm_ntiles(D.rv);
  const int gud = D.relu ? gemm_ntiles(D.ru) : gemm_ntiles(D.rg) + gemm_ntiles(D.ru);
  const int shapes[][2] = {{nt, D.h},
                           {gemm_ntiles(D.qd()), D.rq},
                           {gemm_ntiles(D.ro), D.qd()},
                           {gemm_ntiles(D.h), D.ro},
                           {gud, D.h},
                           {gemm_ntiles(D.f), D.rg},
                           {gemm_ntiles(D.f), D.ru},
                           {gemm_ntiles(D.rd), D.f},
                           {gemm_ntiles(D.h), D.rd}};
  size_t pb = 0;
  for (const auto &sh : shapes) pb = std::max(pb, gemm_part_bytes(D.M, sh[0], sh[1]));
  w.gpart_bytes = pb;
  w.gpart = c.take<float>(pb / sizeof(float));
}

// Decode batches of 65 .. 512 sequences run as chunks of 64 sequences on
// the GEMV path (each chunk reads the weights once): the GEMM's 256-row
// tiles leave most of the GPU idle at such M. Sequences are independent in
// decode, so a chunk is the same layer on a sub-batch.
constexpr int64_t kDecodeChunk = 64, kDecodeChunkedMax = 512;
bool chunked_decode(const dl_layer *L, int64_t Bsz, int64_t T) {
  return L && L->dt == DL_BF16 && T == 1 && Bsz > kDecodeChunk && Bsz <= kDecodeChunkedMax;
}

size_t dl_layer_workspace(const dl_layer *L, int64_t Bsz, int64_t T, int64_t L_max) {
  if (chunked_decode(L, Bsz, T)) {
    // one chunk's workspace, then the batch's queries, attention output and
    // attention workspace (the carve of layer_impl's chunked branch)
    LayerDims D{};
    if (layer_dims(L, Bsz, T, L_max, &D) != DL_OK) return 0;
    Carver c(nullptr);
    c.take<char>(dl_layer_workspace(L, kDecodeChunk, T, L_max));
    c.take<float>(static_cast<size_t>(Bsz * D.qd()));
    c.take<uint16_t>(mpad(Bsz) * D.qd());
    carve_attn(c, D.Bsz, D.nq, D.nkv, D.d, D.rk, D.rv, D.L_max, true);
    return c.off;
  }
  LayerDims D{};
  if (layer_dims(L, Bsz, T, L_max, &D) != DL_OK) return 0;
  Carver c(nullptr);
  LayerWS w{};
  carve_layer(c, D, L, w);
  if (L->dt == DL_BF16)
    c.off += attn_bf16_ws(D.Bsz, D.nq, D.nkv, D.d, D.rk, D.rv, D.L_max, D.T == 1) + kAlign;
  return c.off;
}

// Phases of a small-M (GEMV) layer step: the norm and the q / k / v chain,
// the attention, the o / MLP chain. A chunked decode runs the first and the
// last per chunk and the attention once over all chunks.
enum { PH_PRE = 1, PH_ATTN = 2, PH_POST = 4, PH_ALL = 7 };

static dl_status layer_impl(const dl_layer *L, const void *x, void *y, void *x2_out,
                            const CacheRef &cache, const int32_t *past_lens, int64_t Bsz,
                            int64_t T, void *ws, size_t ws_bytes, void *stream, int phases = PH_ALL,
                            float *q_ext = nullptr, uint16_t *att_ext = nullptr,
                            const AttnWS *aw_zero = nullptr) {
  const int64_t L_max = cache.L_max;
  LayerDims D{};
  dl_status st = layer_dims(L, Bsz, T, L_max, &D);
  if (st != DL_OK) return st;
  DL_CHECK(x && y && cache.k && cache.v && past_lens, DL_ERR_INVALID_ARG, "null pointer");
  if (chunked_decode(L, Bsz, T)) {
    // Chunks of kDecodeChunk sequences: each chunk's norm and q / k / v chain
    // (its queries into one buffer for the batch), then one attention launch
    // over every sequence (a fuller GPU than one per chunk), then each
    // chunk's o / MLP chain on its rows of the attention output. A chunk sees
    // its rows of x, y, x2_out and past_lens and its pages of the cache; the
    // chunks reuse one per-chunk workspace in stream order.
    const size_t chunk_ws = dl_layer_workspace(L, kDecodeChunk, T, L_max);
    const int64_t qd = D.qd();
    Carver cw(ws);
    cw.take<char>(chunk_ws);
    float *q_all = cw.take<float>(static_cast<size_t>(Bsz * qd));
    uint16_t *att_all = cw.take<uint16_t>(mpad(Bsz) * qd);
    const AttnWS aw_all = carve_attn(cw, D.Bsz, D.nq, D.nkv, D.d, D.rk, D.rv, D.L_max, true);
    DL_CHECK(ws && aligned16(ws) && ws_bytes >= cw.off, DL_ERR_WORKSPACE,
             "workspace of %zu bytes required, %zu given", cw.off, ws_bytes);
    const int64_t h = L->hidden;
    auto chunk = [&](int64_t b0, int ph) {
      const int64_t nb = std::min(kDecodeChunk, Bsz - b0);
      CacheRef c = cache;
      if (c.table) {
        c.table += b0 * c.stride;
      } else {
        c.k = static_cast<uint16_t *>(c.k) + b0 * c.stride * kPage * L->k.k;
        c.v = static_cast<uint16_t *>(c.v) + b0 * c.stride * kPage * L->v.k;
        c.pool_pages = nb * c.stride;
      }
      // the batch buffers: queries f32 row-major, attention output in operand
      // tiles (b0 is a multiple of 16, so a chunk's tiles start at row b0)
      return layer_impl(L, static_cast<const uint16_t *>(x) + b0 * h, static_cast<uint16_t *>(y) + b0 * h,
                        x2_out ? static_cast<float *>(x2_out) + b0 * h : nullptr, c, past_lens + b0, nb,
                        T, ws, chunk_ws, stream, ph, q_all + b0 * qd, att_all + b0 * qd,
                        b0 == 0 ? &aw_all : nullptr);
    };
    for (int64_t b0 = 0; b0 < Bsz; b0 += kDecodeChunk)
      if ((st = chunk(b0, PH_PRE)) != DL_OK) return st;
    set_role(R_ATTENTION);
    DL_HIP(run_attn_bf16(q_all, 1, static_cast<int>(qd), cache, L->k.B, L->v.B, past_lens, 1, true,
                         att_all, 0, 1, D.Bsz, D.T, D.nq, D.nkv, D.d, D.rk, D.rv, 0.f, L->rope_theta,
                         aw_all, as_stream(stream)));
    for (int64_t b0 = 0; b0 < Bsz; b0 += kDecodeChunk)
      if ((st = chunk(b0, PH_POST)) != DL_OK) return st;
    return DL_OK;
  }
  void *Ck = cache.k, *Cv = cache.v;
  const dl_factor *fs[7];
  const int nf = layer_factors(L, fs);
  bool al = aligned16(x) && aligned16(y) && aligned16(Ck) && aligned16(Cv) && aligned16(past_lens);
  for (int i = 0; i < nf; ++i) al = al && aligned16(fs[i]->A) && aligned16(fs[i]->B);
  al = al && (!x2_out || aligned16(x2_out)) && (!L->attn_norm || aligned16(L->attn_norm)) &&
       (!L->mlp_norm || aligned16(L->mlp_norm));
  DL_CHECK(al, DL_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
  if (L->dt == DL_BF16 && T > 1) {
    st = check_prefill_pools(cache, L->k.k, L->v.k);
    if (st != DL_OK) return st;
  }
  const size_t need = dl_layer_workspace(L, Bsz, T, L_max);
  DL_CHECK(ws && aligned16(ws) && ws_bytes >= need, DL_ERR_WORKSPACE,
           "workspace of %zu bytes required, %zu given", need, ws_bytes);

  hipStream_t s = as_stream(stream);
  Carver c(ws);
  LayerWS w{};
  carve_layer(c, D, L, w);
  AttnWS aw;
  if (L->dt == DL_BF16) aw = carve_attn(c, D.Bsz, D.nq, D.nkv, D.d, D.rk, D.rv, D.L_max, D.T == 1);
  const int M = D.M, h = D.h, qd = D.qd();
  const float eps = L->rms_eps;
  const int gf32 = L->dt == DL_F32;

  if (L->dt == DL_F32) {
    const float *xf = static_cast<const float *>(x);
    set_role(R_ATTN_NORM);
    DL_HIP(launch_rmsnorm(x, 1, L->attn_norm, 1, w.a, 1, M, h, eps, s));
    set_role(R_QKV_DOWN);
    DL_HIP(gemm_f32(w.a, nullptr, L->k.A, static_cast<float *>(Ck), M, D.rk, h, h, D.rk,
                    F32_OUT_CACHE, nullptr, 0, past_lens, D.T, D.L_max, s));
    DL_HIP(gemm_f32(w.a, nullptr, L->v.A, static_cast<float *>(Cv), M, D.rv, h, h, D.rv,
                    F32_OUT_CACHE_T, nullptr, 0, past_lens, D.T, D.L_max, s));
    set_role(R_QKV_DOWN);
    DL_HIP(gemm_f32(w.a, nullptr, L->q.A, w.tq, M, D.rq, h, h, D.rq, F32_OUT_STORE, nullptr, 0,
                    nullptr, 1, 0, s));
    set_role(R_Q_UP);
    DL_HIP(gemm_f32(w.tq, nullptr, L->q.B, w.qf, M, qd, D.rq, D.rq, qd, F32_OUT_STORE, nullptr, 0,
                    nullptr, 1, 0, s));
    AttnF32Args a{};
    a.q = w.qf;
    a.ck = static_cast<const float *>(Ck);
    a.cv = static_cast<const float *>(Cv);
    a.bk = static_cast<const float *>(L->k.B);
    a.bv = static_cast<const float *>(L->v.B);
    a.lens = past_lens;
    a.out = w.att;
    a.decode = 0;
    a.Bsz = D.Bsz;
    a.T = D.T;
    a.n_q = D.nq;
    a.n_kv = D.nkv;
    a.d = D.d;
    a.r_k = D.rk;
    a.r_v = D.rv;
    a.L_max = D.L_max;
    a.ldq = qd;
    a.sm_scale = 1.0f / sqrtf(static_cast<float>(D.d));
    a.theta = L->rope_theta;
    set_role(R_ATTENTION);
    DL_HIP(launch_attn_f32(a, s));
    set_role(R_O_DOWN);
    DL_HIP(gemm_f32(w.att, nullptr, L->o.A, w.to, M, D.ro, qd, qd, D.ro, F32_OUT_STORE, nullptr, 0,
                    nullptr, 1, 0, s));
    float *x2 = x2_out ? static_cast<float *>(x2_out) : w.x2;
    set_role(R_O_UP);
    DL_HIP(gemm_f32(w.to, nullptr, L->o.B, x2, M, h, D.ro, D.ro, h, F32_OUT_RESID, xf, h, nullptr,
                    1, 0, s));
    set_role(R_MLP_NORM);
    DL_HIP(launch_rmsnorm(x2, 1, L->mlp_norm, 1, w.b, 1, M, h, eps, s));
    set_role(R_GATE_UP_DOWN);
    if (!D.relu)
      DL_HIP(gemm_f32(w.b, nullptr, L->gate.A, w.tg, M, D.rg, h, h, D.rg, F32_OUT_STORE, nullptr, 0,
                      nullptr, 1, 0, s));
    DL_HIP(gemm_f32(w.b, nullptr, L->up.A, w.tu, M, D.ru, h, h, D.ru, F32_OUT_STORE, nullptr, 0,
                    nullptr, 1, 0, s));
    set_role(R_GATE_UP_UP);
    if (!D.relu)
      DL_HIP(gemm_f32(w.tg, nullptr, L->gate.B, w.G, M, D.f, D.rg, D.rg, D.f, F32_OUT_STORE, nullptr,
                      0, nullptr, 1, 0, s));
    DL_HIP(gemm_f32(w.tu, nullptr, L->up.B, w.U, M, D.f, D.ru, D.ru, D.f,
                    D.relu ? F32_OUT_RELU : F32_OUT_STORE, nullptr, 0, nullptr, 1, 0, s));
    set_role(R_DOWN_DOWN);
    // GLU: the down pair reads silu(G) * U, formed as it loads; non-GLU: relu(U)
    DL_HIP(gemm_f32(D.relu ? w.U : w.G, D.relu ? nullptr : w.U, L->down.A, w.td, M, D.rd, D.f, D.f,
                    D.rd, F32_OUT_STORE, nullptr, 0, nullptr, 1, 0, s));
    set_role(R_DOWN_UP);
    DL_HIP(gemm_f32(w.td, nullptr, L->down.B, static_cast<float *>(y), M, h, D.rd, D.rd, h,
                    F32_OUT_RESID, x2, h, nullptr, 1, 0, s));
    return DL_OK;
  }

  if (use_gemv(M)) {
    // a chunk of a chunked decode: the batch's query and attention buffers
    if (q_ext) w.q32 = q_ext;
    if (att_ext) w.att16 = att_ext;
    GvArgs g[G_NUM];
    layer_gemvs(L, D, w, x, y, x2_out, cache, past_lens, g);
    const bool fuse = fuse_mode() == FUSE_ALL;
    static const int roles[G_NUM] = {R_QKV_DOWN, R_Q_UP, R_O_DOWN, R_O_UP,
                                     R_GATE_UP_DOWN, R_GATE_UP_UP, R_DOWN_DOWN, R_DOWN_UP};
    if (phases & PH_PRE) {
      // the attention counters zeroed here are those of the launch that
      // follows: this step's, or the batch's (first chunk of a chunked decode)
      const AttnWS &az = aw_zero ? *aw_zero : aw;
      FillRegion zero[2] = {{reinterpret_cast<float *>(w.counters), nullptr, 0, w.n_counters},
                            {reinterpret_cast<float *>(az.counters), nullptr, 0, az.n_counters}};
      set_role(R_INIT);
      DL_HIP(launch_norm_tiles(static_cast<const uint16_t *>(x), L->attn_norm, L->dt == DL_F32,
                               L->rms_eps, w.a16t, M, static_cast<int>(mpad(M)), h, zero,
                               az.counters ? 2 : 1, s));
      // [A_q A_k A_v] then B_q as one chain (the query latents stay on chip)
      DL_HIP(gemv_sequence(&g[G_QKV], 2, w.part, w.counters, w.chain_sync, 1, fuse, &roles[G_QKV],
                           R_QKV_CHAIN, s));
    }
    if (phases & PH_ATTN) {
      set_role(R_ATTENTION);
      DL_HIP(run_attn_bf16(w.q32, 1, qd, cache, L->k.B, L->v.B, past_lens, 1, D.T == 1, w.att16, 0,
                           D.T == 1 ? 1 : 0, D.Bsz, D.T, D.nq, D.nkv, D.d, D.rk, D.rv, 0.f,
                           L->rope_theta, aw, s));
    }
    if (phases & PH_POST) {
      if (!(phases & PH_PRE)) {
        // other chunks' chains ran since this chunk's counters were zeroed
        FillRegion z[1] = {{reinterpret_cast<float *>(w.counters), nullptr, 0, w.n_counters}};
        set_role(R_INIT);
        DL_HIP(launch_fill(z, 1, s));
      }
      // the o pair, the MLP norm, the gate/up pairs with SwiGLU and the down
      // pair: six dependent GEMV stages in one chain (two runs when the
      // attention output arrives row-major, T > 1)
      DL_HIP(gemv_sequence(&g[G_ODOWN], 6, w.part, w.counters, w.chain_sync + kChainSyncInts, 2,
                           fuse, &roles[G_ODOWN], R_O_MLP_CHAIN, s));
    }
    return DL_OK;
  }

  // bf16 GEMM path. Every activation the step produces and a GEMM reads is
  // stored in operand tiles (a16, tq16, att16, to16, b16, tg16, tu16, G16,
  // td16), so the GEMMs stage each activation fragment as one contiguous 1 KB.
  set_role(R_ATTN_NORM);
  DL_HIP(launch_rmsnorm(x, 0, L->attn_norm, gf32, w.a16, RMS_Y_TILED, M, h, eps, s));
  {
    // the concatenated down factors [A_q, A_k, A_v] in one launch; the k
    // and v segments scatter their latents into the caches
    GemmArgs a{};
    a.nseg = 3;
    a.M = M;
    a.K = h;
    a.omode = GEMM_OUT_BF16;
    a.past_lens = past_lens;
    a.T = D.T;
    a.block_table = cache.table;
    a.page_stride = cache.stride;
    a.xmode = GEMM_X_TILED;
    a.seg[0] = mseg(L->q.A, w.a16, w.tq16, D.rq, h, D.rq);
    a.seg[0].c_tiled = 1;
    a.seg[1] = mseg(L->k.A, w.a16, Ck, D.rk, h, D.rk);
    a.seg[1].omode = GEMM_OUT_CACHE;
    a.seg[2] = mseg(L->v.A, w.a16, Cv, D.rv, h, D.rv);
    a.seg[2].omode = GEMM_OUT_CACHE_T;
    set_role(R_QKV_DOWN);
    DL_HIP(gemm(a, s, w.gpart, w.gpart_bytes));
    GemmArgs q{};
    q.nseg = 1;
    q.M = M;
    q.K = D.rq;
    q.omode = GEMM_OUT_BF16;
    q.xmode = GEMM_X_TILED;
    q.seg[0] = mseg(L->q.B, w.tq16, w.q16, qd, D.rq, qd);
    set_role(R_Q_UP);
    DL_HIP(gemm(q, s, w.gpart, w.gpart_bytes));
  }
  set_role(R_ATTENTION);
  if (aw.counters) {
    FillRegion z[1] = {{reinterpret_cast<float *>(aw.counters), nullptr, 0, aw.n_counters}};
    set_role(R_INIT);
    DL_HIP(launch_fill(z, 1, s));
    set_role(R_ATTENTION);
  }
  DL_HIP(run_attn_bf16(w.q16, 0, qd, cache, L->k.B, L->v.B, past_lens, 1, D.T == 1, w.att16, 0, 1,
                       D.Bsz, D.T, D.nq, D.nkv, D.d, D.rk, D.rv, 0.f, L->rope_theta, aw, s));
  {
    GemmArgs a{};
    a.nseg = 1;
    a.M = M;
    a.K = qd;
    a.omode = GEMM_OUT_BF16;
    a.xmode = GEMM_X_TILED;
    a.seg[0] = mseg(L->o.A, w.att16, w.to16, D.ro, qd, D.ro);
    a.seg[0].c_tiled = 1;
    set_role(R_O_DOWN);
    DL_HIP(gemm(a, s, w.gpart, w.gpart_bytes));
    GemmArgs b{};
    b.nseg = 1;
    b.M = M;
    b.K = D.ro;
    b.omode = GEMM_OUT_F32_RES_BF16;
    b.xmode = GEMM_X_TILED;
    b.seg[0] = mseg(L->o.B, w.to16, nullptr, h, D.ro, h);
    b.seg[0].C32 = w.x2f;
    b.seg[0].R = x;
    b.seg[0].ldr = h;
    set_role(R_O_UP);
    DL_HIP(gemm(b, s, w.gpart, w.gpart_bytes));
  }
  if (x2_out) {
    FillRegion cp[1] = {{static_cast<float *>(x2_out), w.x2f, 0, (int64_t)M * h}};
    set_role(R_OUTPUT);
    DL_HIP(launch_fill(cp, 1, s));
  }
  set_role(R_MLP_NORM);
  DL_HIP(launch_rmsnorm(w.x2f, 1, L->mlp_norm, gf32, w.b16, RMS_Y_TILED, M, h, eps, s));
  {
    GemmArgs a{};
    a.nseg = D.relu ? 1 : 2;
    a.M = M;
    a.K = h;
    a.omode = GEMM_OUT_BF16;
    if (D.relu) {
      a.seg[0] = mseg(L->up.A, w.b16, w.tu16, D.ru, h, D.ru);
    } else {
      a.seg[0] = mseg(L->gate.A, w.b16, w.tg16, D.rg, h, D.rg);
      a.seg[1] = mseg(L->up.A, w.b16, w.tu16, D.ru, h, D.ru);
    }
    a.xmode = GEMM_X_TILED;
    a.seg[0].c_tiled = a.seg[1].c_tiled = 1;
    set_role(R_GATE_UP_DOWN);
    DL_HIP(gemm(a, s, w.gpart, w.gpart_bytes));
  }
  if (D.relu) {
    // non-GLU MLP: H = relu(t_u B_up), into the buffer the down pair reads
    GemmArgs a{};
    a.nseg = 1;
    a.M = M;
    a.K = D.ru;
    a.omode = GEMM_OUT_RELU;
    a.xmode = GEMM_X_TILED;
    a.seg[0] = mseg(L->up.B, w.tu16, w.G16, D.f, D.ru, D.f);
    a.seg[0].c_tiled = 1;
    set_role(R_GATE_UP_UP);
    DL_HIP(gemm(a, s, w.gpart, w.gpart_bytes));
  } else {
    // G = t_g B_g, then the up product's epilogue forms H = silu(G) * (t_u B_u)
    // in place over G
    GemmArgs a{};
    a.nseg = 1;
    a.M = M;
    a.K = D.rg;
    a.omode = GEMM_OUT_BF16;
    a.xmode = GEMM_X_TILED;
    a.seg[0] = mseg(L->gate.B, w.tg16, w.G16, D.f, D.rg, D.f);
    a.seg[0].c_tiled = 1;
    set_role(R_GATE_UP_UP);
    DL_HIP(gemm(a, s, w.gpart, w.gpart_bytes));
    a.K = D.ru;
    a.omode = GEMM_OUT_SWIGLU;
    a.seg[0] = mseg(L->up.B, w.tu16, w.G16, D.f, D.ru, D.f);
    a.seg[0].c_tiled = a.seg[0].r_tiled = 1;
    a.seg[0].R = w.G16;
    a.seg[0].ldr = D.f;
    DL_HIP(gemm(a, s, w.gpart, w.gpart_bytes));
  }
  {
    GemmArgs a{};
    a.nseg = 1;
    a.M = M;
    a.K = D.f;
    a.xmode = GEMM_X_TILED;
    a.omode = GEMM_OUT_BF16;
    a.seg[0] = mseg(L->down.A, w.G16, w.td16, D.rd, D.f, D.rd);
    a.seg[0].c_tiled = 1;
    set_role(R_DOWN_DOWN);
    DL_HIP(gemm(a, s, w.gpart, w.gpart_bytes));
    GemmArgs b{};
    b.nseg = 1;
    b.M = M;
    b.K = D.rd;
    b.omode = GEMM_OUT_BF16_RES_F32;
    b.xmode = GEMM_X_TILED;
    b.seg[0] = mseg(L->down.B, w.td16, y, h, D.rd, h);
    b.seg[0].R = w.x2f;
    b.seg[0].ldr = h;
    set_role(R_DOWN_UP);
    DL_HIP(gemm(b, s, w.gpart, w.gpart_bytes));
  }
  return DL_OK;
}

dl_status dl_decomposed_layer_fwd(const dl_layer *L, const void *x, void *y, void *x2_out,
                                  void *Ck, void *Cv, const int32_t *past_lens, int64_t Bsz,
                                  int64_t T, int64_t L_max, void *ws, size_t ws_bytes,
                                  void *stream) {
  set_role(R_OTHER);
  DL_CHECK(L, DL_ERR_INVALID_ARG, "null layer");
  DL_CHECK(Bsz > 0 && L_max > 0, DL_ERR_INVALID_ARG, "Bsz, T, L_max must be positive");
  return layer_impl(L, x, y, x2_out, contiguous_cache(Ck, Cv, Bsz, L_max), past_lens, Bsz, T, ws,
                    ws_bytes, stream);
}

dl_status dl_decomposed_layer_fwd_paged(const dl_layer *L, const void *x, void *y, void *x2_out,
                                        const dl_kv_cache *cache, const int32_t *past_lens,
                                        int64_t Bsz, int64_t T, void *ws, size_t ws_bytes,
                                        void *stream) {
  set_role(R_OTHER);
  DL_CHECK(L, DL_ERR_INVALID_ARG, "null layer");
  CacheRef c;
  const dl_status st = paged_cache(cache, L->dt, &c);
  if (st != DL_OK) return st;
  return layer_impl(L, x, y, x2_out, c, past_lens, Bsz, T, ws, ws_bytes, stream);
}

size_t dl_workspace_size(const dl_layer *L, int64_t Bsz, int64_t T, int64_t L_max) {
  return dl_layer_workspace(L, Bsz, T, L_max);
}

// ===========================================================================
// Storage conversion
// ===========================================================================
size_t dl_factor_bytes(int64_t rows, int64_t cols, dl_dtype dt) {
  if (rows <= 0 || cols <= 0 || !valid_dtype(dt)) return 0;
  return static_cast<size_t>(rows * cols) * (dt == DL_BF16 ? 2 : 4);
}

dl_status dl_pack_factor(const void *F, int64_t rows, int64_t cols, dl_dtype dt, void *out,
                         void *stream) {
  set_role(R_OTHER);
  DL_CHECK(valid_dtype(dt), DL_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  DL_CHECK(F && out, DL_ERR_INVALID_ARG, "null pointer");
  DL_CHECK(rows > 0 && cols > 0, DL_ERR_INVALID_ARG, "dims must be positive");
  DL_CHECK(rows <= INT32_MAX && cols <= INT32_MAX && rows * cols <= ((int64_t)1 << 34),
           DL_ERR_UNSUPPORTED, "dims too large");
  if (dt == DL_BF16)
    DL_CHECK(rows % 32 == 0 && cols % 16 == 0, DL_ERR_UNSUPPORTED,
             "bf16 factor storage needs rows %% 32 == 0 and cols %% 16 == 0");
  DL_CHECK(aligned16(F) && aligned16(out), DL_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
  DL_HIP(launch_pack_factor(F, static_cast<int>(rows), static_cast<int>(cols), dt == DL_BF16, out,
                            as_stream(stream)));
  return DL_OK;
}

static dl_status pack_cache_common(const void *k_src, const void *v_src, int64_t Bsz, int64_t L_max,
                                   int64_t r_k, int64_t r_v, dl_dtype dt, void *k_dst,
                                   void *v_dst, void *stream, int unpack) {
  set_role(R_OTHER);
  DL_CHECK(valid_dtype(dt), DL_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  DL_CHECK(k_src && v_src && k_dst && v_dst, DL_ERR_INVALID_ARG, "null pointer");
  DL_CHECK(Bsz > 0 && L_max > 0 && r_k > 0 && r_v > 0, DL_ERR_INVALID_ARG, "dims must be positive");
  DL_CHECK(Bsz * L_max <= INT32_MAX && r_k <= INT32_MAX && r_v <= INT32_MAX &&
               Bsz * L_max * std::max(r_k, r_v) <= ((int64_t)1 << 36),
           DL_ERR_UNSUPPORTED, "dims too large");
  if (dt == DL_BF16)
    DL_CHECK(L_max % kPage == 0 && r_k % 32 == 0 && r_v % 32 == 0, DL_ERR_UNSUPPORTED,
             "bf16 caches need L_max %% %d == 0 and r_k, r_v multiples of 32", kPage);
  DL_CHECK(aligned16(k_src) && aligned16(v_src) && aligned16(k_dst) && aligned16(v_dst),
           DL_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
  hipStream_t s = as_stream(stream);
  const int B = static_cast<int>(Bsz), Lm = static_cast<int>(L_max);
  DL_HIP(launch_pack_cache(k_src, k_dst, B, Lm, static_cast<int>(r_k), 0, unpack, dt == DL_BF16, s));
  DL_HIP(launch_pack_cache(v_src, v_dst, B, Lm, static_cast<int>(r_v), 1, unpack, dt == DL_BF16, s));
  return DL_OK;
}

dl_status dl_pack_kv_cache(const void *Ck, const void *Cv, int64_t Bsz, int64_t L_max, int64_t r_k,
                           int64_t r_v, dl_dtype dt, void *Ck_lib, void *Cv_lib, void *stream) {
  return pack_cache_common(Ck, Cv, Bsz, L_max, r_k, r_v, dt, Ck_lib, Cv_lib, stream, 0);
}

dl_status dl_unpack_kv_cache(const void *Ck_lib, const void *Cv_lib, int64_t Bsz, int64_t L_max,
                             int64_t r_k, int64_t r_v, dl_dtype dt, void *Ck, void *Cv,
                             void *stream) {
  return pack_cache_common(Ck_lib, Cv_lib, Bsz, L_max, r_k, r_v, dt, Ck, Cv, stream, 1);
}

}  // extern "C"
