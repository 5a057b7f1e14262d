// Launch tracing shared by the kernel launchers (see dl_trace in dl.h).
#pragma once

#include <hip/hip_runtime.h>

namespace dl {

enum KernelKind : int {
  K_RMSNORM = 0,
  K_FILL,
  K_CONVERT,
  K_STORE_CACHE,
  K_GEMV_BF16,
  K_GEMM_BF16,
  K_GEMM_F32,
  K_PACK_UP,
  K_ATTN_DECODE,
  K_ATTN_COMBINE,
  K_ATTN_PREFILL,
  K_ATTN_F32,
  K_GEMV_CHAIN,
  K_ATTN_LATENT,
  K_NUM_KINDS
};

enum Role : int {
  R_OTHER = 0,
  R_ATTN_NORM,
  R_QKV_DOWN,
  R_KV_STORE,
  R_Q_UP,
  R_ATTENTION,
  R_O_DOWN,
  R_O_UP,
  R_MLP_NORM,
  R_GATE_UP_DOWN,
  R_GATE_UP_UP,
  R_DOWN_DOWN,
  R_DOWN_UP,
  R_OUTPUT,
  R_INIT,
  R_QKV_CHAIN,
  R_O_MLP_CHAIN,
  R_PAIR_CHAIN,
  R_NUM_ROLES
};

// Called by every launcher around its kernel launch.
void trace_begin(int kind, hipStream_t s);
void trace_end(hipStream_t s);
// Set by the orchestration code before each step.
void set_role(int role);

}  // namespace dl

namespace dl {
// Brackets one launcher's kernel with the trace events.
struct TraceGuard {
  hipStream_t s;
  TraceGuard(int kind, hipStream_t st) : s(st) { trace_begin(kind, s); }
  ~TraceGuard() { trace_end(s); }
};
}  // namespace dl
