"""Thin Python binding of libdlayer.so (the C ABI in include/dl.h).

Argument marshalling only: every function here checks tensor placement,
allocates the caller-side workspace with torch, and calls the C entry point
of the same name on the current torch stream. All arithmetic runs in the
library's HIP kernels. If the library is not built or cannot be loaded, the
functions raise; there is no fallback.

Storage order is the library's (include/dl.h): every factor is passed
transposed (At = A^T [k, m], Bt = B^T [n, k]; up factors B_k^T, B_v^T
[n_kv * d, r]) and, for bf16, in 16 x 32 operand tiles; the key cache is
[Bsz, L_max, r_k]; the value cache is rank-major, for bf16 in 64-position
pages [Bsz, L_max / 64, r_v, 64] (f32: [Bsz, r_v, L_max]).
workloads.to_library_* give these orders on the host and pack_factor /
pack_kv_cache produce them on the GPU from the row-major forms. Sizes are
read from the tensors: L_max from the key cache, ranks from the factors.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdlayer.so")

DL_F32, DL_BF16 = 0, 1
STATIC_SCRATCH_BYTES = 16 << 20   # DL_STATIC_SCRATCH_BYTES
STATUS = {0: "DL_OK", 1: "DL_ERR_INVALID_ARG", 2: "DL_ERR_UNSUPPORTED", 3: "DL_ERR_ALIGNMENT",
          4: "DL_ERR_WORKSPACE", 5: "DL_ERR_HIP"}

EXPORTS = (
    "dl_last_error",
    "dl_lowrank_linear_workspace", "dl_lowrank_linear",
    "dl_lowrank_linear_static",
    "dl_kv_append_workspace", "dl_lowrank_kv_append", "dl_lowrank_kv_append_paged",
    "dl_attn_decode_workspace", "dl_lowrank_attn_decode", "dl_lowrank_attn_decode_paged",
    "dl_attn_prefill_workspace", "dl_lowrank_attn_prefill", "dl_lowrank_attn_prefill_paged",
    "dl_layer_workspace", "dl_workspace_size", "dl_decomposed_layer_fwd",
    "dl_decomposed_layer_fwd_paged",
    "dl_factor_bytes", "dl_pack_factor", "dl_pack_kv_cache", "dl_unpack_kv_cache",
    "dl_trace_install", "dl_kernel_kind_name", "dl_role_name",
    "dl_probe_mfma_bf16",
)


class DLError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Factor(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("k", ctypes.c_int64)]


class Layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int64), ("n_q", ctypes.c_int64), ("n_kv", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("ffn", ctypes.c_int64),
                ("q", Factor), ("k", Factor), ("v", Factor), ("o", Factor),
                ("gate", Factor), ("up", Factor), ("down", Factor),
                ("attn_norm", ctypes.c_void_p), ("mlp_norm", ctypes.c_void_p),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("dt", ctypes.c_int), ("mlp", ctypes.c_int)]

MLP_KINDS = {"glu": 0, "relu": 1}   # dl_mlp: DL_MLP_GLU, DL_MLP_RELU


class KvCache(ctypes.Structure):
    """dl_kv_cache: page pools, block table, pages per sequence, pool size."""
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("pages_per_seq", ctypes.c_int64),
                ("num_pages", ctypes.c_int64)]


class TraceStruct(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)),
                ("kinds", ctypes.POINTER(ctypes.c_int32)),
                ("roles", ctypes.POINTER(ctypes.c_int32)),
                ("capacity", ctypes.c_int32), ("count", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None
_i64, _vp, _sz, _f = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float


def load() -> ctypes.CDLL:
    """Load libdlayer.so (built in-tree by rank_decomposed_linear_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m rank_decomposed_linear_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.dl_last_error.restype = ctypes.c_char_p
    lib.dl_last_error.argtypes = []
    lib.dl_lowrank_linear_workspace.restype = _sz
    lib.dl_lowrank_linear_workspace.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int]
    lib.dl_lowrank_linear.restype = ctypes.c_int
    lib.dl_lowrank_linear.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int,
                                      _vp, _sz, _vp]
    lib.dl_lowrank_linear_static.restype = ctypes.c_int
    lib.dl_lowrank_linear_static.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                             ctypes.c_int, _vp]
    lib.dl_kv_append_workspace.restype = _sz
    lib.dl_kv_append_workspace.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int]
    lib.dl_lowrank_kv_append.restype = ctypes.c_int
    lib.dl_lowrank_kv_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                         _i64, _i64, ctypes.c_int, _vp, _sz, _vp]
    lib.dl_attn_decode_workspace.restype = _sz
    lib.dl_attn_decode_workspace.argtypes = [_i64] * 7 + [ctypes.c_int]
    lib.dl_lowrank_attn_decode.restype = ctypes.c_int
    lib.dl_lowrank_attn_decode.argtypes = [_vp] * 7 + [_i64] * 7 + [_f, _f, ctypes.c_int, _vp,
                                                                     _sz, _vp]
    lib.dl_attn_prefill_workspace.restype = _sz
    lib.dl_attn_prefill_workspace.argtypes = [_i64] * 8 + [ctypes.c_int]
    lib.dl_lowrank_attn_prefill.restype = ctypes.c_int
    lib.dl_lowrank_attn_prefill.argtypes = [_vp] * 7 + [_i64] * 8 + [_f, _f, ctypes.c_int, _vp,
                                                                      _sz, _vp]
    lib.dl_layer_workspace.restype = _sz
    lib.dl_layer_workspace.argtypes = [ctypes.POINTER(Layer), _i64, _i64, _i64]
    lib.dl_decomposed_layer_fwd.restype = ctypes.c_int
    lib.dl_decomposed_layer_fwd.argtypes = [ctypes.POINTER(Layer), _vp, _vp, _vp, _vp, _vp, _vp,
                                            _i64, _i64, _i64, _vp, _sz, _vp]
    _kc = ctypes.POINTER(KvCache)
    lib.dl_lowrank_kv_append_paged.restype = ctypes.c_int
    lib.dl_lowrank_kv_append_paged.argtypes = [_vp, _vp, _vp, _kc, _vp, _i64, _i64, _i64, _i64,
                                               _i64, ctypes.c_int, _vp, _sz, _vp]
    lib.dl_lowrank_attn_decode_paged.restype = ctypes.c_int
    lib.dl_lowrank_attn_decode_paged.argtypes = [_vp, _kc, _vp, _vp, _vp, _vp] + [_i64] * 6 + [
        _f, _f, ctypes.c_int, _vp, _sz, _vp]
    lib.dl_lowrank_attn_prefill_paged.restype = ctypes.c_int
    lib.dl_lowrank_attn_prefill_paged.argtypes = [_vp, _kc, _vp, _vp, _vp, _vp] + [_i64] * 7 + [
        _f, _f, ctypes.c_int, _vp, _sz, _vp]
    lib.dl_workspace_size.restype = _sz
    lib.dl_workspace_size.argtypes = [ctypes.POINTER(Layer), _i64, _i64, _i64]
    lib.dl_decomposed_layer_fwd_paged.restype = ctypes.c_int
    lib.dl_decomposed_layer_fwd_paged.argtypes = [ctypes.POINTER(Layer), _vp, _vp, _vp, _kc, _vp,
                                                  _i64, _i64, _vp, _sz, _vp]
    lib.dl_factor_bytes.restype = _sz
    lib.dl_factor_bytes.argtypes = [_i64, _i64, ctypes.c_int]
    lib.dl_pack_factor.restype = ctypes.c_int
    lib.dl_pack_factor.argtypes = [_vp, _i64, _i64, ctypes.c_int, _vp, _vp]
    lib.dl_pack_kv_cache.restype = ctypes.c_int
    lib.dl_pack_kv_cache.argtypes = [_vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp]
    lib.dl_unpack_kv_cache.restype = ctypes.c_int
    lib.dl_unpack_kv_cache.argtypes = [_vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int, _vp, _vp,
                                       _vp]
    lib.dl_probe_mfma_bf16.restype = ctypes.c_int
    lib.dl_probe_mfma_bf16.argtypes = [_vp, _i64, _i64, _vp]
    lib.dl_trace_install.restype = None
    lib.dl_trace_install.argtypes = [ctypes.POINTER(TraceStruct)]
    lib.dl_kernel_kind_name.restype = ctypes.c_char_p
    lib.dl_kernel_kind_name.argtypes = [ctypes.c_int32]
    lib.dl_role_name.restype = ctypes.c_char_p
    lib.dl_role_name.argtypes = [ctypes.c_int32]
    _lib = lib
    return lib


def _hip_runtime() -> ctypes.CDLL:
    """The HIP runtime already loaded by torch (same soname as libdlayer's)."""
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    return hip


_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence


class KernelTrace:
    """Records a hipEvent pair around every kernel the library launches
    while installed (dl_trace_install). Use as a context manager; after a
    device synchronisation, records() yields (kind, role, milliseconds)."""

    def __init__(self, capacity: int = 4096):
        torch.cuda.init()
        self.hip = _hip_runtime()
        self.capacity = capacity
        self.events = (ctypes.c_void_p * (2 * capacity))()
        for i in range(2 * capacity):
            ev = ctypes.c_void_p()
            # timing-only events: no system-scope fence (cache writeback and
            # invalidate) at each record, which would also slow the next kernel;
            # records() is read after a device synchronisation
            if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), _EVENT_DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.events[i] = ev.value
        self.kinds = (ctypes.c_int32 * capacity)()
        self.roles = (ctypes.c_int32 * capacity)()
        self.st = TraceStruct(self.events, self.kinds, self.roles, capacity, 0)

    def __enter__(self):
        self.st.count = 0
        load().dl_trace_install(ctypes.byref(self.st))
        return self

    def __exit__(self, *exc):
        load().dl_trace_install(None)
        return False

    def records(self):
        lib = load()
        out = []
        for i in range(self.st.count):
            ms = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.events[2 * i],
                                            self.events[2 * i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed (synchronise first)")
            out.append((lib.dl_kernel_kind_name(self.kinds[i]).decode(),
                        lib.dl_role_name(self.roles[i]).decode(), float(ms.value)))
        return out

    def close(self):
        for i in range(2 * self.capacity):
            if self.events[i]:
                self.hip.hipEventDestroy(self.events[i])
                self.events[i] = None


def _check(status: int) -> None:
    if status != 0:
        raise DLError(status, load().dl_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DL_BF16
    if t.dtype == torch.float32:
        return DL_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def probe_mfma_bf16(sink, blocks, iters):
    """dl_probe_mfma_bf16 on the current stream of sink's device; returns
    the flops the launch performs."""
    assert sink.dtype == torch.float32 and sink.numel() >= blocks * 512
    _check(load().dl_probe_mfma_bf16(_ptr(sink), blocks, iters, _stream(sink.device)))
    return blocks * 8 * iters * 32 * 16384


def lowrank_linear(x, At, Bt, y=None, ws=None):
    """y = (x A) B for x [M, m], At = A^T [k, m], Bt = B^T [n, k]
    (section 2.1, Eq. (1))."""
    lib = load()
    M, m = x.shape
    k, n = At.shape[0], Bt.shape[0]
    dt = _dt(x)
    if y is None:
        y = torch.empty((M, n), dtype=x.dtype, device=x.device)
    need = lib.dl_lowrank_linear_workspace(M, m, k, n, dt)
    ws = ws if ws is not None else _ws(need, x.device)
    _check(lib.dl_lowrank_linear(_ptr(x), _ptr(At), _ptr(Bt), _ptr(y), M, m, k, n, dt, _ptr(ws),
                                 ws.numel(), _stream(x.device)))
    return y


def lowrank_linear_static(x, At, Bt, y=None):
    """dl_lowrank_linear_static: y = (x A) B with the library's static
    scratch as the workspace (no allocation besides the output)."""
    lib = load()
    M, m = x.shape
    k, n = At.shape[0], Bt.shape[0]
    if y is None:
        y = torch.empty((M, n), dtype=x.dtype, device=x.device)
    _check(lib.dl_lowrank_linear_static(_ptr(x), _ptr(At), _ptr(Bt), _ptr(y), M, m, k, n, _dt(x),
                                        _stream(x.device)))
    return y


def lowrank_kv_append(x, A_kt, A_vt, ck, cv, past_lens, ws=None):
    """ck[b, past[b]+t, :] = x[b, t] A_k and cv[b, :, past[b]+t] = x[b, t] A_v;
    x [Bsz, T, m], A_kt [r_k, m], A_vt [r_v, m]."""
    lib = load()
    Bsz, T, m = x.shape
    r_k, r_v, L_max = A_kt.shape[0], A_vt.shape[0], ck.shape[1]
    dt = _dt(x)
    need = lib.dl_kv_append_workspace(Bsz, T, m, r_k, r_v, dt)
    ws = ws if ws is not None else _ws(need, x.device)
    _check(lib.dl_lowrank_kv_append(_ptr(x), _ptr(A_kt), _ptr(A_vt), _ptr(ck), _ptr(cv),
                                    _ptr(past_lens), Bsz, T, m, r_k, r_v, L_max, dt, _ptr(ws),
                                    ws.numel(), _stream(x.device)))


def lowrank_attn_decode(q, ck, cv, B_kt, B_vt, ctx_lens, n_kv, sm_scale=0.0, rope_theta=0.0,
                        out=None, ws=None):
    """q [Bsz, n_q, d] -> out [Bsz, n_q, d] (section 4.2); ck [Bsz, L_max, r_k],
    cv the value cache, B_kt [n_kv * d, r_k], B_vt [n_kv * d, r_v]."""
    lib = load()
    Bsz, n_q, d = q.shape
    L_max, r_k, r_v = ck.shape[1], B_kt.shape[1], B_vt.shape[1]
    dt = _dt(q)
    if out is None:
        out = torch.empty_like(q)
    need = lib.dl_attn_decode_workspace(Bsz, n_q, n_kv, d, r_k, r_v, L_max, dt)
    ws = ws if ws is not None else _ws(need, q.device)
    _check(lib.dl_lowrank_attn_decode(_ptr(q), _ptr(ck), _ptr(cv), _ptr(B_kt), _ptr(B_vt),
                                      _ptr(ctx_lens), _ptr(out), Bsz, n_q, n_kv, d, r_k, r_v,
                                      L_max, sm_scale, rope_theta, dt, _ptr(ws), ws.numel(),
                                      _stream(q.device)))
    return out


def lowrank_attn_prefill(q, ck, cv, B_kt, B_vt, past_lens, n_kv, sm_scale=0.0, rope_theta=0.0,
                         out=None, ws=None):
    """q [Bsz, T, n_q, d] -> out [Bsz, T, n_q, d], causal (section 4.2);
    cache and factor storage as in lowrank_attn_decode."""
    lib = load()
    Bsz, T, n_q, d = q.shape
    L_max, r_k, r_v = ck.shape[1], B_kt.shape[1], B_vt.shape[1]
    dt = _dt(q)
    if out is None:
        out = torch.empty_like(q)
    need = lib.dl_attn_prefill_workspace(Bsz, T, n_q, n_kv, d, r_k, r_v, L_max, dt)
    ws = ws if ws is not None else _ws(need, q.device)
    _check(lib.dl_lowrank_attn_prefill(_ptr(q), _ptr(ck), _ptr(cv), _ptr(B_kt), _ptr(B_vt),
                                       _ptr(past_lens), _ptr(out), Bsz, T, n_q, n_kv, d, r_k, r_v,
                                       L_max, sm_scale, rope_theta, dt, _ptr(ws), ws.numel(),
                                       _stream(q.device)))
    return out


def kv_cache(pool_k, pool_v, block_table, num_pages):
    """dl_kv_cache over device page pools and a device int32 block table
    [Bsz, pages_per_seq]; keeps the tensors referenced."""
    c = KvCache(_ptr(pool_k), _ptr(pool_v), _ptr(block_table), block_table.shape[1], num_pages)
    c._keep = (pool_k, pool_v, block_table)
    return c


def lowrank_kv_append_paged(x, A_kt, A_vt, cache, past_lens, ws=None):
    """Append T latent rows per sequence through the block table."""
    lib = load()
    Bsz, T, m = x.shape
    r_k, r_v = A_kt.shape[0], A_vt.shape[0]
    dt = _dt(x)
    need = lib.dl_kv_append_workspace(Bsz, T, m, r_k, r_v, dt)
    ws = ws if ws is not None else _ws(need, x.device)
    _check(lib.dl_lowrank_kv_append_paged(_ptr(x), _ptr(A_kt), _ptr(A_vt), ctypes.byref(cache),
                                          _ptr(past_lens), Bsz, T, m, r_k, r_v, dt, _ptr(ws),
                                          ws.numel(), _stream(x.device)))


def lowrank_attn_decode_paged(q, cache, B_kt, B_vt, ctx_lens, n_kv, sm_scale=0.0, rope_theta=0.0,
                              out=None, ws=None):
    """Decode attention reading the cache through its block table."""
    lib = load()
    Bsz, n_q, d = q.shape
    r_k, r_v = B_kt.shape[1], B_vt.shape[1]
    dt = _dt(q)
    if out is None:
        out = torch.empty_like(q)
    L_max = cache.pages_per_seq * 64
    need = lib.dl_attn_decode_workspace(Bsz, n_q, n_kv, d, r_k, r_v, L_max, dt)
    ws = ws if ws is not None else _ws(need, q.device)
    _check(lib.dl_lowrank_attn_decode_paged(_ptr(q), ctypes.byref(cache), _ptr(B_kt), _ptr(B_vt),
                                            _ptr(ctx_lens), _ptr(out), Bsz, n_q, n_kv, d, r_k, r_v,
                                            sm_scale, rope_theta, dt, _ptr(ws), ws.numel(),
                                            _stream(q.device)))
    return out


def lowrank_attn_prefill_paged(q, cache, B_kt, B_vt, past_lens, n_kv, sm_scale=0.0,
                               rope_theta=0.0, out=None, ws=None):
    """Causal prefill attention reading the cache through its block table."""
    lib = load()
    Bsz, T, n_q, d = q.shape
    r_k, r_v = B_kt.shape[1], B_vt.shape[1]
    dt = _dt(q)
    if out is None:
        out = torch.empty_like(q)
    L_max = cache.pages_per_seq * 64
    need = lib.dl_attn_prefill_workspace(Bsz, T, n_q, n_kv, d, r_k, r_v, L_max, dt)
    ws = ws if ws is not None else _ws(need, q.device)
    _check(lib.dl_lowrank_attn_prefill_paged(_ptr(q), ctypes.byref(cache), _ptr(B_kt), _ptr(B_vt),
                                             _ptr(past_lens), _ptr(out), Bsz, T, n_q, n_kv, d, r_k,
                                             r_v, sm_scale, rope_theta, dt, _ptr(ws), ws.numel(),
                                             _stream(q.device)))
    return out


def factor_bytes(rows, cols, dtype) -> int:
    return load().dl_factor_bytes(rows, cols, DL_BF16 if dtype == torch.bfloat16 else DL_F32)


def pack_factor(F, out=None):
    """Library storage of F [rows, cols] row-major (A [m, k] or B [k, n]):
    F^T [cols, rows], operand-tiled for bf16 (dl_pack_factor)."""
    rows, cols = F.shape
    if out is None:
        out = torch.empty((cols, rows), dtype=F.dtype, device=F.device)
    _check(load().dl_pack_factor(_ptr(F), rows, cols, _dt(F), _ptr(out), _stream(F.device)))
    return out


def pack_kv_cache(ck, cv, ck_lib=None, cv_lib=None):
    """Row-major caches ck [Bsz, L_max, r_k], cv [Bsz, L_max, r_v] -> the
    library's contiguous caches (dl_pack_kv_cache)."""
    Bsz, L_max, r_k = ck.shape
    r_v = cv.shape[2]
    dt = _dt(ck)
    if ck_lib is None:
        ck_lib = torch.empty_like(ck)
    if cv_lib is None:
        shape = (Bsz, L_max // 64, r_v, 64) if dt == DL_BF16 else (Bsz, r_v, L_max)
        cv_lib = torch.empty(shape, dtype=cv.dtype, device=cv.device)
    _check(load().dl_pack_kv_cache(_ptr(ck), _ptr(cv), Bsz, L_max, r_k, r_v, dt, _ptr(ck_lib),
                                   _ptr(cv_lib), _stream(ck.device)))
    return ck_lib, cv_lib


def unpack_kv_cache(ck_lib, cv_lib, r_v):
    """Inverse of pack_kv_cache: row-major [Bsz, L_max, r] copies."""
    Bsz, L_max, r_k = ck_lib.shape
    dt = _dt(ck_lib)
    ck = torch.empty_like(ck_lib)
    cv = torch.empty((Bsz, L_max, r_v), dtype=cv_lib.dtype, device=cv_lib.device)
    _check(load().dl_unpack_kv_cache(_ptr(ck_lib), _ptr(cv_lib), Bsz, L_max, r_k, r_v, dt,
                                     _ptr(ck), _ptr(cv), _stream(ck_lib.device)))
    return ck, cv


class DecomposedLayer:
    """Device-resident factor pairs of one layer plus the dl_layer descriptor.

    factors: dict name -> (At [k, m], Bt [n, k]) torch tensors on the GPU
    (each factor stored transposed) for q, k, v, o, gate, up, down; norm
    gains optional. mlp: "glu" (SwiGLU) or "relu" (the non-GLU MLP; no gate
    factor needed)."""

    NAMES = ("q", "k", "v", "o", "gate", "up", "down")

    def __init__(self, factors, hidden, n_q, n_kv, head_dim, ffn, rope_theta, rms_eps=1e-5,
                 attn_norm=None, mlp_norm=None, mlp="glu"):
        self.factors = factors
        self.attn_norm, self.mlp_norm = attn_norm, mlp_norm
        dt = _dt(factors["q"][0])
        L = Layer()
        L.hidden, L.n_q, L.n_kv, L.head_dim, L.ffn = hidden, n_q, n_kv, head_dim, ffn
        for nm in self.NAMES:
            if nm not in factors:
                continue
            At, Bt = factors[nm]
            setattr(L, nm, Factor(_ptr(At), _ptr(Bt), At.shape[0]))
        L.mlp = MLP_KINDS[mlp]
        L.attn_norm = _ptr(attn_norm)
        L.mlp_norm = _ptr(mlp_norm)
        L.rms_eps = rms_eps
        L.rope_theta = rope_theta
        L.dt = dt
        self.desc = L
        self.device = factors["q"][0].device

    def workspace_bytes(self, Bsz, T, L_max) -> int:
        return load().dl_workspace_size(ctypes.byref(self.desc), Bsz, T, L_max)

    def forward_paged(self, x, cache, past_lens, y=None, x2_out=None, ws=None, stream=None):
        """The layer over a paged cache (KvCache from kv_cache())."""
        lib = load()
        Bsz, T, _ = x.shape
        if y is None:
            y = torch.empty_like(x)
        if ws is None:
            ws = _ws(self.workspace_bytes(Bsz, T, cache.pages_per_seq * 64), x.device)
        s = stream.cuda_stream if stream is not None else _stream(x.device)
        _check(lib.dl_decomposed_layer_fwd_paged(ctypes.byref(self.desc), _ptr(x), _ptr(y),
                                                 _ptr(x2_out), ctypes.byref(cache),
                                                 _ptr(past_lens), Bsz, T, _ptr(ws), ws.numel(), s))
        return y

    def forward(self, x, ck, cv, past_lens, y=None, x2_out=None, ws=None, stream=None):
        """y = layer(x) for x [Bsz, T, hidden]; appends T latent rows per
        sequence at past_lens (not advanced). ck [Bsz, L_max, r_k],
        cv [Bsz, r_v, L_max]."""
        lib = load()
        Bsz, T, _ = x.shape
        L_max = ck.shape[1]
        if y is None:
            y = torch.empty_like(x)
        if ws is None:
            ws = _ws(self.workspace_bytes(Bsz, T, L_max), x.device)
        s = stream.cuda_stream if stream is not None else _stream(x.device)
        _check(lib.dl_decomposed_layer_fwd(ctypes.byref(self.desc), _ptr(x), _ptr(y),
                                           _ptr(x2_out), _ptr(ck), _ptr(cv), _ptr(past_lens),
                                           Bsz, T, L_max, _ptr(ws), ws.numel(), s))
        return y
