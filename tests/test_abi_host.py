"""Host-side ABI checks (no GPU): the library loads, exports every entry
point declared in include/dl.h, and rejects bad arguments with the documented
status before any HIP call."""
import ctypes
import os
import re

import pytest

from rank_decomposed_linear_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dl.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE = 0, 1, 2, 3, 4
P = 0x10000          # a 16-byte aligned stand-in pointer; validation rejects before any use
BAD = 0x10008        # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libdlayer.so not built")
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dl_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_five_entry_points():
    fns = declared_functions()
    for f in ("dl_lowrank_linear", "dl_lowrank_kv_append", "dl_lowrank_attn_decode",
              "dl_lowrank_attn_prefill", "dl_decomposed_layer_fwd"):
        assert f in fns


def test_every_declared_symbol_is_exported(lib):
    so = ctypes.CDLL(B.LIB_PATH)
    for f in declared_functions():
        assert hasattr(so, f), f
    assert set(B.EXPORTS) == set(declared_functions())


def err(lib):
    return lib.dl_last_error().decode()


def test_lowrank_linear_validation(lib):
    ws = 1 << 30
    f = lib.dl_lowrank_linear
    assert f(None, P, P, P, 16, 64, 64, 64, B.DL_BF16, P, ws, None) == INVALID
    assert f(P, P, P, P, 0, 64, 64, 64, B.DL_BF16, P, ws, None) == INVALID
    assert f(P, P, P, P, 16, 64, 64, 64, 7, P, ws, None) == INVALID
    assert f(P, P, P, P, 16, 64, 48, 64, B.DL_BF16, P, ws, None) == UNSUPPORTED
    assert "multiples of 64" in err(lib)
    assert f(P, BAD, P, P, 16, 64, 64, 64, B.DL_BF16, P, ws, None) == ALIGN
    need = lib.dl_lowrank_linear_workspace(16, 64, 64, 64, B.DL_BF16)
    assert need > 0
    assert f(P, P, P, P, 16, 64, 64, 64, B.DL_BF16, P, need - 1, None) == WORKSPACE
    assert f(P, P, P, P, 16, 64, 64, 64, B.DL_BF16, None, need, None) == WORKSPACE
    # f32 accepts ragged sizes (validation passes up to the workspace check)
    need32 = lib.dl_lowrank_linear_workspace(3, 5, 7, 9, B.DL_F32)
    assert f(P, P, P, P, 3, 5, 7, 9, B.DL_F32, P, need32 - 1, None) == WORKSPACE


def test_lowrank_linear_static_validation(lib):
    """The allocation-free variant rejects bad arguments, and products whose
    workspace exceeds the static scratch, before touching the device."""
    f = lib.dl_lowrank_linear_static
    assert f(P, P, P, P, 16, 64, 64, 64, 7, None) == INVALID
    assert f(P, P, P, P, 0, 64, 64, 64, B.DL_BF16, None) == INVALID
    need = lib.dl_lowrank_linear_workspace(4096, 4096, 4096, 64, B.DL_BF16)
    assert need > B.STATIC_SCRATCH_BYTES
    assert f(P, P, P, P, 4096, 4096, 4096, 64, B.DL_BF16, None) == WORKSPACE
    assert "static scratch" in err(lib)


def test_kv_append_validation(lib):
    f = lib.dl_lowrank_kv_append
    assert f(P, P, P, P, P, None, 2, 1, 64, 64, 64, 64, B.DL_BF16, P, 1 << 20, None) == INVALID
    assert f(P, P, P, P, P, P, 2, 65, 64, 64, 64, 64, B.DL_BF16, P, 1 << 20, None) == INVALID
    assert f(P, P, P, P, P, P, 2, 1, 64, 96, 64, 64, B.DL_BF16, P, 1 << 20, None) == UNSUPPORTED
    # bf16 caches are 64-position pages: L_max must be a multiple of 64
    assert f(P, P, P, P, P, P, 2, 1, 64, 64, 64, 40, B.DL_BF16, P, 1 << 20, None) == UNSUPPORTED
    assert "cache pages" in err(lib)
    assert f(P, P, P, BAD, P, P, 2, 1, 64, 64, 64, 64, B.DL_BF16, P, 1 << 20, None) == ALIGN
    need = lib.dl_kv_append_workspace(2, 1, 64, 64, 64, B.DL_BF16)
    assert f(P, P, P, P, P, P, 2, 1, 64, 64, 64, 64, B.DL_BF16, P, need - 1, None) == WORKSPACE


def test_attention_validation(lib):
    dec = lib.dl_lowrank_attn_decode
    args = dict(Bsz=2, n_q=8, n_kv=2, d=128, r_k=64, r_v=64, L=64)

    def call(q=P, n_q=8, n_kv=2, d=128, r_k=64, r_v=64, dt=B.DL_BF16, ws=1 << 24, wsp=P,
             scale=0.0, theta=10000.0, L_max=64):
        return dec(q, P, P, P, P, P, P, 2, n_q, n_kv, d, r_k, r_v, L_max, scale, theta, dt, wsp, ws,
                   None)

    assert call(q=None) == INVALID
    assert call(n_kv=3) == INVALID
    assert "multiple of n_kv" in err(lib)
    assert call(d=96) == UNSUPPORTED
    assert call(r_k=100) == UNSUPPORTED
    assert call(L_max=96) == UNSUPPORTED                # bf16 cache pages need L_max % 64
    assert call(r_v=8256) == UNSUPPORTED                # above the largest rank (8192)
    assert call(n_q=34, n_kv=2) == UNSUPPORTED          # group of 17 > 16
    assert call(scale=-1.0) == INVALID
    assert call(q=BAD) == ALIGN
    assert call(ws=16) == WORKSPACE
    # f32 accepts any even head_dim: d = 6 passes the shape checks and is
    # rejected only by the later scale check (no launch is reached)
    assert call(d=6, dt=B.DL_F32, scale=-1.0) == INVALID
    assert call(d=7, dt=B.DL_F32, scale=-1.0) == UNSUPPORTED
    assert call(d=258, dt=B.DL_F32) == UNSUPPORTED
    pre = lib.dl_lowrank_attn_prefill
    assert pre(P, P, P, P, P, P, P, 2, 4, 12, 4, 128, 64, 64, 64, 0.0, 0.0, B.DL_BF16, P, 1 << 24,
               None) == UNSUPPORTED                      # group 3 not a power of two
    assert pre(P, P, P, P, P, P, P, 2, 80, 8, 2, 128, 64, 64, 64, 0.0, 0.0, B.DL_BF16, P, 1 << 24,
               None) == INVALID                          # T > L_max


def _layer(dt=B.DL_BF16, rank=64, hidden=256, ffn=512, n_q=4, n_kv=2, d=64):
    L = B.Layer()
    L.hidden, L.n_q, L.n_kv, L.head_dim, L.ffn = hidden, n_q, n_kv, d, ffn
    for nm in B.DecomposedLayer.NAMES:
        setattr(L, nm, B.Factor(P, P, rank))
    L.rms_eps, L.rope_theta, L.dt = 1e-5, 10000.0, dt
    return L


def test_layer_validation(lib):
    f = lib.dl_decomposed_layer_fwd
    L = _layer()
    need = lib.dl_layer_workspace(ctypes.byref(L), 2, 1, 64)
    assert need > 0
    assert f(ctypes.byref(L), P, P, None, P, P, P, 2, 1, 64, P, need - 1, None) == WORKSPACE
    assert f(None, P, P, None, P, P, P, 2, 1, 64, P, need, None) == INVALID
    assert f(ctypes.byref(L), P, P, None, P, P, P, 2, 0, 64, P, need, None) == INVALID
    assert f(ctypes.byref(L), P, P, BAD, P, P, P, 2, 1, 64, P, need, None) == ALIGN
    assert f(ctypes.byref(L), P, P, None, P, P, P, 2, 1, 96, P, need, None) == UNSUPPORTED
    L2 = _layer(rank=96)
    assert f(ctypes.byref(L2), P, P, None, P, P, P, 2, 1, 64, P, need, None) == UNSUPPORTED
    L3 = _layer()
    L3.gate = B.Factor(None, P, 64)
    assert f(ctypes.byref(L3), P, P, None, P, P, P, 2, 1, 64, P, need, None) == INVALID
    L4 = _layer(n_kv=3)
    assert f(ctypes.byref(L4), P, P, None, P, P, P, 2, 1, 64, P, need, None) == INVALID
    # workspace grows with the batch and is defined for both dtypes
    assert lib.dl_layer_workspace(ctypes.byref(L), 64, 1, 64) > need
    assert lib.dl_layer_workspace(ctypes.byref(_layer(dt=B.DL_F32, rank=5, hidden=20, ffn=30,
                                                      d=10)), 2, 3, 16) > 0


def test_probe_rejects_bad_arguments(lib):
    assert lib.dl_probe_mfma_bf16(None, 1, 1, None) == INVALID
    assert lib.dl_probe_mfma_bf16(P, 0, 1, None) == INVALID
    assert lib.dl_probe_mfma_bf16(P, 1, 0, None) == INVALID
    assert lib.dl_probe_mfma_bf16(P, 1 << 31, 1, None) == INVALID


def test_paged_and_pack_validation(lib):
    """Paged entry points reject a missing or f32 cache descriptor; the pack
    calls reject shapes their layouts cannot hold; no launch is reached."""
    c = B.KvCache(P, P, P, 4, 16)
    cref = ctypes.byref(c)
    dec = lib.dl_lowrank_attn_decode_paged
    assert dec(P, None, P, P, P, P, 2, 8, 2, 128, 64, 64, 0.0, 0.0, B.DL_BF16, P, 1 << 24,
               None) == INVALID
    assert dec(P, cref, P, P, P, P, 2, 8, 2, 128, 64, 64, 0.0, 0.0, B.DL_F32, P, 1 << 24,
               None) == UNSUPPORTED
    assert "bf16 only" in err(lib)
    bad = B.KvCache(P, P, P, 0, 16)
    assert dec(P, ctypes.byref(bad), P, P, P, P, 2, 8, 2, 128, 64, 64, 0.0, 0.0, B.DL_BF16, P,
               1 << 24, None) == INVALID
    mis = B.KvCache(BAD, P, P, 4, 16)
    assert dec(P, ctypes.byref(mis), P, P, P, P, 2, 8, 2, 128, 64, 64, 0.0, 0.0, B.DL_BF16, P,
               1 << 24, None) == ALIGN
    app = lib.dl_lowrank_kv_append_paged
    assert app(P, P, P, cref, P, 2, 300, 64, 64, 64, B.DL_BF16, P, 1 << 20, None) == INVALID  # T > 4 pages
    L = _layer()
    assert lib.dl_workspace_size(ctypes.byref(L), 2, 1, 64) == lib.dl_layer_workspace(
        ctypes.byref(L), 2, 1, 64)
    fwd = lib.dl_decomposed_layer_fwd_paged
    assert fwd(ctypes.byref(L), P, P, None, None, P, 2, 1, P, 1 << 30, None) == INVALID
    assert lib.dl_pack_factor(P, 64, 40, B.DL_BF16, P, None) == UNSUPPORTED   # cols % 16
    assert lib.dl_pack_factor(P, 48, 64, B.DL_BF16, P, None) == UNSUPPORTED   # rows % 32
    assert lib.dl_pack_factor(None, 64, 64, B.DL_BF16, P, None) == INVALID
    assert lib.dl_factor_bytes(64, 32, B.DL_BF16) == 64 * 32 * 2
    assert lib.dl_pack_kv_cache(P, P, 2, 96, 64, 64, B.DL_BF16, P, P, None) == UNSUPPORTED
    assert lib.dl_unpack_kv_cache(P, P, 2, 64, 64, 48, B.DL_BF16, P, P, None) == UNSUPPORTED
    assert lib.dl_pack_kv_cache(P, P, 2, 64, 64, 64, B.DL_BF16, BAD, P, None) == ALIGN
