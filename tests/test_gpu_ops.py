"""GPU parity of the four single-op entry points against the fp64 oracle,
through the C ABI. Sizes span several tiles, ragged tails, both the GEMV
(M <= 64) and GEMM paths, ragged lengths, every supported GQA group and
head_dim, RoPE on and off, and both dtypes.

Inputs are drawn in the row-vector convention the oracle uses and uploaded
in the library's storage order (factors transposed, value cache rank-major,
bf16 factors and caches in operand tiles).

Tolerance: max|got - ref| / max|ref| <= 1e-4 (f32) and 2e-2 (bf16)."""
import numpy as np
import pytest

from oracle import ref
from rank_decomposed_linear_amd import workloads as W
from tests._helpers import TOL, f64, rand, relerr, to_dev, to_host

lib_f = W.to_library_factor
lib_ck = W.to_library_key_cache
lib_cv = W.to_library_value_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rank_decomposed_linear_amd import binding
    binding.load()
    return binding


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ----------------------------------------------------------------------------
# factor pair
# ----------------------------------------------------------------------------
LINEAR_CASES = [
    # (M, m, k, n, dtype)
    (1, 256, 64, 128, "bf16"),
    (16, 4096, 1216, 4096, "bf16"),     # the q pair of the 8B shape at 40%
    (37, 512, 448, 192, "bf16"),
    (64, 1024, 320, 576, "bf16"),
    (65, 512, 192, 320, "bf16"),
    (300, 256, 128, 448, "bf16"),
    (128, 512, 64, 64, "bf16"),
    (600, 1024, 320, 1088, "bf16"),     # several 256 x 256 GEMM tiles, ragged in M and N
    # long k ranges on few tiles: the GEMMs' k ranges are cut into parts
    # whose f32 partials a fixup kernel sums (all tiles: fewer than one
    # round; 2560 rows: 260 tiles of the first product, so a remainder of 4)
    (300, 8192, 1088, 320, "bf16"),
    (2560, 4096, 6656, 64, "bf16"),
    # 17 x 32 tiles of the second product: more than two rounds of tiles
    # over the compute units, ragged in M and N, four k tiles each
    (4100, 1024, 128, 8000, "bf16"),
    (2, 256, 64, 688, "f32"),
    (64, 688, 64, 256, "f32"),
    (100, 70, 9, 33, "f32"),
]


@pytest.mark.parametrize("M,m,k,n,dt", LINEAR_CASES)
def test_lowrank_linear(B, M, m, k, n, dt):
    print(f"lowrank_linear M={M} m={m} k={k} n={n} {dt}", flush=True)
    r = rng(M * 7 + k)
    x, A, Bf = rand(r, (M, m), 1.0, dt), rand(r, (m, k), 0.02, dt), rand(r, (k, n), 0.02, dt)
    y = B.lowrank_linear(to_dev(x), to_dev(lib_f(A)), to_dev(lib_f(Bf)))
    want = ref.lowrank_linear(f64(x), f64(A), f64(Bf))
    assert relerr(to_host(y), want) <= TOL[dt]


def test_lowrank_linear_split_plan(B):
    """The prefill GEMMs of the long-k cases above do take the remainder
    split: their workspace holds f32 partial tiles beyond the bf16
    intermediate (the cut is chosen by the device's compute-unit count)."""
    lib = B.load()
    for M, m, k, n in [(300, 8192, 1088, 320), (2560, 4096, 6656, 64)]:
        need = lib.dl_lowrank_linear_workspace(M, m, k, n, B.DL_BF16)
        assert need >= M * k * 2 + 2 * 256 * 256 * 4, (M, m, k, n, need)


@pytest.mark.parametrize("R", ["1", "2", "4"])
@pytest.mark.parametrize("M,m,k,n", [(16, 4096, 1216, 4096), (37, 512, 448, 192), (5, 2048, 128, 1088)])
def test_lowrank_linear_row_tiles(B, monkeypatch, R, M, m, k, n):
    """Every GEMV work-item width (one, two or four 16-row tiles sharing each
    activation fragment), forced through DL_GEMV_R, with K splits (the first
    factor) and without, and multi-block M (four-tile items fall back to two
    above 32 rows). bf16 factor pairs have m, k, n multiples of 64, so every
    item's tiles are real."""
    monkeypatch.setenv("DL_GEMV_R", R)
    print(f"lowrank_linear R={R} M={M} m={m} k={k} n={n}", flush=True)
    r = rng(M * 11 + n)
    x, A, Bf = rand(r, (M, m), 1.0, "bf16"), rand(r, (m, k), 0.02, "bf16"), rand(r, (k, n), 0.02, "bf16")
    y = B.lowrank_linear(to_dev(x), to_dev(lib_f(A)), to_dev(lib_f(Bf)))
    want = ref.lowrank_linear(f64(x), f64(A), f64(Bf))
    assert relerr(to_host(y), want) <= TOL["bf16"]


# ----------------------------------------------------------------------------
# cache append
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 7, 30])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_kv_append(B, T, dt):
    print(f"kv_append T={T} {dt}", flush=True)
    import torch
    r = rng(100 + T)
    Bsz, m, rk, rv, L_max = 3, 256, 128, 64, 64
    past = np.array([0, 5, 20], np.int32)
    x = rand(r, (Bsz, T, m), 1.0, dt)
    Ak, Av = rand(r, (m, rk), 0.02, dt), rand(r, (m, rv), 0.02, dt)
    ck0, cv0 = rand(r, (Bsz, L_max, rk), 1.0, dt), rand(r, (Bsz, L_max, rv), 1.0, dt)
    ck, cv = to_dev(lib_ck(ck0)), to_dev(lib_cv(cv0))
    B.lowrank_kv_append(to_dev(x), to_dev(lib_f(Ak)), to_dev(lib_f(Av)), ck, cv, to_dev(past))
    torch.cuda.synchronize()
    wk, wv = ref.kv_append(f64(x), f64(Ak), f64(Av), f64(ck0), f64(cv0), past)
    bf = dt == "bf16"
    gk, gv = W.from_library_key_cache(to_host(ck), bf), W.from_library_value_cache(to_host(cv), bf)
    for b in range(Bsz):
        rows = slice(past[b], past[b] + T)
        assert relerr(gk[b, rows], wk[b, rows]) <= TOL[dt]
        assert relerr(gv[b, rows], wv[b, rows]) <= TOL[dt]
        keep = np.ones(L_max, bool)
        keep[rows] = False
        # rows outside the append window are untouched, bit for bit
        assert np.array_equal(gk[b, keep], f64(ck0)[b, keep])
        assert np.array_equal(gv[b, keep], f64(cv0)[b, keep])


# ----------------------------------------------------------------------------
# decode attention
# ----------------------------------------------------------------------------
DECODE_CASES = [
    # (Bsz, n_q, n_kv, d, r_k, r_v, L_max, ctx_lens, theta, dtype)
    (3, 8, 2, 128, 448, 448, 320, [1, 130, 300], 500000.0, "bf16"),
    (2, 4, 4, 64, 64, 128, 64, [17, 40], 10000.0, "bf16"),
    (2, 16, 1, 128, 128, 64, 320, [255, 129], 0.0, "bf16"),
    (1, 64, 8, 128, 448, 448, 1152, [1025], 500000.0, "bf16"),
    (2, 32, 8, 128, 320, 384, 640, [600, 77], 500000.0, "bf16"),
    (2, 8, 2, 128, 640, 640, 2112, [2049, 700], 500000.0, "bf16"),   # ranks staged in chunks
    (1, 40, 8, 128, 64, 128, 576, [515], 10000.0, "bf16"),             # 5 heads per kv head
    (2, 12, 12, 64, 1024, 960, 192, [130, 64], 10000.0, "bf16"),       # largest ranks
    # several 64-position groups per wave: the running max shared across
    # groups, value products two groups behind, key tiles requested by the
    # group before (rank-step counts that are and are not multiples of the
    # prefetch depth), ragged and partial last groups
    (8, 32, 8, 128, 448, 448, 1088, [1025, 1000, 700, 1025, 513, 64, 1025, 999], 500000.0, "bf16"),
    (8, 16, 4, 128, 640, 640, 2112, [2049, 2049, 1900, 2000, 1, 2049, 1500, 2049], 500000.0,
     "bf16"),                                                          # ranks staged in chunks
    (16, 16, 4, 128, 64, 128, 2112, [2049] * 8 + [1111] * 8, 10000.0, "bf16"),   # 2 rank steps
    (16, 32, 8, 128, 128, 256, 1088, [1025] * 15 + [300], 500000.0, "bf16"),     # 4 rank steps
    (16, 8, 8, 128, 256, 256, 1088, [1025] * 16, 0.0, "bf16"),                   # MHA
    (8, 12, 12, 64, 1024, 960, 1088, [1025] * 7 + [777], 10000.0, "bf16"),
    # value ranks past the accumulators (r_v > 1024): U kept in the
    # workspace between context chunks, several value passes; MHA with the
    # LLaMA-65B ranks at 40% compression, d = 64
    (2, 8, 8, 128, 2432, 2432, 576, [512, 200], 10000.0, "bf16"),
    (3, 4, 4, 64, 1280, 1152, 640, [600, 1, 333], 10000.0, "bf16"),
    # rotary embedding off: attention in the latent space (B_k absorbed into
    # the query, B_v applied to P C_v); MHA with ranks past the rebuilding
    # kernel's limit, several context splits, head groups of 16 with a
    # partial last group, d = 64
    (4, 56, 56, 128, 2112, 2112, 576, [512, 100, 1, 575], 0.0, "bf16"),
    (2, 64, 8, 128, 448, 448, 8256, [8193, 3000], 0.0, "bf16"),
    (3, 40, 8, 64, 512, 640, 1088, [1025, 17, 700], 0.0, "bf16"),
    (2, 4, 4, 64, 64, 64, 40, [33, 40], 10000.0, "f32"),
    (2, 6, 2, 32, 12, 20, 50, [1, 50], 100.0, "f32"),
]


@pytest.mark.parametrize("case", DECODE_CASES)
def test_attn_decode(B, case):
    Bsz, n_q, n_kv, d, rk, rv, L_max, lens, theta, dt = case
    print(f"attn_decode {case}", flush=True)
    r = rng(200 + L_max + d)
    q = rand(r, (Bsz, n_q, d), 1.0, dt)
    ck, cv = rand(r, (Bsz, L_max, rk), 1.0, dt), rand(r, (Bsz, L_max, rv), 1.0, dt)
    Bk, Bv = rand(r, (rk, n_kv * d), 0.05, dt), rand(r, (rv, n_kv * d), 0.05, dt)
    lens = np.array(lens, np.int32)
    out = B.lowrank_attn_decode(to_dev(q), to_dev(lib_ck(ck)), to_dev(lib_cv(cv)), to_dev(lib_f(Bk)),
                                to_dev(lib_f(Bv)), to_dev(lens), n_kv, 0.0, theta)
    want = ref.attn_decode(f64(q), f64(ck), f64(cv), f64(Bk), f64(Bv), lens, n_kv, theta)
    assert relerr(to_host(out), want) <= TOL[dt]


# ----------------------------------------------------------------------------
# prefill attention
# ----------------------------------------------------------------------------
PREFILL_CASES = [
    # (Bsz, T, n_q, n_kv, d, r_k, r_v, L_max, past, theta, dtype)
    (2, 70, 8, 1, 128, 64, 64, 256, [0, 50], 10000.0, "bf16"),
    (2, 33, 8, 2, 64, 128, 64, 128, [5, 0], 500000.0, "bf16"),
    (1, 130, 4, 4, 128, 64, 128, 320, [100], 10000.0, "bf16"),
    (1, 20, 32, 2, 64, 64, 64, 64, [3], 0.0, "bf16"),
    (2, 1, 16, 2, 128, 448, 448, 320, [299, 10], 500000.0, "bf16"),
    (1, 200, 64, 8, 128, 448, 448, 256, [0], 500000.0, "bf16"),
    (2, 32, 4, 4, 64, 64, 64, 40, [0, 3], 10000.0, "f32"),
]


@pytest.mark.parametrize("case", PREFILL_CASES)
def test_attn_prefill(B, case):
    Bsz, T, n_q, n_kv, d, rk, rv, L_max, past, theta, dt = case
    print(f"attn_prefill {case}", flush=True)
    r = rng(300 + T + d)
    q = rand(r, (Bsz, T, n_q, d), 1.0, dt)
    ck, cv = rand(r, (Bsz, L_max, rk), 1.0, dt), rand(r, (Bsz, L_max, rv), 1.0, dt)
    Bk, Bv = rand(r, (rk, n_kv * d), 0.05, dt), rand(r, (rv, n_kv * d), 0.05, dt)
    past = np.array(past, np.int32)
    out = B.lowrank_attn_prefill(to_dev(q), to_dev(lib_ck(ck)), to_dev(lib_cv(cv)), to_dev(lib_f(Bk)),
                                 to_dev(lib_f(Bv)), to_dev(past), n_kv, 0.0, theta)
    want = ref.attn_prefill(f64(q), f64(ck), f64(cv), f64(Bk), f64(Bv), past, n_kv, theta)
    assert relerr(to_host(out), want) <= TOL[dt]


def test_explicit_softmax_scale(B):
    r = rng(5)
    Bsz, n_q, n_kv, d, rk, L_max = 2, 8, 2, 128, 64, 128
    q = rand(r, (Bsz, n_q, d), 1.0, "bf16")
    ck, cv = rand(r, (Bsz, L_max, rk), 1.0, "bf16"), rand(r, (Bsz, L_max, rk), 1.0, "bf16")
    Bk, Bv = rand(r, (rk, n_kv * d), 0.1, "bf16"), rand(r, (rk, n_kv * d), 0.1, "bf16")
    lens = np.array([70, 3], np.int32)
    out = B.lowrank_attn_decode(to_dev(q), to_dev(lib_ck(ck)), to_dev(lib_cv(cv)), to_dev(lib_f(Bk)),
                                to_dev(lib_f(Bv)), to_dev(lens), n_kv, 0.3, 1000.0)
    want = ref.attn_decode(f64(q), f64(ck), f64(cv), f64(Bk), f64(Bv), lens, n_kv, 1000.0, 0.3)
    assert relerr(to_host(out), want) <= TOL["bf16"]


def test_mfma_probe(B):
    """The matrix-pipe probe runs, writes every sink entry, and reports its flops."""
    import torch
    sink = torch.full((64 * 512,), float("nan"), dtype=torch.float32, device="cuda:0")
    flops = B.probe_mfma_bf16(sink, 64, 16)
    torch.cuda.synchronize()
    assert flops == 64 * 8 * 16 * 32 * 16384
    assert torch.isfinite(sink).all().item()


@pytest.mark.parametrize("R", ["1", "4"])
@pytest.mark.parametrize("M,m,k,n", [(16, 4096, 1216, 4096), (32, 8192, 448, 1024), (48, 1024, 320, 576)])
def test_fused_pair_matches_separate_launches(B, monkeypatch, R, M, m, k, n):
    """The decode-sized factor pair as one persistent launch (x A, then t B
    after an on-chip handoff, DL_FUSED_CHAIN=pair) and as two launches
    (none): the same work items, the same split order, so the same bits;
    both within tolerance of the oracle."""
    import torch
    monkeypatch.setenv("DL_GEMV_R", R)
    print(f"fused pair R={R} M={M} m={m} k={k} n={n}", flush=True)
    r = rng(M * 13 + k)
    x, A, Bf = rand(r, (M, m), 1.0, "bf16"), rand(r, (m, k), 0.02, "bf16"), rand(r, (k, n), 0.02, "bf16")
    xd, Ad, Bd = to_dev(x), to_dev(lib_f(A)), to_dev(lib_f(Bf))
    monkeypatch.setenv("DL_FUSED_CHAIN", "pair")
    y_fused = B.lowrank_linear(xd, Ad, Bd)
    monkeypatch.setenv("DL_FUSED_CHAIN", "none")
    y_sep = B.lowrank_linear(xd, Ad, Bd)
    torch.cuda.synchronize()
    assert torch.equal(y_fused, y_sep)
    assert relerr(to_host(y_fused), ref.lowrank_linear(f64(x), f64(A), f64(Bf))) <= TOL["bf16"]
