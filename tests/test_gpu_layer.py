"""GPU parity of dl_decomposed_layer_fwd against the fp64 oracle, on small
layers (both dtypes, GEMV and GEMM paths, decode and prefill, ragged cache
lengths) and on the five workload configurations at their full sizes.

For each check the attention delta (x2 - x) and the MLP delta (y - x2) are
compared separately, so the residual stream cannot hide an error, and the
appended cache rows are compared too. Tolerance as in test_gpu_ops.
Full-size configurations compare every sequence: the decode
configurations in one pass, the prefill configuration one sequence per test
(each sequence's rows depend only on that sequence), after one GPU run shared
by those tests. Inputs are uploaded in the library's storage
order (factors transposed, value cache rank-major, bf16 factors and caches
in operand tiles) and the caches are read back into the oracle's
[Bsz, L, r] order before comparing."""
import numpy as np
import pytest

from oracle import ref
from rank_decomposed_linear_amd import workloads as W
from tests._helpers import TOL, f64, rand, relerr, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rank_decomposed_linear_amd import binding
    binding.load()
    return binding


def make_gpu_layer(B, weights: W.LayerWeights):
    shp = weights.shape
    facs = {p: (to_dev(W.to_library_factor(a)), to_dev(W.to_library_factor(b)))
            for p, (a, b) in weights.factors.items()}
    gain = lambda g: None if g is None else to_dev(g)
    return B.DecomposedLayer(facs, shp.hidden, shp.n_q, shp.n_kv, shp.head_dim, shp.ffn,
                             shp.rope_theta, shp.rms_eps, attn_norm=gain(weights.attn_norm),
                             mlp_norm=gain(weights.mlp_norm), mlp=shp.mlp)


def oracle_layer(weights, x, ck, cv, past, seqs=None):
    shp = weights.shape
    sl = slice(None) if seqs is None else seqs
    F = {p: (f64(a), f64(b)) for p, (a, b) in weights.factors.items()}
    gain = lambda g: None if g is None else f64(g)
    return ref.decomposed_layer(F, f64(x)[sl], f64(ck)[sl], f64(cv)[sl], np.asarray(past)[sl],
                                shp.n_q, shp.n_kv, shp.head_dim, shp.rope_theta, shp.rms_eps,
                                attn_norm=gain(weights.attn_norm), mlp_norm=gain(weights.mlp_norm),
                                mlp=shp.mlp)


#: Bound on the residual-branch deltas (x2 - x and y - x2). The outputs
#: themselves (y, appended cache rows) are held to TOL, the stated bar. A
#: branch delta can be a small fraction of the residual stream, and the bf16
#: rounding of the branch's intermediates (latents, G, H) that bf16 layers may
#: apply is then large relative to it: on the 80-sequence small layer, a CPU
#: emulation of only that rounding, started from the exact x2, leaves 2.6% of
#: the MLP delta. A wrong term, index or operand moves a delta by O(100%).
DELTA_TOL = {"f32": TOL["f32"], "bf16": 2 * TOL["bf16"]}

#: unit roundoff of the stored outputs; y is stored in the layer dtype
#: (x2_out is always f32), so a delta recovered as y - x2 carries up to one
#: rounding of y plus one of x2 on top of the kernel's own error.
UNIT_ROUNDOFF = {"f32": 2.0 ** -24, "bf16": 2.0 ** -9}


def delta_err(got_delta, want_delta, stream_max, dt_y, dt_x2="f32"):
    """Relative error of a residual-branch delta after removing the part
    that the storage rounding of the stream values (|value| <= stream_max)
    can introduce: max(0, |d_gpu - d_ref| - (u_y + u_x2) * stream_max) / max|d_ref|."""
    slack = (UNIT_ROUNDOFF[dt_y] + UNIT_ROUNDOFF[dt_x2]) * stream_max
    excess = np.maximum(np.abs(got_delta - want_delta) - slack, 0.0)
    return float(np.max(excess)) / max(float(np.max(np.abs(want_delta))), 1e-30)


def check_step(dt, x, y_dev, x2_dev, ck_dev, cv_dev, want, past, T, seqs=None):
    import torch
    torch.cuda.synchronize()
    sl = slice(None) if seqs is None else seqs
    xh = f64(x)[sl]
    y, x2 = to_host(y_dev)[sl], to_host(x2_dev)[sl]
    smax = float(max(np.max(np.abs(want["y"])), np.max(np.abs(want["x2"]))))
    errs = {
        "attn_delta": delta_err(x2 - xh, want["x2"] - xh, smax, "f32"),
        "mlp_delta": delta_err(y - x2, want["y"] - want["x2"], smax, dt),
        "y": relerr(y, want["y"]),
    }
    bf = dt == "bf16"
    gk = W.from_library_key_cache(to_host(ck_dev), bf)[sl]
    gv = W.from_library_value_cache(to_host(cv_dev), bf)[sl]
    pst = np.asarray(past)[sl]
    for i in range(len(pst)):
        rows = slice(pst[i], pst[i] + T)
        errs[f"ck{i}"] = relerr(gk[i, rows], want["ck"][i, rows])
        errs[f"cv{i}"] = relerr(gv[i, rows], want["cv"][i, rows])
    bad = {k: v for k, v in errs.items()
           if not v <= (DELTA_TOL[dt] if k.endswith("_delta") else TOL[dt])}
    assert not bad, (bad, max(errs.values()))
    return errs


def run_layer(B, layer, x, ck, cv, past):
    import torch
    xd = to_dev(x)
    x2 = torch.empty(x.shape, dtype=torch.float32, device="cuda:0")
    y = layer.forward(xd, ck, cv, to_dev(np.asarray(past, np.int32)), x2_out=x2)
    return y, x2


# ----------------------------------------------------------------------------
# small layers
# ----------------------------------------------------------------------------
SMALL = [
    # (name, dtype, hidden, n_q, n_kv, d, ffn, rank_attn, rank_kv, rank_mlp, Bsz, T, past, L_max, theta)
    ("gemv_decode", "bf16", 512, 8, 2, 128, 1024, 192, 128, 256, 4, 1, [0, 7, 100, 33], 128, 500000.0),
    ("gemv_prefill", "bf16", 256, 4, 2, 64, 512, 128, 64, 192, 2, 8, [0, 20], 64, 10000.0),
    ("gemm_prefill", "bf16", 512, 8, 2, 128, 768, 256, 128, 320, 2, 100, [0, 20], 192, 10000.0),
    # hidden and FFN 4096 over 200 rows: the GEMMs with 4096-deep k ranges
    # (the latent scatter into the caches among them) run as k parts plus a
    # fixup that sums them
    ("gemm_prefill_ksplit", "bf16", 4096, 8, 2, 128, 4096, 256, 128, 320, 2, 100, [0, 20], 192,
     10000.0),
    ("gemm_decode_b80", "bf16", 256, 4, 1, 64, 512, 128, 64, 128, 80, 1, None, 64, 10000.0),
    # beyond 512 sequences decode runs on the GEMM path (tiled activations
    # from the decode attention into the o pair)
    ("gemm_decode_b520", "bf16", 256, 4, 1, 64, 512, 128, 64, 128, 520, 1, None, 64, 10000.0),
    ("gemv_decode_norope", "bf16", 512, 8, 2, 128, 1024, 192, 128, 256, 4, 1, [0, 7, 100, 33], 128, 0.0),
    ("gemm_decode_norope", "bf16", 256, 4, 1, 64, 512, 128, 64, 128, 80, 1, None, 64, 0.0),
    ("f32_prefill", "f32", 96, 4, 2, 16, 160, 24, 12, 40, 3, 6, [0, 2, 9], 20, 100.0),
    ("f32_decode", "f32", 96, 6, 3, 16, 160, 24, 12, 40, 3, 1, [0, 2, 9], 20, 100.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_layer(B, case, rank_up=None, gains=False, mlp="glu"):
    name, dt, h, nq, nkv, d, f, ra, rkv, rm, Bsz, T, past, L_max, theta = case
    print(f"layer {case} rank_up={rank_up} gains={gains} mlp={mlp}", flush=True)
    r = np.random.Generator(np.random.PCG64(sum(map(ord, name))))
    if past is None:
        past = list(r.integers(0, L_max - T, size=Bsz))
    shp_ranks = {"q": ra, "k": rkv, "v": rkv, "o": ra, "gate": rm, "up": rank_up or rm, "down": rm}
    projs = [p for p in W.PROJECTIONS if not (p == "gate" and mlp == "relu")]
    shp = W.LayerShape(h, nq, nkv, d, f, tuple((p, shp_ranks[p]) for p in projs), dt, theta,
                       mlp=mlp)
    facs = {}
    for p, (m, n) in shp.shapes().items():
        facs[p] = (rand(r, (m, shp.rank(p)), 0.05, dt), rand(r, (shp.rank(p), n), 0.05, dt))
    weights = W.LayerWeights(shp, facs)
    if gains:
        # distinct per-channel gains for the two norms (stored in the layer dtype)
        enc = lambda a: W.f32_to_bf16_bits(a) if dt == "bf16" else a.astype(np.float32)
        weights.attn_norm = enc(0.5 + r.random(h, dtype=np.float32))
        weights.mlp_norm = enc(0.5 + r.random(h, dtype=np.float32) * 1.5)
    x = rand(r, (Bsz, T, h), 1.0, dt)
    ck0 = rand(r, (Bsz, L_max, rkv), 1.0, dt)
    cv0 = rand(r, (Bsz, L_max, rkv), 1.0, dt)
    layer = make_gpu_layer(B, weights)
    ck, cv = to_dev(W.to_library_key_cache(ck0)), to_dev(W.to_library_value_cache(cv0))
    y, x2 = run_layer(B, layer, x, ck, cv, past)
    want = oracle_layer(weights, x, ck0, cv0, past)
    check_step(dt, x, y, x2, ck, cv, want, past, T)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_layer_relu_mlp(B, case):
    """The non-GLU MLP (relu of the up pair, then the down pair; no gate
    factor) on every path: the decode GEMV chain's ReLU tile epilogue, the
    prefill GEMM's ReLU epilogue, the f32 kernels."""
    test_small_layer(B, case, mlp="relu", gains=True)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_layer_norm_gains(B, case):
    """Non-unit RMSNorm gains on both norms: the decode path folds the MLP
    gain into the o pair's residual epilogue (gamma * x2 tiles) and the
    attention gain into the first normalisation; the prefill path applies
    both in its row kernels; the f32 path in its own kernels."""
    test_small_layer(B, case, gains=True)


@pytest.mark.parametrize("R", ["2", "4"])
@pytest.mark.parametrize("case", SMALL[:2], ids=[c[0] for c in SMALL[:2]])
def test_small_layer_row_tiles(B, monkeypatch, case, R):
    """The small-M layer with every GEMV on two- or four-tile work items
    (DL_GEMV_R): cache scatter, SwiGLU pairs, residual epilogue with the MLP
    norm's tiles and row sums, split merges."""
    monkeypatch.setenv("DL_GEMV_R", R)
    test_small_layer(B, case)


@pytest.mark.parametrize("case", [SMALL[2], SMALL[1]], ids=[SMALL[2][0], SMALL[1][0]])
def test_small_layer_unequal_mlp_ranks(B, case):
    """Gate and up factors of different rank: the prefill up GEMM (its own K)
    applies SwiGLU in its epilogue over the gate output; the decode GEMV pairs
    them with different K halves."""
    test_small_layer(B, case, rank_up=case[9] - 64)


# ----------------------------------------------------------------------------
# the workload configurations
# ----------------------------------------------------------------------------
def test_tiny_chain_prefill_then_decode(B):
    """Tiny MHA layer, f32: prefill 32 tokens, then 8 decode steps on fresh
    input vectors; every step and the cache compared to the oracle chain."""
    import torch
    w = W.TINY
    weights, inp = W.draw(w)
    layer = make_gpu_layer(B, weights)
    ck, cv = to_dev(W.to_library_key_cache(inp.ck)), to_dev(W.to_library_value_cache(inp.cv))
    ck_ref, cv_ref = f64(inp.ck), f64(inp.cv)
    past = np.zeros(w.batch, np.int32)
    steps = [inp.x] + [inp.decode_x[s] for s in range(w.decode_steps)]
    for s, x in enumerate(steps):
        print(f"tiny chain step {s} past={past.tolist()}", flush=True)
        y, x2 = run_layer(B, layer, x, ck, cv, past)
        F = {p: (f64(a), f64(b)) for p, (a, b) in weights.factors.items()}
        want = ref.decomposed_layer(F, f64(x), ck_ref, cv_ref, past, w.shape.n_q, w.shape.n_kv,
                                    w.shape.head_dim, w.shape.rope_theta, w.shape.rms_eps)
        check_step("f32", x, y, x2, ck, cv, want, past, x.shape[1])
        ck_ref, cv_ref = want["ck"], want["cv"]
        past = past + x.shape[1]
    torch.cuda.synchronize()
    assert relerr(W.from_library_key_cache(to_host(ck), False), ck_ref) <= TOL["f32"]


def _decode_config(B, w, seqs=None):
    weights, inp = W.draw(w)
    layer = make_gpu_layer(B, weights)
    ck, cv = to_dev(W.to_library_key_cache(inp.ck)), to_dev(W.to_library_value_cache(inp.cv))
    y, x2 = run_layer(B, layer, inp.x, ck, cv, inp.past_lens)
    want = oracle_layer(weights, inp.x, inp.ck, inp.cv, inp.past_lens, seqs)
    return check_step("bf16", inp.x, y, x2, ck, cv, want, inp.past_lens, 1, seqs)


def test_llama3_8b_c40_decode(B):
    print("llama3_8b_c40_decode all sequences", flush=True)
    _decode_config(B, W.LLAMA3_8B_C40_DECODE)


@pytest.mark.parametrize("w", W.LLAMA3_8B_SWEEP, ids=[f"c{w.compression_pct}" for w in W.LLAMA3_8B_SWEEP])
def test_llama3_8b_sweep_decode(B, w):
    print(f"{w.name} all sequences", flush=True)
    _decode_config(B, w)


def test_llama3_70b_c50_decode(B):
    print("llama3_70b_c50_decode all sequences", flush=True)
    _decode_config(B, W.LLAMA3_70B_C50_DECODE)


# The other foundation models of section 5.1 (MHA; OPT-30B with the non-GLU
# MLP and no rotary embedding) at their full layer sizes. The GPU runs the
# whole batch; the oracle, whose explicit K and V rebuild costs about 40
# GFLOP per sequence here, checks the listed sequences.
def test_llama65b_c40_decode(B):
    print("llama65b_c40_decode sequences 0 17 42 63", flush=True)
    _decode_config(B, W.LLAMA65B_C40_DECODE, np.array([0, 17, 42, 63]))


def test_opt30b_c40_decode(B):
    print("opt30b_c40_decode sequences 0 77 150 191", flush=True)
    _decode_config(B, W.OPT30B_C40_DECODE, np.array([0, 77, 150, 191]))


@pytest.mark.parametrize("w,seqs", [(W.LLAMA65B_C40_PREFILL, [0, 31, 63]),
                                    (W.OPT30B_C40_PREFILL, [0, 100, 191])],
                         ids=["llama65b_c40", "opt30b_c40"])
def test_mha_prefill_configs(B, w, seqs):
    import torch
    print(f"{w.name} sequences {seqs}", flush=True)
    weights, inp = W.draw(w)
    layer = make_gpu_layer(B, weights)
    ck, cv = to_dev(W.to_library_key_cache(inp.ck)), to_dev(W.to_library_value_cache(inp.cv))
    y, x2 = run_layer(B, layer, inp.x, ck, cv, inp.past_lens)
    sl = np.array(seqs)
    want = oracle_layer(weights, inp.x, inp.ck, inp.cv, inp.past_lens, sl)
    check_step("bf16", inp.x, y, x2, ck, cv, want, inp.past_lens, w.prefill, sl)
    del layer, ck, cv, y, x2
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def prefill_70b(B):
    """One GPU prefill step of the 70B 8 x 2048 workload; host copies of the
    outputs and caches, shared by the per-sequence comparisons."""
    import torch
    w = W.LLAMA3_70B_C50_PREFILL
    print("llama3_70b_c50_prefill: GPU step", flush=True)
    weights, inp = W.draw(w)
    layer = make_gpu_layer(B, weights)
    ck, cv = to_dev(W.to_library_key_cache(inp.ck)), to_dev(W.to_library_value_cache(inp.cv))
    y, x2 = run_layer(B, layer, inp.x, ck, cv, inp.past_lens)
    torch.cuda.synchronize()
    got = {"y": to_host(y), "x2": to_host(x2),
           "ck": W.from_library_key_cache(to_host(ck), True),
           "cv": W.from_library_value_cache(to_host(cv), True)}
    del layer, ck, cv, y, x2
    torch.cuda.empty_cache()
    return w, weights, inp, got


@pytest.mark.parametrize("seq", range(8))
def test_llama3_70b_c50_prefill(prefill_70b, seq):
    """Every sequence of the prefill batch, all 2048 rows: every row tile of
    the factor GEMMs, every query tile of the causal attention (including the
    heaviest-first work order) and every appended cache row."""
    w, weights, inp, got = prefill_70b
    print(f"llama3_70b_c50_prefill sequence {seq}", flush=True)
    sl = np.array([seq])
    want = oracle_layer(weights, inp.x, inp.ck, inp.cv, inp.past_lens, sl)
    xh = f64(inp.x)[sl]
    smax = float(max(np.max(np.abs(want["y"])), np.max(np.abs(want["x2"]))))
    errs = {
        "attn_delta": delta_err(got["x2"][sl] - xh, want["x2"] - xh, smax, "f32"),
        "mlp_delta": delta_err(got["y"][sl] - got["x2"][sl], want["y"] - want["x2"], smax, "bf16"),
        "y": relerr(got["y"][sl], want["y"]),
        "ck": relerr(got["ck"][seq, :w.prefill], want["ck"][0, :w.prefill]),
        "cv": relerr(got["cv"][seq, :w.prefill], want["cv"][0, :w.prefill]),
    }
    bad = {k: v for k, v in errs.items()
           if not v <= (DELTA_TOL["bf16"] if k.endswith("_delta") else TOL["bf16"])}
    assert not bad, (bad, errs)


@pytest.mark.parametrize("case", SMALL[:2], ids=[c[0] for c in SMALL[:2]])
def test_small_layer_fused_chains(B, monkeypatch, case):
    """The decode step's GEMV stages fused into two persistent launches
    (DL_FUSED_CHAIN=all): [A_q A_k A_v] -> B_q and o -> MLP norm -> gate/up
    -> SwiGLU -> down, including a first stage that reads row-major
    activations (T > 1)."""
    monkeypatch.setenv("DL_FUSED_CHAIN", "all")
    test_small_layer(B, case, gains=True)


def test_llama3_8b_c40_decode_fused_chains_bitwise(B, monkeypatch):
    """Full 8B decode step with the fused chains against the separate-launch
    path: identical bits for y, x2 and the appended cache rows, and the
    oracle for every sequence."""
    import torch
    w = W.LLAMA3_8B_C40_DECODE
    print(f"{w.name}: fused chains vs separate launches", flush=True)
    weights, inp = W.draw(w)
    layer = make_gpu_layer(B, weights)
    outs = []
    for mode in ("all", "none"):
        monkeypatch.setenv("DL_FUSED_CHAIN", mode)
        ck, cv = to_dev(W.to_library_key_cache(inp.ck)), to_dev(W.to_library_value_cache(inp.cv))
        y, x2 = run_layer(B, layer, inp.x, ck, cv, inp.past_lens)
        torch.cuda.synchronize()
        outs.append((y, x2, ck, cv))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    y, x2, ck, cv = outs[0]
    want = oracle_layer(weights, inp.x, inp.ck, inp.cv, inp.past_lens)
    check_step("bf16", inp.x, y, x2, ck, cv, want, inp.past_lens, 1)
