"""GPU parity of the paged low-rank cache and of the storage-conversion calls
against the fp64 oracle, through the C ABI.

Paged cache (DeInfer section 4.2, Fig. 4(b)): the latents live in 64-position
pages of a pool, reached through a block table whose pages are shuffled and
interleaved between sequences; pool pages that no sequence owns hold
sentinels and must come back bit for bit. The oracle gathers each sequence
through its block-table row (oracle.ref.decomposed_layer_paged). A decode
step captured once in a HIP graph is replayed over several steps while the
lengths, inputs and block table change in device memory, crossing page
boundaries; every replay is compared with the oracle chain.

Storage conversion: dl_pack_factor / dl_pack_kv_cache must produce exactly
the layouts the host helpers describe, dl_unpack_kv_cache must invert the
cache packing, and a layer run from row-major factors and caches packed on
the GPU must match the oracle."""
import numpy as np
import pytest

from oracle import ref
from rank_decomposed_linear_amd import workloads as W
from tests._helpers import TOL, f64, rand, relerr, to_dev, to_host

pytestmark = pytest.mark.gpu
PAGE = W.PAGE


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rank_decomposed_linear_amd import binding
    binding.load()
    return binding


def small_shape(dt="bf16", theta=500000.0):
    ranks = {"q": 192, "k": 128, "v": 64, "o": 192, "gate": 256, "up": 256, "down": 256}
    return W.LayerShape(512, 8, 2, 128, 1024, tuple((p, ranks[p]) for p in W.PROJECTIONS), dt,
                        theta)


def draw_factors(r, shp, dt="bf16"):
    return {p: (rand(r, (m, shp.rank(p)), 0.05, dt), rand(r, (shp.rank(p), n), 0.05, dt))
            for p, (m, n) in shp.shapes().items()}


def gpu_layer(B, shp, facs):
    lf = W.to_library_factor
    return B.DecomposedLayer({p: (to_dev(lf(a)), to_dev(lf(b))) for p, (a, b) in facs.items()},
                             shp.hidden, shp.n_q, shp.n_kv, shp.head_dim, shp.ffn, shp.rope_theta,
                             shp.rms_eps)


def make_pool(r, Bsz, pages_per_seq, num_pages, rk, rv):
    """Row-major pools (bf16 bits) with random owned pages and sentinel
    values elsewhere, plus a shuffled block table."""
    table = W.random_block_table(r, Bsz, pages_per_seq, num_pages)
    pk = np.full((num_pages, PAGE, rk), W.f32_to_bf16_bits(np.float32(3.0)), np.uint16)
    pv = np.full((num_pages, PAGE, rv), W.f32_to_bf16_bits(np.float32(-3.0)), np.uint16)
    L = pages_per_seq * PAGE
    pk = W.scatter_to_pages(rand(r, (Bsz, L, rk), 1.0, "bf16"), table, pk)
    pv = W.scatter_to_pages(rand(r, (Bsz, L, rv), 1.0, "bf16"), table, pv)
    return table, pk, pv


def dev_pool(B, pk, pv, table):
    gk = to_dev(W.to_library_key_pages(pk))
    gv = to_dev(W.to_library_value_pages(pv))
    gt = to_dev(table)
    return gk, gv, gt, B.kv_cache(gk, gv, gt, pk.shape[0])


def _bits(t):
    """bf16 device tensor -> uint16 bit patterns on the host."""
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def compare_pools(got_k, got_v, want_k, want_v, owned_rows, tol):
    """Appended rows within tolerance, every other row bit-identical."""
    gk, gv = f64(got_k), f64(got_v)
    for (pg, row) in owned_rows:
        assert relerr(gk[pg, row], want_k[pg, row]) <= tol
        assert relerr(gv[pg, row], want_v[pg, row]) <= tol
    mask = np.ones(gk.shape[:2], bool)
    for (pg, row) in owned_rows:
        mask[pg, row] = False
    assert np.array_equal(gk[mask], want_k[mask])
    assert np.array_equal(gv[mask], want_v[mask])


# ----------------------------------------------------------------------------
# storage conversion
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_pack_factor_and_cache_match_host_layouts(B, dt):
    import torch
    r = np.random.Generator(np.random.PCG64(70))
    for rows, cols in ((256, 192), (64, 512)):
        print(f"pack_factor {dt} {rows}x{cols}", flush=True)
        F = rand(r, (rows, cols), 1.0, dt)
        got = B.pack_factor(to_dev(F))
        torch.cuda.synchronize()
        want = W.to_library_factor(F)
        if dt == "bf16":
            assert np.array_equal(_bits(got), want)
        else:
            assert np.array_equal(got.cpu().numpy(), want)
    Bsz, L_max, rk, rv = 3, 192, 96, 64
    ck, cv = rand(r, (Bsz, L_max, rk), 1.0, dt), rand(r, (Bsz, L_max, rv), 1.0, dt)
    print(f"pack_kv_cache {dt}", flush=True)
    gk, gv = B.pack_kv_cache(to_dev(ck), to_dev(cv))
    torch.cuda.synchronize()
    wk, wv = W.to_library_key_cache(ck), W.to_library_value_cache(cv)
    host = _bits if dt == "bf16" else (lambda t: t.cpu().numpy())
    assert np.array_equal(host(gk), wk) and np.array_equal(host(gv), wv)
    uk, uv = B.unpack_kv_cache(gk, gv, rv)
    torch.cuda.synchronize()
    assert np.array_equal(host(uk), ck) and np.array_equal(host(uv), cv)


def test_layer_from_row_major_inputs(B):
    """The pages' W ~ A B form end to end: row-major A [m, k], B [k, n] and
    caches [Bsz, L_max, r] uploaded as they are, converted on the GPU by the
    C ABI, one decode step, caches converted back, compared with the oracle."""
    import torch
    r = np.random.Generator(np.random.PCG64(71))
    shp = small_shape()
    facs = draw_factors(r, shp)
    Bsz, L_max = 4, 256
    past = np.array([0, 63, 64, 200], np.int32)
    x = rand(r, (Bsz, 1, shp.hidden), 1.0, "bf16")
    ck, cv = rand(r, (Bsz, L_max, 128), 1.0, "bf16"), rand(r, (Bsz, L_max, 64), 1.0, "bf16")
    packed = {p: (B.pack_factor(to_dev(a)), B.pack_factor(to_dev(b))) for p, (a, b) in facs.items()}
    layer = B.DecomposedLayer(packed, shp.hidden, shp.n_q, shp.n_kv, shp.head_dim, shp.ffn,
                              shp.rope_theta, shp.rms_eps)
    gk, gv = B.pack_kv_cache(to_dev(ck), to_dev(cv))
    x2 = torch.empty((Bsz, 1, shp.hidden), dtype=torch.float32, device="cuda:0")
    y = layer.forward(to_dev(x), gk, gv, to_dev(past), x2_out=x2)
    uk, uv = B.unpack_kv_cache(gk, gv, 64)
    torch.cuda.synchronize()
    F = {p: (f64(a), f64(b)) for p, (a, b) in facs.items()}
    want = ref.decomposed_layer(F, f64(x), f64(ck), f64(cv), past, shp.n_q, shp.n_kv,
                                shp.head_dim, shp.rope_theta, shp.rms_eps)
    assert relerr(to_host(y), want["y"]) <= TOL["bf16"]
    assert relerr(to_host(x2) - f64(x), want["x2"] - f64(x)) <= TOL["bf16"]
    hk, hv = f64(_bits(uk)), f64(_bits(uv))
    for b in range(Bsz):
        assert relerr(hk[b, past[b]], want["ck"][b, past[b]]) <= TOL["bf16"]
        assert relerr(hv[b, past[b]], want["cv"][b, past[b]]) <= TOL["bf16"]
        keep = np.arange(L_max) != past[b]
        assert np.array_equal(hk[b, keep], f64(ck)[b, keep])
        assert np.array_equal(hv[b, keep], f64(cv)[b, keep])


# ----------------------------------------------------------------------------
# paged cache
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T,past", [(1, [0, 63, 64, 200]), (70, [0, 100]), (8, [60, 1])],
                         ids=["decode_gemv", "prefill_gemm", "prefill_gemv"])
def test_paged_layer(B, T, past):
    """One layer step over a shuffled paged pool: outputs, appended rows, and
    untouched pages."""
    import torch
    print(f"paged layer T={T} past={past}", flush=True)
    r = np.random.Generator(np.random.PCG64(72 + T))
    shp = small_shape()
    facs = draw_factors(r, shp)
    Bsz, pages_per_seq = len(past), 4
    num_pages = Bsz * pages_per_seq + 5
    past = np.array(past, np.int32)
    table, pk, pv = make_pool(r, Bsz, pages_per_seq, num_pages, 128, 64)
    gk, gv, gt, cache = dev_pool(B, pk, pv, table)
    layer = gpu_layer(B, shp, facs)
    x = rand(r, (Bsz, T, shp.hidden), 1.0, "bf16")
    x2 = torch.empty((Bsz, T, shp.hidden), dtype=torch.float32, device="cuda:0")
    y = layer.forward_paged(to_dev(x), cache, to_dev(past), x2_out=x2)
    torch.cuda.synchronize()
    F = {p: (f64(a), f64(b)) for p, (a, b) in facs.items()}
    want = ref.decomposed_layer_paged(F, f64(x), f64(pk), f64(pv), table, past, shp.n_q,
                                      shp.n_kv, shp.head_dim, shp.rope_theta, shp.rms_eps)
    assert relerr(to_host(y), want["y"]) <= TOL["bf16"]
    assert relerr(to_host(x2) - f64(x), want["x2"] - f64(x)) <= TOL["bf16"]
    rows = [(table[b, (past[b] + t) // PAGE], (past[b] + t) % PAGE)
            for b in range(Bsz) for t in range(T)]
    compare_pools(W.from_library_key_pages(_bits(gk)), W.from_library_value_pages(_bits(gv)),
                  want["pool_k"], want["pool_v"], rows, TOL["bf16"])


@pytest.mark.parametrize("G,theta", [(4, 500000.0), (1, 0.0)])
def test_paged_attention_ops(B, G, theta):
    """Paged decode and prefill attention entry points on a shuffled pool."""
    import torch
    print(f"paged attention G={G} theta={theta}", flush=True)
    r = np.random.Generator(np.random.PCG64(80 + G))
    n_kv, d, rk, rv = 2, 128, 192, 128
    n_q = G * n_kv
    Bsz, pages_per_seq = 3, 5
    num_pages = Bsz * pages_per_seq + 2
    table, pk, pv = make_pool(r, Bsz, pages_per_seq, num_pages, rk, rv)
    gk, gv, gt, cache = dev_pool(B, pk, pv, table)
    Bk, Bv = rand(r, (rk, n_kv * d), 0.05, "bf16"), rand(r, (rv, n_kv * d), 0.05, "bf16")
    lens = np.array([1, 129, 320], np.int32)
    q = rand(r, (Bsz, n_q, d), 1.0, "bf16")
    out = B.lowrank_attn_decode_paged(to_dev(q), cache, to_dev(W.to_library_factor(Bk)),
                                      to_dev(W.to_library_factor(Bv)), to_dev(lens), n_kv, 0.0, theta)
    torch.cuda.synchronize()
    want = ref.attn_decode_paged(f64(q), f64(pk), f64(pv), table, f64(Bk), f64(Bv), lens, n_kv, theta)
    assert relerr(to_host(out), want) <= TOL["bf16"]
    T, past = 40, np.array([0, 70, 250], np.int32)
    qp = rand(r, (Bsz, T, n_q, d), 1.0, "bf16")
    outp = B.lowrank_attn_prefill_paged(to_dev(qp), cache, to_dev(W.to_library_factor(Bk)),
                                        to_dev(W.to_library_factor(Bv)), to_dev(past), n_kv, 0.0,
                                        theta)
    torch.cuda.synchronize()
    for b in range(Bsz):
        L = int(past[b]) + T
        ckb = ref.paged_gather(f64(pk), table[b], L)[None]
        cvb = ref.paged_gather(f64(pv), table[b], L)[None]
        wb = ref.attn_prefill(f64(qp)[b:b + 1], ckb, cvb, f64(Bk), f64(Bv), past[b:b + 1], n_kv,
                              theta)
        assert relerr(to_host(outp)[b:b + 1], wb) <= TOL["bf16"]


def test_paged_decode_attention_long(B):
    """Paged decode attention where every wave walks several position groups
    (16 sequences of up to 17 pages on a shuffled pool)."""
    import torch
    print("paged decode attention, long contexts", flush=True)
    r = np.random.Generator(np.random.PCG64(85))
    n_kv, G, d, rk, rv = 8, 4, 128, 448, 448
    n_q = G * n_kv
    Bsz, pages_per_seq = 16, 17
    num_pages = Bsz * pages_per_seq + 3
    table, pk, pv = make_pool(r, Bsz, pages_per_seq, num_pages, rk, rv)
    gk, gv, gt, cache = dev_pool(B, pk, pv, table)
    Bk, Bv = rand(r, (rk, n_kv * d), 0.05, "bf16"), rand(r, (rv, n_kv * d), 0.05, "bf16")
    lens = np.array([1025, 1088, 900, 65, 1025, 1025, 1, 640] * 2, np.int32)
    q = rand(r, (Bsz, n_q, d), 1.0, "bf16")
    out = B.lowrank_attn_decode_paged(to_dev(q), cache, to_dev(W.to_library_factor(Bk)),
                                      to_dev(W.to_library_factor(Bv)), to_dev(lens), n_kv, 0.0,
                                      500000.0)
    torch.cuda.synchronize()
    want = ref.attn_decode_paged(f64(q), f64(pk), f64(pv), table, f64(Bk), f64(Bv), lens, n_kv,
                                 500000.0)
    assert relerr(to_host(out), want) <= TOL["bf16"]


def test_paged_decode_graph_replay(B):
    """One decode step captured in a HIP graph, replayed six times while the
    device-resident inputs, lengths and block table advance (two sequences
    cross a page boundary and get a fresh pool page). Each replay is
    compared with the oracle chain over the same pool."""
    import torch
    r = np.random.Generator(np.random.PCG64(90))
    shp = small_shape()
    facs = draw_factors(r, shp)
    Bsz, pages_per_seq = 4, 4
    num_pages = Bsz * pages_per_seq + 4
    past = np.array([61, 126, 0, 190], np.int32)
    table, pk, pv = make_pool(r, Bsz, pages_per_seq, num_pages, 128, 64)
    # pages a sequence has not reached yet are unassigned (-1, never read);
    # they are handed out from the free pool pages as lengths grow
    owned = (past + 1 + PAGE - 1) // PAGE
    live = np.full_like(table, -1)
    for b in range(Bsz):
        live[b, :owned[b]] = table[b, :owned[b]]
    used = set(live[live >= 0].ravel().tolist())
    free = [p for p in range(num_pages) if p not in used]
    gk, gv, gt, cache = dev_pool(B, pk, pv, live)
    layer = gpu_layer(B, shp, facs)
    x_dev = torch.empty((Bsz, 1, shp.hidden), dtype=torch.bfloat16, device="cuda:0")
    past_dev = to_dev(past)
    y = torch.empty_like(x_dev)
    ws = torch.empty(layer.workspace_bytes(Bsz, 1, pages_per_seq * PAGE), dtype=torch.uint8,
                     device="cuda:0")
    xs = [rand(r, (Bsz, 1, shp.hidden), 1.0, "bf16") for _ in range(6)]
    x_dev.copy_(to_dev(xs[0]))
    # warm-up on a side stream, then capture (the warm-up step's append is
    # undone by reloading the pools before the first replay)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward_paged(x_dev, cache, past_dev, y=y, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward_paged(x_dev, cache, past_dev, y=y, ws=ws)
    torch.cuda.synchronize()
    gk.copy_(to_dev(W.to_library_key_pages(pk)))
    gv.copy_(to_dev(W.to_library_value_pages(pv)))
    F = {p: (f64(a), f64(b)) for p, (a, b) in facs.items()}
    ref_k, ref_v = f64(pk), f64(pv)
    cur = past.copy()
    for step in range(6):
        # a sequence whose new position starts a page gets a free pool page
        for b in range(Bsz):
            if live[b, cur[b] // PAGE] < 0:
                live[b, cur[b] // PAGE] = free.pop()
        gt.copy_(to_dev(live))
        past_dev.copy_(to_dev(cur))
        x_dev.copy_(to_dev(xs[step]))
        print(f"paged graph replay {step}: past={cur.tolist()}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        want = ref.decomposed_layer_paged(F, f64(xs[step]), ref_k, ref_v, live, cur, shp.n_q,
                                          shp.n_kv, shp.head_dim, shp.rope_theta, shp.rms_eps)
        assert relerr(to_host(y), want["y"]) <= TOL["bf16"], step
        ref_k, ref_v = want["pool_k"], want["pool_v"]
        # the device pool follows the GPU's own appended rows; the oracle
        # chain continues from its own, so compare the appended rows here
        gkh = f64(W.from_library_key_pages(_bits(gk)))
        for b in range(Bsz):
            pg, row = live[b, cur[b] // PAGE], cur[b] % PAGE
            assert relerr(gkh[pg, row], ref_k[pg, row]) <= TOL["bf16"], (step, b)
        cur = cur + 1
