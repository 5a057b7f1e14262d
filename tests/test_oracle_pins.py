"""Pins of the fp64 oracle against facts fixed by the DeInfer paper and by
mathematics, independent of the oracle's own formulas:

- Eq. (1) factor pairs: exact reconstruction at full rank, Eckart-Young
  error at truncated rank, balanced square-root split;
- full-rank decomposed layer == an independently written dense layer
  (prefill, decode, chunked prefill);
- attention == brute force with an explicit masked score matrix;
- prefill of S+1 tokens == prefill of S then one decode step;
- RoPE closed forms and invariants; attention special cases (L = 1, q = 0,
  MHA/MQA/GQA equivalences); cache-append row invariants.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import ref
from tests.dense_layer import dense_layer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------
# Eq. (1): W ~ A B
# --------------------------------------------------------------------------
@pytest.mark.parametrize("m,n", [(12, 20), (33, 7), (16, 16)])
def test_svd_factors_full_rank_exact(m, n):
    W = rng(1).standard_normal((m, n))
    A, B = ref.svd_factors(W, min(m, n))
    assert A.shape == (m, min(m, n)) and B.shape == (min(m, n), n)
    assert np.max(np.abs(A @ B - W)) < 1e-12 * max(1.0, np.max(np.abs(W)))


@pytest.mark.parametrize("k", [1, 3, 6])
def test_svd_factors_eckart_young(k):
    W = rng(2).standard_normal((14, 9))
    s = np.linalg.svd(W, compute_uv=False)
    A, B = ref.svd_factors(W, k)
    E = W - A @ B
    assert abs(np.linalg.norm(E, 2) - s[k]) < 1e-10
    assert abs(np.linalg.norm(E, "fro") ** 2 - np.sum(s[k:] ** 2)) < 1e-9
    # balanced split sqrt(S) on both sides: A^T A = B B^T = diag(s_1..s_k)
    assert np.allclose(A.T @ A, np.diag(s[:k]), atol=1e-10)
    assert np.allclose(B @ B.T, np.diag(s[:k]), atol=1e-10)


def test_lowrank_linear_associativity_and_full_rank():
    r = rng(3)
    W = r.standard_normal((24, 10))
    x = r.standard_normal((5, 24))
    A, B = ref.svd_factors(W, 10)
    y = ref.lowrank_linear(x, A, B)
    assert np.allclose(y, x @ W, atol=1e-11)
    A2, B2 = r.standard_normal((24, 4)), r.standard_normal((4, 10))
    assert np.allclose(ref.lowrank_linear(x, A2, B2), x @ (A2 @ B2), atol=1e-11)
    # a transposed or swapped operand order must not pass
    assert not np.allclose(ref.lowrank_linear(x, A2, B2), (x @ A2) @ B2[:, ::-1])


# --------------------------------------------------------------------------
# Full-rank decomposed layer == dense layer
# --------------------------------------------------------------------------
def _dense_and_factors(seed, h, n_q, n_kv, d, f):
    r = rng(seed)
    shapes = {"q": (h, n_q * d), "k": (h, n_kv * d), "v": (h, n_kv * d),
              "o": (n_q * d, h), "gate": (h, f), "up": (h, f), "down": (f, h)}
    W = {p: r.standard_normal(s) * 0.3 for p, s in shapes.items()}
    F = {p: ref.svd_factors(Wp, min(Wp.shape)) for p, Wp in W.items()}
    return r, W, F


@pytest.mark.parametrize("P,T,n_q,n_kv,theta", [
    (0, 5, 4, 2, 10000.0),     # prefill, GQA
    (6, 1, 4, 2, 10000.0),     # decode, GQA
    (3, 4, 4, 4, 50.0),        # chunked prefill, MHA, fast rotation
    (4, 2, 4, 1, 0.0),         # MQA without RoPE
])
def test_layer_matches_dense_at_full_rank(P, T, n_q, n_kv, theta):
    h, d, f, Bsz, eps = 16, 8, 24, 2, 1e-5
    r, W, F = _dense_and_factors(10 + P + T, h, n_q, n_kv, d, f)
    x = r.standard_normal((Bsz, T, h))
    past_norm = r.standard_normal((Bsz, P, h)) if P else None
    L_max = P + T + 2
    ck = np.zeros((Bsz, L_max, F["k"][0].shape[1]))
    cv = np.zeros((Bsz, L_max, F["v"][0].shape[1]))
    if P:
        ck[:, :P] = past_norm @ F["k"][0]
        cv[:, :P] = past_norm @ F["v"][0]
    out = ref.decomposed_layer(F, x, ck, cv, np.full(Bsz, P), n_q, n_kv, d, theta, eps)
    y_d, x2_d = dense_layer(W, x, past_norm, n_q, n_kv, d, theta, eps)
    assert np.max(np.abs(out["x2"] - x2_d)) < 1e-9
    assert np.max(np.abs(out["y"] - y_d)) < 1e-9


@pytest.mark.parametrize("P,T,theta", [(0, 5, 0.0), (4, 1, 0.0), (3, 2, 10000.0)])
def test_relu_mlp_layer_matches_dense_at_full_rank(P, T, theta):
    """The non-GLU MLP (OPT's fc1 -> ReLU -> fc2; Table 2 and section 5.1 of
    the pages) at full rank equals the dense layer with a ReLU MLP; the GLU
    form on the same factors must not."""
    h, n_q, n_kv, d, f, Bsz, eps = 16, 4, 4, 8, 24, 2, 1e-5
    r, W, F = _dense_and_factors(60 + P + T, h, n_q, n_kv, d, f)
    x = r.standard_normal((Bsz, T, h))
    past_norm = r.standard_normal((Bsz, P, h)) if P else None
    L_max = P + T + 1
    ck = np.zeros((Bsz, L_max, F["k"][0].shape[1]))
    cv = np.zeros((Bsz, L_max, F["v"][0].shape[1]))
    if P:
        ck[:, :P] = past_norm @ F["k"][0]
        cv[:, :P] = past_norm @ F["v"][0]
    past = np.full(Bsz, P)
    out = ref.decomposed_layer(F, x, ck, cv, past, n_q, n_kv, d, theta, eps, mlp="relu")
    y_d, x2_d = dense_layer(W, x, past_norm, n_q, n_kv, d, theta, eps, relu_mlp=True)
    assert np.max(np.abs(out["x2"] - x2_d)) < 1e-9
    assert np.max(np.abs(out["y"] - y_d)) < 1e-9
    glu = ref.decomposed_layer(F, x, ck, cv, past, n_q, n_kv, d, theta, eps)
    assert np.max(np.abs(glu["y"] - y_d)) > 1e-3
    # about half the hidden units are clipped, so the activation matters
    b2 = ref.rmsnorm(out["x2"], None, eps)
    u = ref.lowrank_linear(b2, *F["up"])
    assert 0.2 < float(np.mean(u < 0)) < 0.8


@pytest.mark.parametrize("P,T", [(0, 4), (5, 1)])
def test_layer_gains_match_dense_at_full_rank(P, T):
    """Norm gains: attn_norm scales the attention input and mlp_norm the MLP
    input. Distinct random gains; the swapped wiring must not match."""
    h, n_q, n_kv, d, f, Bsz, eps, theta = 16, 4, 2, 8, 24, 2, 1e-5, 10000.0
    r, W, F = _dense_and_factors(40 + P, h, n_q, n_kv, d, f)
    g_attn = 0.5 + r.random(h)
    g_mlp = 0.5 + r.random(h)
    x = r.standard_normal((Bsz, T, h))
    past_norm = r.standard_normal((Bsz, P, h)) if P else None
    L_max = P + T + 1
    ck = np.zeros((Bsz, L_max, F["k"][0].shape[1]))
    cv = np.zeros((Bsz, L_max, F["v"][0].shape[1]))
    if P:
        ck[:, :P] = past_norm @ F["k"][0]
        cv[:, :P] = past_norm @ F["v"][0]
    past = np.full(Bsz, P)
    out = ref.decomposed_layer(F, x, ck, cv, past, n_q, n_kv, d, theta, eps,
                               attn_norm=g_attn, mlp_norm=g_mlp)
    y_d, x2_d = dense_layer(W, x, past_norm, n_q, n_kv, d, theta, eps, attn_gain=g_attn,
                            mlp_gain=g_mlp)
    assert np.max(np.abs(out["x2"] - x2_d)) < 1e-9
    assert np.max(np.abs(out["y"] - y_d)) < 1e-9
    swapped = ref.decomposed_layer(F, x, ck, cv, past, n_q, n_kv, d, theta, eps,
                                   attn_norm=g_mlp, mlp_norm=g_attn)
    assert np.max(np.abs(swapped["y"] - y_d)) > 1e-3


# --------------------------------------------------------------------------
# Attention vs brute force
# --------------------------------------------------------------------------
def _brute_attention(q, ck, cv, B_k, B_v, past_lens, n_kv, theta, scale=None):
    """Per query: explicit score row over ALL cache rows with -inf beyond the
    causal limit, math.exp normalisation, explicit rotation by angle."""
    Bsz, T, n_q, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    half = d // 2
    G = n_q // n_kv
    L_max = ck.shape[1]
    out = np.zeros(q.shape)

    def rot(vec, pos):
        o = np.array(vec, dtype=float)
        if theta == 0:
            return o
        for i in range(half):
            a = pos * theta ** (-2.0 * i / d)
            o[i] = vec[i] * math.cos(a) - vec[i + half] * math.sin(a)
            o[i + half] = vec[i] * math.sin(a) + vec[i + half] * math.cos(a)
        return o

    for b in range(Bsz):
        for t in range(T):
            p = past_lens[b] + t
            for hh in range(n_q):
                g = hh // G
                qv = rot(q[b, t, hh], p)
                row = []
                for j in range(L_max):
                    if j > p:
                        row.append(-math.inf)
                        continue
                    kv = rot((ck[b, j] @ B_k)[g * d:(g + 1) * d], j)
                    row.append(sum(qv[i] * kv[i] for i in range(d)) * scale)
                mx = max(row)
                e = [0.0 if s == -math.inf else math.exp(s - mx) for s in row]
                z = sum(e)
                acc = np.zeros(d)
                for j in range(L_max):
                    if e[j]:
                        acc += (e[j] / z) * (cv[b, j] @ B_v)[g * d:(g + 1) * d]
                out[b, t, hh] = acc
    return out


@pytest.mark.parametrize("n_q,n_kv,theta", [(4, 2, 10000.0), (2, 2, 30.0), (4, 1, 0.0)])
def test_attention_matches_brute_force_ragged(n_q, n_kv, theta):
    r = rng(5)
    Bsz, T, d, rk, rv, L_max = 3, 3, 8, 5, 6, 11
    past = np.array([0, 4, 8])
    q = r.standard_normal((Bsz, T, n_q, d))
    ck = r.standard_normal((Bsz, L_max, rk))
    cv = r.standard_normal((Bsz, L_max, rv))
    B_k = r.standard_normal((rk, n_kv * d)) * 0.5
    B_v = r.standard_normal((rv, n_kv * d))
    got = ref.attn_prefill(q, ck, cv, B_k, B_v, past, n_kv, theta)
    want = _brute_attention(q, ck, cv, B_k, B_v, past, n_kv, theta)
    assert np.max(np.abs(got - want)) < 1e-12
    # decode form: the last query of each sequence
    got_dec = ref.attn_decode(q[:, -1], ck, cv, B_k, B_v, past + T, n_kv, theta)
    assert np.max(np.abs(got_dec - want[:, -1])) < 1e-12


@pytest.mark.parametrize("scale", [0.05, 1.7])
def test_attention_explicit_scale_matches_brute_force(scale):
    """The explicit softmax-scale branch: a scale other than 1/sqrt(d) must
    reach the scores unchanged (a sharper and a flatter softmax)."""
    r = rng(6)
    Bsz, T, n_q, n_kv, d, rk, rv, L_max = 2, 2, 4, 2, 8, 5, 6, 9
    past = np.array([1, 6])
    q = r.standard_normal((Bsz, T, n_q, d))
    ck = r.standard_normal((Bsz, L_max, rk))
    cv = r.standard_normal((Bsz, L_max, rv))
    B_k = r.standard_normal((rk, n_kv * d)) * 0.5
    B_v = r.standard_normal((rv, n_kv * d))
    got = ref.attn_prefill(q, ck, cv, B_k, B_v, past, n_kv, 1000.0, sm_scale=scale)
    want = _brute_attention(q, ck, cv, B_k, B_v, past, n_kv, 1000.0, scale=scale)
    assert np.max(np.abs(got - want)) < 1e-12
    got_dec = ref.attn_decode(q[:, -1], ck, cv, B_k, B_v, past + T, n_kv, 1000.0, sm_scale=scale)
    assert np.max(np.abs(got_dec - want[:, -1])) < 1e-12
    # the default scale gives a different result: the branch is not a no-op
    assert np.max(np.abs(ref.attn_prefill(q, ck, cv, B_k, B_v, past, n_kv, 1000.0) - want)) > 1e-3


def test_prefill_then_decode_equals_longer_prefill():
    h, n_q, n_kv, d, f, Bsz, S = 16, 4, 2, 8, 24, 2, 6
    r = rng(7)
    F = {}
    for p, (m, n) in {"q": (h, n_q * d), "k": (h, n_kv * d), "v": (h, n_kv * d),
                      "o": (n_q * d, h), "gate": (h, f), "up": (h, f), "down": (f, h)}.items():
        k = 5 if p in ("k", "v") else 7
        F[p] = (r.standard_normal((m, k)) * 0.4, r.standard_normal((k, n)) * 0.4)
    x = r.standard_normal((Bsz, S + 1, h))
    L_max = S + 3
    z = lambda: np.zeros((Bsz, L_max, 5))
    full = ref.decomposed_layer(F, x, z(), z(), np.zeros(Bsz, int), n_q, n_kv, d, 1000.0, 1e-5)
    pre = ref.decomposed_layer(F, x[:, :S], z(), z(), np.zeros(Bsz, int), n_q, n_kv, d, 1000.0, 1e-5)
    dec = ref.decomposed_layer(F, x[:, S:], pre["ck"], pre["cv"], np.full(Bsz, S), n_q, n_kv, d,
                               1000.0, 1e-5)
    assert np.max(np.abs(full["y"][:, S] - dec["y"][:, 0])) < 1e-12
    assert np.max(np.abs(full["y"][:, :S] - pre["y"])) < 1e-12
    assert np.array_equal(full["ck"], dec["ck"])


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------
def test_rope_closed_forms():
    g = json.load(open(os.path.join(GOLDEN, "rope_closed_form.json")))
    env = {"cos": math.cos, "sin": math.sin}
    for c in g["cases"]:
        want = [eval(e, {"__builtins__": {}}, env) for e in c["expect"]]
        got = ref.rope(np.array(c["v"], float), c["pos"], g["theta"])
        assert np.allclose(got, want, atol=1e-15), c


def test_rope_invariants():
    r = rng(8)
    d, theta = 16, 10000.0
    v = r.standard_normal((5, d))
    assert np.array_equal(ref.rope(v, 0, theta), v)
    pos = np.arange(5) * 37
    assert np.allclose(np.linalg.norm(ref.rope(v, pos, theta), axis=-1), np.linalg.norm(v, axis=-1))
    q, k = r.standard_normal(d), r.standard_normal(d)
    a = ref.rope(q, 11, theta) @ ref.rope(k, 4, theta)
    b = ref.rope(q, 11 + 100, theta) @ ref.rope(k, 4 + 100, theta)
    assert abs(a - b) < 1e-10
    assert np.array_equal(ref.rope(v, 5, 0.0), v)


# --------------------------------------------------------------------------
# Attention special cases
# --------------------------------------------------------------------------
def _attn_case(seed, n_q, n_kv, d=8, rk=6, rv=5, L_max=9, Bsz=2):
    r = rng(seed)
    return (r.standard_normal((Bsz, n_q, d)), r.standard_normal((Bsz, L_max, rk)),
            r.standard_normal((Bsz, L_max, rv)), r.standard_normal((rk, n_kv * d)),
            r.standard_normal((rv, n_kv * d)))


def test_single_row_returns_that_value_row():
    q, ck, cv, Bk, Bv = _attn_case(9, 4, 2)
    out = ref.attn_decode(q, ck, cv, Bk, Bv, np.array([1, 1]), 2, 10000.0)
    for b in range(2):
        for hh in range(4):
            g = hh // 2
            assert np.allclose(out[b, hh], (cv[b, 0] @ Bv)[g * 8:(g + 1) * 8], atol=1e-13)


def test_zero_query_averages_values():
    q, ck, cv, Bk, Bv = _attn_case(10, 4, 2)
    out = ref.attn_decode(np.zeros_like(q), ck, cv, Bk, Bv, np.array([7, 3]), 2, 10000.0)
    for b, L in enumerate([7, 3]):
        V = (cv[b, :L] @ Bv).reshape(L, 2, 8)
        for hh in range(4):
            assert np.allclose(out[b, hh], V[:, hh // 2].mean(axis=0), atol=1e-13)


@pytest.mark.parametrize("n_kv", [1, 2])
def test_gqa_equals_mha_with_repeated_kv_heads(n_kv):
    n_q, d = 4, 8
    G = n_q // n_kv
    q, ck, cv, Bk, Bv = _attn_case(11, n_q, n_kv)
    rep = lambda M: np.concatenate([M[:, (h // G) * d:(h // G + 1) * d] for h in range(n_q)], axis=1)
    lens = np.array([9, 5])
    a = ref.attn_decode(q, ck, cv, Bk, Bv, lens, n_kv, 500.0)
    b = ref.attn_decode(q, ck, cv, rep(Bk), rep(Bv), lens, n_q, 500.0)
    assert np.allclose(a, b, atol=1e-13)


# --------------------------------------------------------------------------
# Cache append
# --------------------------------------------------------------------------
def test_kv_append_touches_only_new_rows():
    r = rng(12)
    Bsz, T, m, rk, rv, L_max = 3, 2, 10, 4, 6, 9
    x = r.standard_normal((Bsz, T, m))
    Ak, Av = r.standard_normal((m, rk)), r.standard_normal((m, rv))
    ck, cv = r.standard_normal((Bsz, L_max, rk)), r.standard_normal((Bsz, L_max, rv))
    past = np.array([0, 3, 7])
    ck2, cv2 = ref.kv_append(x, Ak, Av, ck, cv, past)
    for b in range(Bsz):
        for row in range(L_max):
            t = row - past[b]
            if 0 <= t < T:
                assert np.allclose(ck2[b, row], sum(x[b, t, i] * Ak[i] for i in range(m)), atol=1e-12)
                assert np.allclose(cv2[b, row], sum(x[b, t, i] * Av[i] for i in range(m)), atol=1e-12)
            else:
                assert np.array_equal(ck2[b, row], ck[b, row])
                assert np.array_equal(cv2[b, row], cv[b, row])


def test_rmsnorm_and_silu_special_values():
    x = np.full((1, 6), -3.0)
    assert np.allclose(ref.rmsnorm(x, None, 0.0), -1.0)
    assert np.allclose(ref.rmsnorm(x, np.arange(6.0), 0.0), -np.arange(6.0))
    assert ref.silu(0.0) == 0.0
    assert abs(ref.silu(40.0) - 40.0) < 1e-12
    assert abs(ref.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


# --------------------------------------------------------------------------
# Paged cache: page placement must not change any result
# --------------------------------------------------------------------------
def _pages_of(cache, table, num_pages, page):
    """Scatter contiguous [Bsz, L, r] rows into pool pages with explicit
    loops (position p -> page table[b, p // page], row p % page)."""
    Bsz, L, r = cache.shape
    pool = np.full((num_pages, page, r), np.nan)
    for b in range(Bsz):
        for p in range(L):
            pool[table[b, p // page], p % page] = cache[b, p]
    return pool


def test_paged_gather_reads_pages_in_table_order():
    r = rng(20)
    Bsz, L, rk, page, num = 2, 12, 3, 4, 9
    ck = r.standard_normal((Bsz, L, rk))
    table = r.permutation(num)[:Bsz * (L // page)].reshape(Bsz, L // page)
    pool = _pages_of(ck, table, num, page)
    for b in range(Bsz):
        for n in (1, 5, L):
            assert np.array_equal(ref.paged_gather(pool, table[b], n), ck[b, :n])
    # the identity table over a reshaped contiguous cache
    ident = np.arange(Bsz * (L // page)).reshape(Bsz, L // page)
    assert np.array_equal(ref.paged_gather(ck.reshape(-1, page, rk), ident[1], L), ck[1])


@pytest.mark.parametrize("T", [1, 3])
def test_paged_layer_equals_contiguous_layer(T):
    """A shuffled block table gives the contiguous result; appended rows land
    on the pages the table names; every other pool row is untouched."""
    h, n_q, n_kv, d, f, Bsz, page = 16, 4, 2, 8, 24, 3, 4
    r = rng(21 + T)
    F = {}
    for p, (m, n) in {"q": (h, n_q * d), "k": (h, n_kv * d), "v": (h, n_kv * d),
                      "o": (n_q * d, h), "gate": (h, f), "up": (h, f), "down": (f, h)}.items():
        k = 5 if p in ("k", "v") else 7
        F[p] = (r.standard_normal((m, k)) * 0.4, r.standard_normal((k, n)) * 0.4)
    past = np.array([0, 5, 9])
    L_max, num = 16, 14
    x = r.standard_normal((Bsz, T, h))
    ck, cv = r.standard_normal((Bsz, L_max, 5)), r.standard_normal((Bsz, L_max, 5))
    table = r.permutation(num)[:Bsz * (L_max // page)].reshape(Bsz, L_max // page)
    pk, pv = _pages_of(ck, table, num, page), _pages_of(cv, table, num, page)
    # pool rows that belong to no sequence hold sentinels
    pk[np.isnan(pk)] = 7.0
    pv[np.isnan(pv)] = -7.0
    want = ref.decomposed_layer(F, x, ck, cv, past, n_q, n_kv, d, 1000.0, 1e-5)
    got = ref.decomposed_layer_paged(F, x, pk, pv, table, past, n_q, n_kv, d, 1000.0, 1e-5)
    assert np.max(np.abs(got["y"] - want["y"])) < 1e-12
    assert np.max(np.abs(got["x2"] - want["x2"])) < 1e-12
    written = np.zeros(pk.shape[:2], bool)
    for b in range(Bsz):
        for t in range(T):
            pos = past[b] + t
            pg, row = table[b, pos // page], pos % page
            written[pg, row] = True
            assert np.allclose(got["pool_k"][pg, row], want["ck"][b, pos], atol=1e-12)
            assert np.allclose(got["pool_v"][pg, row], want["cv"][b, pos], atol=1e-12)
    assert np.array_equal(got["pool_k"][~written], pk[~written])
    assert np.array_equal(got["pool_v"][~written], pv[~written])
    lens = past + T
    att = ref.attn_decode_paged(r.standard_normal((Bsz, n_q, d)), got["pool_k"], got["pool_v"],
                                table, F["k"][1], F["v"][1], lens, n_kv, 1000.0)
    assert att.shape == (Bsz, n_q, d) and np.all(np.isfinite(att))


def test_paged_decode_attention_equals_contiguous():
    r = rng(23)
    Bsz, n_q, n_kv, d, rk, rv, page, L = 2, 4, 2, 8, 6, 5, 4, 12
    q = r.standard_normal((Bsz, n_q, d))
    ck, cv = r.standard_normal((Bsz, L, rk)), r.standard_normal((Bsz, L, rv))
    Bk, Bv = r.standard_normal((rk, n_kv * d)), r.standard_normal((rv, n_kv * d))
    table = r.permutation(7)[:6].reshape(Bsz, 3)
    lens = np.array([12, 7])
    want = ref.attn_decode(q, ck, cv, Bk, Bv, lens, n_kv, 500.0)
    got = ref.attn_decode_paged(q, _pages_of(ck, table, 7, page), _pages_of(cv, table, 7, page),
                                table, Bk, Bv, lens, n_kv, 500.0)
    assert np.max(np.abs(got - want)) < 1e-12
