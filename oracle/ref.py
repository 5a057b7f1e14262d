"""Plain fp64 CPU oracle of one SVD-decomposed transformer layer.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module; the library's HIP path never
imports, links or calls anything here, and this module imports nothing from
the library.

It is written from "DeInfer: Efficient Parallel Inferencing for Decomposed
Large Language Models" (Huang, Huang, Liao, Wen; DAC '26):
  * section 2.1, Eq. (1): W ~ A B, A = U_k sqrt(S_k) (m x k),
    B = sqrt(S_k) V_k^T (k x n); a projection y = x W becomes y = (x A) B.
  * section 2.1: the low-rank intermediates of the K and V pairs are the
    KV cache.
  * section 4.1 / Fig. 3: down factors of q, k, v (and gate, up) read the
    same normalised activations; the k and v latents are stored as cache.
  * section 4.2 / Fig. 4(b): attention rebuilds K and V by multiplying the
    cached latents with the up factors, applies rotary position embedding to
    the rebuilt keys, then attends.
  * Table 2: MHA, MQA and GQA attention, GLU-based and non-GLU MLPs,
    rotary embedding; Fig. 3(b) shows SiLU as the MLP activation; section
    5.1 names OPT-30B as the non-GLU model.

Readings where the paper is silent (each also listed in the design notes):
  * row-vector convention, head-major projection outputs (head j occupies
    columns [j*d, (j+1)*d)); GQA maps query head h to kv head
    h // (n_q / n_kv);
  * LLaMA pre-norm block: RMSNorm -> attention -> residual -> RMSNorm ->
    SwiGLU MLP (silu(x A_g B_g) * (x A_u B_u)) -> residual;
  * the non-GLU MLP is OPT's fc1 -> ReLU -> fc2, i.e. relu(x A_u B_u)
    A_d B_d with the up and down pairs (same block around it: OPT's
    LayerNorm, biases and learned positions are outside this reading);
  * RoPE pairs (i, i + d/2) rotated by pos * theta^(-2i/d), applied to the
    query and to the rebuilt keys, never to the cached latents; theta == 0
    disables it;
  * softmax scale 1/sqrt(d) unless given; causal: a query at position p sees
    keys 0..p.

Every function upcasts its inputs to float64 and never rounds internally.
The paged forms gather each sequence's rows through its block table and
reuse the contiguous functions unchanged.
Parity of every function is pinned by tests/test_oracle_pins.py.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

F64 = np.float64


def _f(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


# ----------------------------------------------------------------------------
# Factor pairs (section 2.1, Eq. (1))
# ----------------------------------------------------------------------------
def svd_factors(W, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Truncated-SVD factor pair of W (m x n): A = U_k sqrt(S_k),
    B = sqrt(S_k) V_k^T, so that A @ B is the best rank-k approximation."""
    U, s, Vt = np.linalg.svd(_f(W), full_matrices=False)
    root = np.sqrt(s[:k])
    return U[:, :k] * root[None, :], root[:, None] * Vt[:k, :]


def lowrank_linear(x, A, B) -> np.ndarray:
    """y = (x A) B for row vectors x [..., m], A [m, k], B [k, n]."""
    return (_f(x) @ _f(A)) @ _f(B)


# ----------------------------------------------------------------------------
# Low-rank KV cache (section 2.1; section 4.1)
# ----------------------------------------------------------------------------
def kv_append(x, A_k, A_v, ck, cv, past_lens) -> Tuple[np.ndarray, np.ndarray]:
    """Store the k/v latents of T new tokens per sequence.

    x [Bsz, T, m]; ck [Bsz, L_max, r_k]; cv [Bsz, L_max, r_v];
    past_lens [Bsz]. Row past_lens[b] + t of ck[b] becomes x[b, t] A_k and the
    same row of cv[b] becomes x[b, t] A_v. Returns updated float64 copies;
    every other row is copied unchanged."""
    x = _f(x)
    ck2, cv2 = _f(ck).copy(), _f(cv).copy()
    Ak, Av = _f(A_k), _f(A_v)
    Bsz, T, _ = x.shape
    for b in range(Bsz):
        p = int(past_lens[b])
        for t in range(T):
            ck2[b, p + t] = x[b, t] @ Ak
            cv2[b, p + t] = x[b, t] @ Av
    return ck2, cv2


# ----------------------------------------------------------------------------
# Rotary position embedding (Table 2; section 4.2 applies it to rebuilt keys)
# ----------------------------------------------------------------------------
def rope_frequencies(d: int, theta: float) -> np.ndarray:
    i = np.arange(d // 2, dtype=F64)
    return float(theta) ** (-2.0 * i / d)


def rope(v, pos, theta: float) -> np.ndarray:
    """Rotate pairs (v_i, v_{i+d/2}) of the last axis by angle pos * w_i,
    w_i = theta^(-2i/d). pos broadcasts against v.shape[:-1]. theta == 0
    returns v unchanged."""
    v = _f(v)
    if theta == 0:
        return v.copy()
    d = v.shape[-1]
    half = d // 2
    ang = np.asarray(pos, dtype=F64)[..., None] * rope_frequencies(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = v[..., :half], v[..., half:]
    return np.concatenate([lo * c - hi * s, lo * s + hi * c], axis=-1)


# ----------------------------------------------------------------------------
# Attention over rebuilt K/V (section 4.2)
# ----------------------------------------------------------------------------
def reconstruct_kv(ck_b, cv_b, B_k, B_v, n_kv: int, d: int,
                   theta: float) -> Tuple[np.ndarray, np.ndarray]:
    """K = RoPE(C_k B_k) with row index as position, V = C_v B_v, both
    reshaped to [L, n_kv, d]."""
    ck_b, cv_b = _f(ck_b), _f(cv_b)
    L = ck_b.shape[0]
    K = (ck_b @ _f(B_k)).reshape(L, n_kv, d)
    K = rope(K, np.arange(L, dtype=F64)[:, None], theta)
    V = (cv_b @ _f(B_v)).reshape(L, n_kv, d)
    return K, V


def softmax_attend(q_rot, q_pos, K, V, sm_scale: float) -> np.ndarray:
    """q_rot [T, n_q, d] (already rotated), q_pos [T]; K, V [L, n_kv, d].
    Query t attends keys 0..q_pos[t] with a max-subtracted softmax."""
    T, n_q, d = q_rot.shape
    n_kv = K.shape[1]
    group = n_q // n_kv
    Kh = np.ascontiguousarray(np.transpose(K, (1, 0, 2)))   # [n_kv, L, d]
    Vh = np.ascontiguousarray(np.transpose(V, (1, 0, 2)))
    out = np.zeros((T, n_q, d), dtype=F64)
    for t in range(T):
        p = int(q_pos[t])
        for g in range(n_kv):
            heads = slice(g * group, (g + 1) * group)        # query heads reading kv head g
            s = (Kh[g, :p + 1] @ q_rot[t, heads].T) * sm_scale   # [p+1, group]
            s = s - s.max(axis=0, keepdims=True)
            w = np.exp(s)
            w = w / w.sum(axis=0, keepdims=True)
            out[t, heads] = w.T @ Vh[g, :p + 1]
    return out


def _scale(d: int, sm_scale: Optional[float]) -> float:
    return 1.0 / np.sqrt(d) if sm_scale is None else float(sm_scale)


def attn_prefill(q, ck, cv, B_k, B_v, past_lens, n_kv: int, theta: float,
                 sm_scale: Optional[float] = None) -> np.ndarray:
    """q [Bsz, T, n_q, d] un-rotated. Query t of sequence b sits at position
    past_lens[b] + t and sees cache rows 0..past_lens[b] + t (those rows must
    already hold the latents). Returns [Bsz, T, n_q, d]."""
    q = _f(q)
    Bsz, T, n_q, d = q.shape
    out = np.zeros_like(q)
    for b in range(Bsz):
        L = int(past_lens[b]) + T
        K, V = reconstruct_kv(_f(ck[b])[:L], _f(cv[b])[:L], B_k, B_v, n_kv, d, theta)
        pos = int(past_lens[b]) + np.arange(T)
        q_rot = rope(q[b], pos[:, None], theta)
        out[b] = softmax_attend(q_rot, pos, K, V, _scale(d, sm_scale))
    return out


def attn_decode(q, ck, cv, B_k, B_v, ctx_lens, n_kv: int, theta: float,
                sm_scale: Optional[float] = None) -> np.ndarray:
    """q [Bsz, n_q, d] un-rotated; sequence b has ctx_lens[b] cached rows and
    its query sits at position ctx_lens[b] - 1. Returns [Bsz, n_q, d]."""
    q = _f(q)
    past = np.asarray(ctx_lens, dtype=np.int64) - 1
    return attn_prefill(q[:, None], ck, cv, B_k, B_v, past, n_kv, theta,
                        sm_scale)[:, 0]


# ----------------------------------------------------------------------------
# The layer
# ----------------------------------------------------------------------------
def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    x = _f(x)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x / r
    return y if gamma is None else y * _f(gamma)


def silu(z) -> np.ndarray:
    z = _f(z)
    return z / (1.0 + np.exp(-z))


def relu(z) -> np.ndarray:
    return np.maximum(_f(z), 0.0)


def decomposed_layer(factors: Dict[str, Tuple[np.ndarray, np.ndarray]], x, ck, cv,
                     past_lens, n_q: int, n_kv: int, head_dim: int,
                     rope_theta: float, rms_eps: float, attn_norm=None,
                     mlp_norm=None, mlp: str = "glu") -> Dict[str, np.ndarray]:
    """Forward pass of one decomposed pre-norm layer for T new tokens per
    sequence. x [Bsz, T, h]; the T new latents are stored at rows
    past_lens[b] .. past_lens[b] + T - 1 before attention reads them.
    mlp: "glu" (silu(gate) * up, then down) or "relu" (the non-GLU form:
    relu(up), then down; the gate pair is not used).

    Returns y (layer output), x2 (residual stream after attention), attn
    (attention output before the o pair) and the updated caches."""
    x = _f(x)
    Bsz, T, h = x.shape
    F = {p: (_f(A), _f(B)) for p, (A, B) in factors.items()}
    a = rmsnorm(x, attn_norm, rms_eps)
    ck2, cv2 = kv_append(a, F["k"][0], F["v"][0], ck, cv, past_lens)
    q = lowrank_linear(a, *F["q"]).reshape(Bsz, T, n_q, head_dim)
    att = attn_prefill(q, ck2, cv2, F["k"][1], F["v"][1], past_lens, n_kv,
                       rope_theta)
    att = att.reshape(Bsz, T, n_q * head_dim)
    x2 = x + lowrank_linear(att, *F["o"])
    b2 = rmsnorm(x2, mlp_norm, rms_eps)
    if mlp == "glu":
        hidden = silu(lowrank_linear(b2, *F["gate"])) * lowrank_linear(b2, *F["up"])
    elif mlp == "relu":
        hidden = relu(lowrank_linear(b2, *F["up"]))
    else:
        raise ValueError(f"unknown MLP kind {mlp!r}")
    y = x2 + lowrank_linear(hidden, *F["down"])
    return {"y": y, "x2": x2, "attn": att, "ck": ck2, "cv": cv2}


# ----------------------------------------------------------------------------
# Paged cache (section 4.2, Fig. 4(a)/(b): the cache lives in fixed-size
# blocks of a pool and a block table lists each sequence's blocks in order)
# ----------------------------------------------------------------------------
def paged_gather(pool, table_row, L: int) -> np.ndarray:
    """Positions 0..L-1 of one sequence from a pool of pages
    [num_pages, page, r], reading its pages in block-table order: position p
    is row p % page of pool page table_row[p // page]."""
    pool = _f(pool)
    page = pool.shape[1]
    out = np.zeros((L, pool.shape[2]), dtype=F64)
    for p in range(L):
        out[p] = pool[int(table_row[p // page]), p % page]
    return out


def decomposed_layer_paged(factors, x, pool_k, pool_v, table, past_lens, n_q: int,
                           n_kv: int, head_dim: int, rope_theta: float, rms_eps: float,
                           attn_norm=None, mlp_norm=None, mlp: str = "glu") -> Dict[str, np.ndarray]:
    """decomposed_layer over a paged cache, one sequence at a time: its
    past_lens[b] + T rows are gathered through its block-table row (the
    last T are overwritten by the append), the layer runs on that contiguous
    cache, and the T appended rows are written back to the pages the table
    names. Returns y, x2, attn and the updated pools (float64 copies); every
    other pool row is unchanged."""
    x = _f(x)
    Bsz, T, _ = x.shape
    pk, pv = _f(pool_k).copy(), _f(pool_v).copy()
    page = pk.shape[1]
    ys, x2s, atts = [], [], []
    for b in range(Bsz):
        past = int(past_lens[b])
        ck = paged_gather(pk, table[b], past + T)[None]
        cv = paged_gather(pv, table[b], past + T)[None]
        out = decomposed_layer(factors, x[b:b + 1], ck, cv, [past], n_q, n_kv, head_dim,
                               rope_theta, rms_eps, attn_norm=attn_norm, mlp_norm=mlp_norm,
                               mlp=mlp)
        for t in range(T):
            p = past + t
            pk[int(table[b][p // page]), p % page] = out["ck"][0, p]
            pv[int(table[b][p // page]), p % page] = out["cv"][0, p]
        ys.append(out["y"][0])
        x2s.append(out["x2"][0])
        atts.append(out["attn"][0])
    return {"y": np.stack(ys), "x2": np.stack(x2s), "attn": np.stack(atts), "pool_k": pk,
            "pool_v": pv}


def attn_decode_paged(q, pool_k, pool_v, table, B_k, B_v, ctx_lens, n_kv: int, theta: float,
                      sm_scale: Optional[float] = None) -> np.ndarray:
    """attn_decode with each sequence's ctx_lens[b] cached rows gathered
    through its block-table row."""
    q = _f(q)
    out = np.zeros_like(q)
    for b in range(q.shape[0]):
        L = int(ctx_lens[b])
        ck = paged_gather(pool_k, table[b], L)[None]
        cv = paged_gather(pool_v, table[b], L)[None]
        out[b] = attn_decode(q[b:b + 1], ck, cv, B_k, B_v, [L], n_kv, theta, sm_scale)[0]
    return out
