"""A dense (undecomposed) LLaMA-style layer written independently of the
oracle, used to pin it: at full rank with exact SVD factors the decomposed
layer must reproduce this one (the decomposition W ~ A B of section 2.1,
Eq. (1), of the DeInfer paper is then exact).

Written token by token with the math module and explicit rotation matrices so
that it shares no code path with oracle/ref.py. Tiny shapes only.
"""
import math

import numpy as np


def _rot_matrix(d, pos, theta):
    """d x d matrix applying RoPE at position pos: block rotation of the pair
    (i, i + d/2) by pos * theta^(-2i/d)."""
    R = np.eye(d)
    if theta == 0:
        return R
    half = d // 2
    for i in range(half):
        a = pos * theta ** (-2.0 * i / d)
        c, s = math.cos(a), math.sin(a)
        R[i, i], R[i, i + half] = c, -s
        R[i + half, i], R[i + half, i + half] = s, c
    return R


def _rmsnorm_row(v, eps, gain=None):
    ms = sum(float(t) * float(t) for t in v) / len(v)
    g = [1.0] * len(v) if gain is None else [float(t) for t in gain]
    return np.array([float(t) / math.sqrt(ms + eps) * gi for t, gi in zip(v, g)])


def _silu(z):
    return z / (1.0 + math.exp(-z))


def dense_layer(W, x, cache_in_x, n_q, n_kv, d, theta, eps, attn_gain=None, mlp_gain=None,
                sm_scale=None, relu_mlp=False):
    """W: dict of dense [in, out] matrices q, k, v, o, gate, up, down
    (relu_mlp: the MLP is down(max(up(b), 0)), OPT's fc1 / ReLU / fc2, and
    W["gate"] is not read).
    x: [Bsz, T, h] new tokens; cache_in_x: [Bsz, P, h] normalised
    activations of the P tokens already in the cache (or None), whose keys
    and values are recomputed densely. attn_gain / mlp_gain: per-channel
    gains of the two RMSNorms (None = 1). Returns (y, x2)."""
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    Bsz, T, h = x.shape
    group = n_q // n_kv
    y = np.zeros((Bsz, T, h))
    x2_all = np.zeros((Bsz, T, h))
    for b in range(Bsz):
        past = [] if cache_in_x is None else [cache_in_x[b, j] for j in range(cache_in_x.shape[1])]
        P = len(past)
        normed_new = [_rmsnorm_row(x[b, t], eps, attn_gain) for t in range(T)]
        seq = past + normed_new                     # normalised rows, position = index
        keys = []
        vals = []
        for pos, a in enumerate(seq):
            kf = a @ W["k"]
            vf = a @ W["v"]
            keys.append([_rot_matrix(d, pos, theta) @ kf[g * d:(g + 1) * d] for g in range(n_kv)])
            vals.append([vf[g * d:(g + 1) * d] for g in range(n_kv)])
        for t in range(T):
            pos = P + t
            a = normed_new[t]
            qf = a @ W["q"]
            heads = []
            for hh in range(n_q):
                g = hh // group
                qh = _rot_matrix(d, pos, theta) @ qf[hh * d:(hh + 1) * d]
                scores = [float(qh @ keys[j][g]) * scale for j in range(pos + 1)]
                mx = max(scores)
                ws = [math.exp(s - mx) for s in scores]
                tot = sum(ws)
                o = sum((ws[j] / tot) * vals[j][g] for j in range(pos + 1))
                heads.append(o)
            att = np.concatenate(heads)
            x2 = x[b, t] + att @ W["o"]
            bn = _rmsnorm_row(x2, eps, mlp_gain)
            u_ = bn @ W["up"]
            if relu_mlp:
                hid = np.array([float(uv) if float(uv) > 0.0 else 0.0 for uv in u_])
            else:
                g_ = bn @ W["gate"]
                hid = np.array([_silu(float(gv)) * float(uv) for gv, uv in zip(g_, u_)])
            y[b, t] = x2 + hid @ W["down"]
            x2_all[b, t] = x2
    return y, x2_all
