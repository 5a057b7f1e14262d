"""Seeded synthetic workloads for the decomposed-layer forward pass.

This module is shared by the tests, the benchmark and the smoke check: it
describes the five workload shapes, computes the factor ranks and draws the
seeded inputs. It holds none of the layer's arithmetic (no projection, no
attention, no normalisation); both the HIP path and the CPU oracle receive
the arrays it produces, bit for bit.

Shapes follow "DeInfer: Efficient Parallel Inferencing for Decomposed Large
Language Models" (Huang et al., DAC '26): each projection W (m x n) becomes a
factor pair A (m x k), B (k x n) (section 2.1, Eq. (1)), whose parameter count
is (m + n) * k (section 2.1). The LLaMA-3-70B dimensions h = 8192,
h_kv = 1024, m = 28672 are the ones listed under Table 1.

Rank rule: k = floor64((1 - c) * m * n / (m + n)), where c is the fraction of
the projection's parameters removed, rounded down to a multiple of 64.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

PROJECTIONS = ("q", "k", "v", "o", "gate", "up", "down")


# ----------------------------------------------------------------------------
# bf16 encoding (storage only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Expand bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Rank and shape bookkeeping
# ----------------------------------------------------------------------------
def rank_floor64(m: int, n: int, compression_pct: int) -> int:
    """floor64((1 - c) * m * n / (m + n)) with c = compression_pct / 100,
    evaluated in exact integer arithmetic."""
    if not 0 <= compression_pct < 100:
        raise ValueError("compression_pct must be in [0, 100)")
    k = ((100 - compression_pct) * m * n) // (100 * (m + n))
    return (k // 64) * 64


def projection_shapes(hidden: int, n_q: int, n_kv: int, head_dim: int,
                      ffn: int) -> Dict[str, Tuple[int, int]]:
    """(m, n) of each projection in the row-vector convention y = x W."""
    return {
        "q": (hidden, n_q * head_dim),
        "k": (hidden, n_kv * head_dim),
        "v": (hidden, n_kv * head_dim),
        "o": (n_q * head_dim, hidden),
        "gate": (hidden, ffn),
        "up": (hidden, ffn),
        "down": (ffn, hidden),
    }


def factor_params(m: int, n: int, k: int) -> int:
    """Parameter count of a factor pair: (m + n) * k (section 2.1)."""
    return (m + n) * k


def table1_comm_elements(h: int, h_kv: int, m: int, l_q: int, l_k: int,
                         l_v: int, l_up: int, l_gate: int,
                         l_down: int) -> Dict[str, int]:
    """Per-token, per-block communication volume in elements, as tabulated
    in Table 1 of the DeInfer paper. The unoptimised decomposition reduces
    after every pair: 2(2h + 2h_kv) in attention and 2(2m + h) in the MLP
    (a reduce-sum costs twice an all-gather). DeInfer all-gathers the
    concatenated latents once per sub-layer and keeps one reduce-sum of
    2h; the printed LLaMA-3-70B total counts that 2h term once."""
    unopt_attn = 2 * (2 * h + 2 * h_kv)
    unopt_mlp = 2 * (2 * m + h)
    allgather = l_q + l_k + l_v + l_up + l_gate + l_down
    reduce_sum = 2 * h
    unopt = unopt_attn + unopt_mlp
    deinfer = allgather + reduce_sum
    return {
        "unoptimized_attention": unopt_attn,
        "unoptimized_mlp": unopt_mlp,
        "unoptimized_total": unopt,
        "deinfer_allgather": allgather,
        "deinfer_reduce_sum": reduce_sum,
        "deinfer_total": deinfer,
        "reduction_pct": round(100.0 * (1.0 - deinfer / unopt)),
    }


# ----------------------------------------------------------------------------
# Workload descriptions
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class LayerShape:
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    ffn: int
    ranks: Tuple[Tuple[str, int], ...]   # ordered (projection, k)
    dtype: str                           # "f32" or "bf16"
    rope_theta: float
    rms_eps: float = 1e-5
    mlp: str = "glu"                     # "glu" (SwiGLU) or "relu" (non-GLU, no gate pair)

    def rank(self, name: str) -> int:
        return dict(self.ranks)[name]

    def projections(self) -> Tuple[str, ...]:
        """The factor pairs the layer has (no gate pair in a non-GLU MLP)."""
        return tuple(p for p in PROJECTIONS if not (p == "gate" and self.mlp == "relu"))

    def shapes(self) -> Dict[str, Tuple[int, int]]:
        shp = projection_shapes(self.hidden, self.n_q, self.n_kv, self.head_dim, self.ffn)
        return {p: shp[p] for p in self.projections()}

    def weight_elements(self) -> int:
        return sum(factor_params(m, n, self.rank(p))
                   for p, (m, n) in self.shapes().items())


def make_shape(hidden, n_q, n_kv, head_dim, ffn, dtype, rope_theta,
               compression_pct: Optional[int] = None,
               fixed_rank: Optional[int] = None, mlp: str = "glu") -> LayerShape:
    shp = projection_shapes(hidden, n_q, n_kv, head_dim, ffn)
    ranks = []
    for p in PROJECTIONS:
        if p == "gate" and mlp == "relu":
            continue
        m, n = shp[p]
        k = fixed_rank if fixed_rank is not None else rank_floor64(m, n, compression_pct)
        ranks.append((p, k))
    return LayerShape(hidden, n_q, n_kv, head_dim, ffn, tuple(ranks), dtype,
                      rope_theta, mlp=mlp)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    batch: int
    phase: str                    # "decode" or "prefill" or "chain"
    context: int = 0              # cached rows before the step (decode)
    prefill: int = 0              # tokens per sequence (prefill / chain)
    decode_steps: int = 0         # chain only
    seed: int = 0
    factor_std: float = 0.02
    b_row_decay: bool = False     # scale row i (1-based) of every B by i^-1/2
    compression_pct: Optional[int] = None

    @property
    def l_max(self) -> int:
        """Cache capacity per sequence: the rows the workload fills, rounded
        up to whole 64-row pages."""
        rows = self.context + 1 if self.phase == "decode" else self.prefill + self.decode_steps
        return (rows + 63) // 64 * 64


def _llama3_8b(pct):
    return make_shape(4096, 32, 8, 128, 14336, "bf16", 500000.0, compression_pct=pct)


def _llama3_70b(pct):
    return make_shape(8192, 64, 8, 128, 28672, "bf16", 500000.0, compression_pct=pct)


TINY = Workload("tiny_mha_f32_chain",
                make_shape(256, 4, 4, 64, 688, "f32", 10000.0, fixed_rank=64),
                batch=2, phase="chain", prefill=32, decode_steps=8, seed=0)
LLAMA3_8B_C40_DECODE = Workload("llama3_8b_c40_decode_b16_l1024", _llama3_8b(40),
                                batch=16, phase="decode", context=1024, seed=1,
                                compression_pct=40)
LLAMA3_8B_SWEEP = tuple(
    Workload(f"llama3_8b_c{p}_decode_b64_l4096", _llama3_8b(p), batch=64,
             phase="decode", context=4096, seed=2, b_row_decay=True,
             compression_pct=p)
    for p in (20, 30, 40, 50, 60))
LLAMA3_70B_C50_DECODE = Workload("llama3_70b_c50_decode_b32_l8192", _llama3_70b(50),
                                 batch=32, phase="decode", context=8192, seed=3,
                                 compression_pct=50)
LLAMA3_70B_C50_PREFILL = Workload("llama3_70b_c50_prefill_8x2048", _llama3_70b(50),
                                  batch=8, phase="prefill", prefill=2048, seed=4,
                                  compression_pct=50)

# The other foundation models of section 5.1, at the 40% compression of
# Tables 3 and 4, in the pages' second throughput setting (batch 64 for
# LLaMA-65B and 192 for OPT-30B, 64 prefill tokens, sequences up to 512):
# LLaMA-65B is a 64-head MHA LLaMA block; OPT-30B (56-head MHA) has the
# non-GLU MLP and no rotary embedding (its learned positions are outside the
# block).
def _llama_65b(pct):
    return make_shape(8192, 64, 64, 128, 22016, "bf16", 10000.0, compression_pct=pct)


def _opt_30b(pct):
    return make_shape(7168, 56, 56, 128, 28672, "bf16", 0.0, compression_pct=pct, mlp="relu")


LLAMA65B_C40_DECODE = Workload("llama65b_c40_decode_b64_l512", _llama_65b(40), batch=64,
                               phase="decode", context=511, seed=5, compression_pct=40)
LLAMA65B_C40_PREFILL = Workload("llama65b_c40_prefill_64x64", _llama_65b(40), batch=64,
                                phase="prefill", prefill=64, seed=6, compression_pct=40)
OPT30B_C40_DECODE = Workload("opt30b_c40_decode_b192_l512", _opt_30b(40), batch=192,
                             phase="decode", context=511, seed=7, compression_pct=40)
OPT30B_C40_PREFILL = Workload("opt30b_c40_prefill_192x64", _opt_30b(40), batch=192,
                              phase="prefill", prefill=64, seed=8, compression_pct=40)

ALL_WORKLOADS: List[Workload] = [TINY, LLAMA3_8B_C40_DECODE, *LLAMA3_8B_SWEEP,
                                 LLAMA3_70B_C50_DECODE, LLAMA3_70B_C50_PREFILL,
                                 LLAMA65B_C40_DECODE, LLAMA65B_C40_PREFILL,
                                 OPT30B_C40_DECODE, OPT30B_C40_PREFILL]


def by_name(name: str) -> Workload:
    for w in ALL_WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


# ----------------------------------------------------------------------------
# Seeded draws
# ----------------------------------------------------------------------------
def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _encode(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, np.float32)


def decode_array(a: np.ndarray) -> np.ndarray:
    """Stored array (uint16 bf16 bits or float32) -> float32 values."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


@dataclasses.dataclass
class LayerWeights:
    """Factor pairs of one layer in storage encoding (uint16 bf16 bits or
    float32), row-major: A is [m, k], B is [k, n]. Norm gains are None (= 1)."""
    shape: LayerShape
    factors: Dict[str, Tuple[np.ndarray, np.ndarray]]
    attn_norm: Optional[np.ndarray] = None
    mlp_norm: Optional[np.ndarray] = None


def draw_weights(w: Workload, rng: np.random.Generator) -> LayerWeights:
    """Factors q, k, v, o, gate, up, down (A then B), each entry drawn from
    N(0, std^2). With b_row_decay, row i (1-based) of each B is multiplied
    by i^-1/2 before encoding."""
    shp = w.shape
    out = {}
    for p in shp.projections():
        m, n = shp.shapes()[p]
        k = shp.rank(p)
        A = _normal(rng, (m, k), w.factor_std)
        B = _normal(rng, (k, n), w.factor_std)
        if w.b_row_decay:
            B *= (np.arange(1, k + 1, dtype=np.float64) ** -0.5).astype(np.float32)[:, None]
        out[p] = (_encode(A, shp.dtype), _encode(B, shp.dtype))
    return LayerWeights(shp, out)


@dataclasses.dataclass
class LayerInputs:
    """Everything one forward step reads besides the weights.

    x: [batch, T, hidden] activations; past_lens: [batch] int32 rows already
    cached; ck/cv: [batch, l_max, r_k] / [batch, l_max, r_v] latent caches
    (rows >= past_lens[b] are zero). For the chain workload, decode_x holds
    the per-step decode inputs [steps, batch, 1, hidden]."""
    x: np.ndarray
    past_lens: np.ndarray
    ck: np.ndarray
    cv: np.ndarray
    decode_x: Optional[np.ndarray] = None


def draw_inputs(w: Workload, rng: np.random.Generator) -> LayerInputs:
    """Activations ~ N(0, 1). A pre-filled cache (decode workloads) holds
    latents drawn i.i.d. from N(0, (std * sqrt(hidden))^2): the marginal law
    of x A for x ~ N(0, I) and A with N(0, std^2) entries."""
    shp = w.shape
    B, h = w.batch, shp.hidden
    r_k, r_v = shp.rank("k"), shp.rank("v")
    T = 1 if w.phase == "decode" else w.prefill
    x = _encode(_normal(rng, (B, T, h), 1.0), shp.dtype)
    decode_x = None
    if w.phase == "chain":
        decode_x = _encode(_normal(rng, (w.decode_steps, B, 1, h), 1.0), shp.dtype)
    store = np.uint16 if shp.dtype == "bf16" else np.float32
    ck = np.zeros((B, w.l_max, r_k), dtype=store)
    cv = np.zeros((B, w.l_max, r_v), dtype=store)
    past = np.zeros(B, dtype=np.int32)
    if w.phase == "decode" and w.context > 0:
        std = w.factor_std * float(np.sqrt(h))
        for b in range(B):
            ck[b, :w.context] = _encode(_normal(rng, (w.context, r_k), std), shp.dtype)
        for b in range(B):
            cv[b, :w.context] = _encode(_normal(rng, (w.context, r_v), std), shp.dtype)
        past[:] = w.context
    return LayerInputs(x, past, ck, cv, decode_x)


def draw(w: Workload) -> Tuple[LayerWeights, LayerInputs]:
    """All seeded draws of a workload, in the fixed order: factors, inputs,
    decode inputs, cache."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    weights = draw_weights(w, rng)
    inputs = draw_inputs(w, rng)
    return weights, inputs


def algorithmic_decode_bytes(shape: LayerShape, batch: int, ctx: int) -> Dict[str, int]:
    """Bytes one decode step must move at minimum: every factor once, the
    latent cache rows read by attention (ctx rows per sequence, K and V),
    and the activations in and out."""
    es = 2 if shape.dtype == "bf16" else 4
    w_bytes = shape.weight_elements() * es
    cache = batch * ctx * (shape.rank("k") + shape.rank("v")) * es
    act = 2 * batch * shape.hidden * es
    return {"weights": w_bytes, "cache": cache, "activations": act,
            "total": w_bytes + cache + act}


def factor_pair_flops(shape: LayerShape, tokens: int) -> Dict[str, int]:
    """2*M*(m*k + k*n) per projection pair for M tokens."""
    return {p: 2 * tokens * (m * shape.rank(p) + shape.rank(p) * n)
            for p, (m, n) in shape.shapes().items()}


# ----------------------------------------------------------------------------
# Library storage order (data movement only)
# ----------------------------------------------------------------------------
def tile_operands(a: np.ndarray) -> np.ndarray:
    """Matrix (or stack of matrices) [..., R, C] -> the library's bf16
    operand-tile order: 16 x 32 tiles, row-tile major, each tile in MFMA
    lane order (element (r, c) of a tile at ((c // 8) * 16 + r) * 8 + c % 8).
    Needs R % 16 == 0 and C % 32 == 0."""
    *lead, R, C = a.shape
    if R % 16 or C % 32:
        raise ValueError(f"operand tiles need rows % 16 == 0 and cols % 32 == 0, got {R} x {C}")
    t = a.reshape(*lead, R // 16, 16, C // 32, 4, 8)          # [.., rt, r, ct, g, e]
    t = np.moveaxis(t, -3, -4)                                  # [.., rt, ct, r, g, e]
    t = np.swapaxes(t, -3, -2)                                  # [.., rt, ct, g, r, e]
    return np.ascontiguousarray(t).reshape(*lead, R, C)


def untile_operands(t: np.ndarray) -> np.ndarray:
    """Inverse of tile_operands."""
    *lead, R, C = t.shape
    a = t.reshape(*lead, R // 16, C // 32, 4, 16, 8)            # [.., rt, ct, g, r, e]
    a = np.swapaxes(a, -3, -2)                                  # [.., rt, ct, r, g, e]
    a = np.moveaxis(a, -4, -3)                                  # [.., rt, r, ct, g, e]
    return np.ascontiguousarray(a).reshape(*lead, R, C)


def to_library_factor(a: np.ndarray) -> np.ndarray:
    """A factor in the row-vector convention (A [m, k] or B [k, n]) -> the
    library's storage: its transpose, whose rows run along the reduction
    index; bf16 factors (uint16 arrays) in operand-tile order."""
    t = np.ascontiguousarray(np.swapaxes(a, -1, -2))
    return tile_operands(t) if a.dtype == np.uint16 else t


def to_library_key_cache(ck: np.ndarray) -> np.ndarray:
    """Key latents [Bsz, L, r_k] -> the library's key cache: the same rows,
    per sequence in operand-tile order for bf16 (L % 16 == 0)."""
    return tile_operands(ck) if ck.dtype == np.uint16 else np.ascontiguousarray(ck)


def from_library_key_cache(ck: np.ndarray, bf16: bool) -> np.ndarray:
    """Inverse of to_library_key_cache (bf16: tiled storage order)."""
    return untile_operands(ck) if bf16 else np.ascontiguousarray(ck)


#: positions per cache page of the bf16 caches
PAGE = 64


def to_library_key_pages(pool: np.ndarray) -> np.ndarray:
    """Key-latent pages [..., PAGE, r_k] (bf16 bits) -> library key pages:
    each page's [PAGE, r_k] matrix in operand-tile order."""
    return tile_operands(pool)


def to_library_value_pages(pool: np.ndarray) -> np.ndarray:
    """Value-latent pages [..., PAGE, r_v] (bf16 bits) -> library value
    pages [..., r_v, PAGE]: each page rank-major, in operand-tile order."""
    return tile_operands(np.ascontiguousarray(np.swapaxes(pool, -1, -2)))


def from_library_key_pages(t: np.ndarray) -> np.ndarray:
    """Inverse of to_library_key_pages."""
    return untile_operands(t)


def from_library_value_pages(t: np.ndarray) -> np.ndarray:
    """Inverse of to_library_value_pages."""
    return np.ascontiguousarray(np.swapaxes(untile_operands(t), -1, -2))


def to_library_value_cache(cv: np.ndarray) -> np.ndarray:
    """Value latents [Bsz, L, r_v] -> the library's value cache. bf16: pages
    of PAGE positions, each rank-major [r_v, PAGE] in operand-tile order,
    stored [Bsz, L / PAGE, r_v, PAGE] (L % PAGE == 0); f32: rank-major
    [Bsz, r_v, L]."""
    if cv.dtype == np.uint16:
        Bsz, L, r = cv.shape
        return to_library_value_pages(cv.reshape(Bsz, L // PAGE, PAGE, r))
    return np.ascontiguousarray(np.swapaxes(cv, -1, -2))


def from_library_value_cache(cv_t: np.ndarray, bf16: bool) -> np.ndarray:
    """Inverse of to_library_value_cache."""
    if bf16:
        Bsz, P, r, _ = cv_t.shape
        return from_library_value_pages(cv_t).reshape(Bsz, P * PAGE, r)
    return np.ascontiguousarray(np.swapaxes(cv_t, -1, -2))


# ----------------------------------------------------------------------------
# Paged caches (data movement only)
# ----------------------------------------------------------------------------
def random_block_table(rng: np.random.Generator, Bsz: int, pages_per_seq: int,
                       num_pages: int) -> np.ndarray:
    """A block table [Bsz, pages_per_seq] whose entries are distinct pool
    pages drawn at random from range(num_pages) (num_pages >= Bsz *
    pages_per_seq): no sequence's pages are contiguous or ordered."""
    if num_pages < Bsz * pages_per_seq:
        raise ValueError("pool too small")
    return rng.permutation(num_pages)[:Bsz * pages_per_seq].astype(np.int32).reshape(
        Bsz, pages_per_seq)


def scatter_to_pages(cache: np.ndarray, table: np.ndarray, pool: np.ndarray) -> np.ndarray:
    """Copy contiguous latents [Bsz, P * PAGE, r] into pool pages
    [num_pages, PAGE, r] following the block table; returns the pool."""
    Bsz, L, r = cache.shape
    pool = pool.copy()
    for b in range(Bsz):
        for p in range(L // PAGE):
            pool[table[b, p]] = cache[b, p * PAGE:(p + 1) * PAGE]
    return pool


def random_array(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    """A seeded N(0, std^2) array in storage encoding ("bf16" -> uint16 bits,
    "f32" -> float32), for tests of single entry points."""
    return _encode(_normal(rng, shape, std), dtype)
