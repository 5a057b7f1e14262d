#!/usr/bin/env python3
"""Throughput of one SVD-decomposed transformer layer on one MI355X.

Headline: decode tokens/s of a LLaMA-3-70B-shaped decomposed layer at 50%
compression (batch 32, 8192 cached tokens, one new token per sequence per
step) -- the largest decode configuration that fits one GPU -- with every
projection a factor pair (W ~ A B) and attention rebuilding K/V from the
low-rank cache. The same JSON line carries extra decode legs (the
LLaMA-3-8B-shaped layer at 40%, batch 16 x 1024, and its 20-60% compression
sweep at batch 64 x 4096), the prefill figure of the 70B-shaped layer
(8 sequences x 2048 tokens, TFLOP/s), the roofline of the dominant decode
kernel, a per-kernel breakdown, and the fp64 CPU oracle timed on bounded
samples of the decode and prefill workloads.

A "step" is one dl_decomposed_layer_fwd call over the whole batch. Inputs
are seeded synthetic data resident in HBM before timing starts; two
independent device copies of weights and cache are used in turn so the
256 MB Infinity Cache cannot serve one step from the previous one. Steps are
replayed from one HIP graph that holds --graph-steps steps (the copies in
turn), as a multi-layer model captures its layers, unless --no-graph; a step
count that is not a multiple of that ends with single-step graphs, so exactly
K steps run.

Per-kernel durations come from hipEvents that the library records around
each of its launches on the launch stream. A traced step is queued behind a
spin kernel, so every launch and event is enqueued before the GPU reaches
them and the events time back-to-back execution, not host launch gaps.

The roofline object describes the kernel kind that takes the largest share
of the decode step: achieved = algorithmic bytes (or flops) per launch /
average launch duration. Its "traffic" field is the HBM bytes per launch
measured by rocprofv3 FETCH_SIZE + WRITE_SIZE counters (scaled by the same
counters on a plain copy of known size), read from profiles/traffic.json
only while the kernel sources hash to the value recorded there.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
       python bench.py --calibrate-copy   (one plain device copy of 1 GiB;
                                           run under rocprofv3 --pmc)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decomposed-layer decode tokens/s + % HBM peak; prefill TFLOP/s + % MFMA peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="llama3_70b_c50_decode_b32_l8192")
    p.add_argument("--legs", default="llama3_8b_c40_decode_b16_l1024,"
                   + ",".join(f"llama3_8b_c{c}_decode_b64_l4096" for c in (20, 30, 40, 50, 60))
                   + ",opt30b_c40_decode_b192_l512",
                   help="comma-separated extra decode workloads (empty: none)")
    p.add_argument("--leg-steps", type=int, default=30)
    p.add_argument("--leg-warmup", type=int, default=5)
    p.add_argument("--leg-trace-steps", type=int, default=4)
    p.add_argument("--prefill-workload", default="llama3_70b_c50_prefill_8x2048")
    p.add_argument("--prefill-steps", type=int, default=4)
    p.add_argument("--trace-steps", type=int, default=10)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--graph-steps", type=int, default=8,
                   help="decode steps per graph replay (copies in turn)")
    p.add_argument("--sets", type=int, default=2)
    p.add_argument("--calibrate-copy", action="store_true")
    p.add_argument("--no-pairs", action="store_true",
                   help="skip the fused-versus-separate factor-pair timings")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# algorithmic work per launch role (bytes moved at minimum / flops of the method)
# ----------------------------------------------------------------------------
def decode_role_work(shape, M, ctx_total):
    """Per-step algorithmic bytes of each GEMV launch (bf16 weights read once,
    activations in and out at the dtype the layer passes between launches)
    and of the attention kernel, plus attention flops, counted two ways:

    own   -- the kernel's association: keys rebuilt per attended position
             (2 r_k n_kv d), scores (2 d per query head), probabilities
             applied to the value latents (2 r_v per query head), then the
             value factor once per query head (2 r_v d);
    pages -- the pages' explicit rebuild of K and V per position
             (2 (r_k + r_v) n_kv d) plus scores and P V (4 n_q d).

    ctx_total = sum over sequences of the rows attended."""
    h, f, qd, kvd = shape.hidden, shape.ffn, shape.n_q * shape.head_dim, shape.n_kv * shape.head_dim
    r = {p: shape.rank(p) for p in shape.projections()}
    b16, f32 = 2, 4
    rqkv, rgu = r["q"] + r["k"] + r["v"], r.get("gate", 0) + r["up"]
    gemv = {
        "qkv_down": b16 * h * rqkv + M * h * b16 + M * rqkv * b16,
        "q_up": b16 * r["q"] * qd + M * r["q"] * b16 + M * qd * f32,
        "o_down": b16 * qd * r["o"] + M * qd * b16 + M * r["o"] * b16,
        "o_up": b16 * r["o"] * h + M * r["o"] * b16 + M * h * b16 + M * h * f32,
        "gate_up_down": b16 * h * rgu + M * h * f32 + M * rgu * b16,
        "gate_up_up": b16 * rgu * f + M * rgu * b16 + M * f * b16,
        "down_down": b16 * f * r["down"] + M * f * b16 + M * r["down"] * b16,
        "down_up": b16 * r["down"] * h + M * r["down"] * b16 + M * h * f32 + M * h * b16,
    }
    # the fused chains: [A_q A_k A_v] then B_q; the o pair through the down pair
    gemv["qkv_chain"] = gemv["qkv_down"] + gemv["q_up"]
    gemv["o_mlp_chain"] = sum(gemv[k] for k in ("o_down", "o_up", "gate_up_down", "gate_up_up",
                                                "down_down", "down_up"))
    attn_bytes = ctx_total * (r["k"] + r["v"]) * b16 + b16 * kvd * (r["k"] + r["v"]) + M * qd * (f32 + b16)
    if shape.rope_theta == 0:
        # latent path: B_k into the query, scores and P C_v on the latents,
        # B_v once per query head
        attn_flops_own = (ctx_total * shape.n_q * 2 * (r["k"] + r["v"])
                          + M * shape.n_q * 2 * shape.head_dim * (r["k"] + r["v"]))
    else:
        attn_flops_own = (ctx_total * (2 * r["k"] * kvd + shape.n_q * (2 * shape.head_dim + 2 * r["v"]))
                          + M * shape.n_q * 2 * r["v"] * shape.head_dim)
    attn_flops_pages = ctx_total * (2 * (r["k"] + r["v"]) * kvd + 4 * qd)
    return gemv, attn_bytes, attn_flops_own, attn_flops_pages


def prefill_flops(shape, Bsz, T):
    """Algorithmic flops of one prefill step: all factor pairs over M = Bsz*T
    tokens (the k/v up halves are the one-time rebuild of every cached row)
    plus the causal attention core 4 * n_q * d per (query, visible key)."""
    M = Bsz * T
    pairs = sum(2 * M * (m * shape.rank(p) + shape.rank(p) * n) for p, (m, n) in shape.shapes().items())
    core = Bsz * (T * (T + 1) // 2) * 4 * shape.n_q * shape.head_dim
    gemm = pairs - sum(2 * M * shape.rank(p) * n for p, (m, n) in shape.shapes().items() if p in ("k", "v"))
    return pairs + core, gemm, core


# ----------------------------------------------------------------------------
# GPU runs
# ----------------------------------------------------------------------------
def to_dev(torch, a):
    import numpy as np
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    if a.dtype == np.int32:
        return torch.from_numpy(a).to("cuda:0")
    return torch.from_numpy(a.astype(np.float32)).to("cuda:0")


def make_sets(torch, binding, weights, inp, nsets):
    from rank_decomposed_linear_amd import workloads as W
    shp = weights.shape
    Bsz, T = inp.x.shape[0], inp.x.shape[1]
    L_max = inp.ck.shape[1]
    sets = []
    for _ in range(nsets):
        lf = W.to_library_factor
        facs = {p: (to_dev(torch, lf(a)), to_dev(torch, lf(b))) for p, (a, b) in weights.factors.items()}
        layer = binding.DecomposedLayer(facs, shp.hidden, shp.n_q, shp.n_kv, shp.head_dim, shp.ffn,
                                        shp.rope_theta, shp.rms_eps, mlp=shp.mlp)
        st = dict(layer=layer, x=to_dev(torch, inp.x), ck=to_dev(torch, W.to_library_key_cache(inp.ck)),
                  cv=to_dev(torch, W.to_library_value_cache(inp.cv)),
                  past=to_dev(torch, inp.past_lens))
        st["y"] = torch.empty_like(st["x"])
        st["ws"] = torch.empty(max(layer.workspace_bytes(Bsz, T, L_max), 16), dtype=torch.uint8,
                               device="cuda:0")
        sets.append(st)
    return sets


def run_step(st):
    st["layer"].forward(st["x"], st["ck"], st["cv"], st["past"], y=st["y"], ws=st["ws"])


def capture_graphs(torch, sets, chain_steps):
    """One graph per copy, plus one graph of chain_steps steps that runs the
    copies in turn."""
    graphs = []
    side = torch.cuda.Stream()
    for st in sets:
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run_step(st)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_step(st)
        graphs.append(g)
    chain = torch.cuda.CUDAGraph()
    with torch.cuda.graph(chain):
        for i in range(chain_steps):
            run_step(sets[i % len(sets)])
    torch.cuda.synchronize()
    return graphs, chain


def step_fn(graphs, chain, chain_steps, steps):
    """fn(i) for i < calls runs the steps: chained replays, then singles (the
    copies continue in turn)."""
    full = steps // chain_steps
    calls = full + steps % chain_steps
    return (lambda i: chain.replay() if i < full else
            graphs[(full * chain_steps + i - full) % len(graphs)].replay()), calls


def timed(torch, fn, steps, warmup):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        fn(i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return t0.elapsed_time(t1) / steps, wall


def trace_breakdown(torch, binding, sets, nsteps):
    """Per-kernel durations from hipEvents recorded around every library
    launch, over nsteps steps, each queued behind a spin kernel so the
    events time GPU execution only. Returns {(kind, role): [ms, ...]}."""
    tr = binding.KernelTrace(capacity=64 * nsteps + 64)
    torch.cuda.synchronize()
    with tr:
        for i in range(nsteps):
            torch.cuda._sleep(2_000_000)   # spin so the step's launches queue up behind it
            run_step(sets[i % len(sets)])
            torch.cuda.synchronize()
    per = {}
    for kind, role, ms in tr.records():
        per.setdefault((kind, role), []).append(ms)
    tr.close()
    return per


def kernel_source_hash():
    from rank_decomposed_linear_amd.profiling import source_hash
    return source_hash()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary, or None when absent or taken on other sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def decode_bench(args, torch, binding, W, name, steps, warmup, trace_steps, nsets):
    """Times `steps` decode steps of workload `name` (after `warmup`) and
    traces `trace_steps` more for the per-kernel breakdown and rooflines."""
    w = W.by_name(name)
    log(f"decode workload {w.name}: drawing inputs")
    weights, inp = W.draw(w)
    sets = make_sets(torch, binding, weights, inp, nsets)
    Bsz = w.batch
    # eager reference output of set 0, then (optionally) graphs
    run_step(sets[0])
    torch.cuda.synchronize()
    y_eager = sets[0]["y"].clone()
    use_graph = not args.no_graph
    graphs = None
    chain_steps = max(1, args.graph_steps)
    if use_graph:
        try:
            graphs, chain = capture_graphs(torch, sets, chain_steps)
            for g in (graphs[0], chain, graphs[0]):
                sets[0]["y"].zero_()
                g.replay()
                torch.cuda.synchronize()
                if not torch.equal(sets[0]["y"], y_eager):
                    raise RuntimeError("graph replay differs from the eager output")
        except Exception as e:  # keep the eager figure if capture is refused
            log(f"graph capture disabled: {e}")
            use_graph, graphs = False, None
    log(f"timing {steps} steps after {warmup} warmup (graph={use_graph})")
    if graphs:
        fn, calls = step_fn(graphs, chain, chain_steps, steps)
        wfn, wcalls = step_fn(graphs, chain, chain_steps, warmup)
        for i in range(wcalls):
            wfn(i)
        ms, wall = timed(torch, fn, calls, 0)
        ms *= calls / steps
    else:
        fn = lambda i: run_step(sets[i % len(sets)])
        ms, wall = timed(torch, fn, steps, warmup)

    per = trace_breakdown(torch, binding, sets, trace_steps)
    ctx_total = int(sum(int(p) + 1 for p in inp.past_lens))
    gemv_bytes, attn_bytes, attn_own, attn_pages = decode_role_work(w.shape, Bsz, ctx_total)
    n = trace_steps
    kinds = {}
    for (kind, role), lst in per.items():
        k = kinds.setdefault(kind, {"ms_per_step": 0.0, "launches_per_step": 0, "bytes_per_step": 0,
                                    "flops_per_step": 0, "pages_flops_per_step": 0})
        k["ms_per_step"] += sum(lst) / n
        k["launches_per_step"] += len(lst) // n
        if kind in ("gemv_bf16", "gemv_chain", "gemm_bf16"):
            k["bytes_per_step"] += gemv_bytes.get(role, 0) * (len(lst) // n)
        if kind in ("attn_decode_bf16", "attn_latent"):
            k["bytes_per_step"] += attn_bytes
            k["flops_per_step"] += attn_own
            k["pages_flops_per_step"] += attn_pages
    breakdown = {}
    for kind, k in sorted(kinds.items(), key=lambda kv: -kv[1]["ms_per_step"]):
        e = {"us_per_step": round(k["ms_per_step"] * 1e3, 2), "launches_per_step": k["launches_per_step"],
             "avg_us": round(k["ms_per_step"] * 1e3 / max(k["launches_per_step"], 1), 2)}
        if k["bytes_per_step"]:
            gbs = k["bytes_per_step"] / (k["ms_per_step"] * 1e-3) / 1e9
            e["GB_per_s"] = round(gbs, 1)
            e["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
        if k["flops_per_step"]:
            tf = k["flops_per_step"] / (k["ms_per_step"] * 1e-3) / 1e12
            e["TFLOP_per_s"] = round(tf, 2)
            e["mfma_frac"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
        breakdown[kind] = e
    roles = {f"{kind}/{role}": round(sum(lst) / n * 1e3, 2) for (kind, role), lst in sorted(per.items())}

    def roofline(kname):
        k = kinds[kname]
        nl = max(k["launches_per_step"], 1)
        avg_s = k["ms_per_step"] * 1e-3 / nl
        if kname == "attn_latent":
            # HBM-bound: the latents once per head group, plus the factors
            achieved = k["bytes_per_step"] / nl / avg_s / 1e9
            tf = k["flops_per_step"] / nl / avg_s / 1e12
            return {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(kname, w.name),
                    "avg_us": round(avg_s * 1e6, 2), "launches_per_step": nl,
                    "algorithmic_bytes_per_launch": int(k["bytes_per_step"] / nl),
                    "algorithmic_flops_per_launch": int(k["flops_per_step"] / nl),
                    "TFLOP_per_s": round(tf, 2),
                    "flops_counted": "latent association: B_k into the query, scores and P C_v on "
                                     "the cached latents, B_v once per query head"}
        if kname == "attn_decode_bf16":
            achieved = k["flops_per_step"] / nl / avg_s / 1e12
            pages = k["pages_flops_per_step"] / nl / avg_s / 1e12
            return {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 2),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": measured_traffic(kname, w.name),
                    "avg_us": round(avg_s * 1e6, 2), "launches_per_step": nl,
                    "algorithmic_flops_per_launch": int(k["flops_per_step"] / nl),
                    "flops_counted": "own association: K rebuilt per position, scores, P C_v, "
                                     "then B_v once per query head",
                    "pages_explicit_rebuild_flops_per_launch": int(k["pages_flops_per_step"] / nl),
                    "pages_explicit_rebuild_TFLOP_per_s": round(pages, 2),
                    "pages_explicit_rebuild_frac": round(pages / MFMA_BF16_PEAK_TFLOPS, 4),
                    "algorithmic_bytes_per_launch": int(k["bytes_per_step"] / nl)}
        achieved = k["bytes_per_step"] / nl / avg_s / 1e9
        return {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(kname, w.name),
                "avg_us": round(avg_s * 1e6, 2), "launches_per_step": nl,
                "algorithmic_bytes_per_launch": int(k["bytes_per_step"] / nl)}

    # dominant kernel kind of the step (largest share of the step time)
    dname = max(kinds.items(), key=lambda kv: kv[1]["ms_per_step"])[0]
    roof = roofline(dname)
    aname = "attn_latent" if "attn_latent" in kinds else "attn_decode_bf16"
    roof_attn = roofline(aname) if aname in kinds else None
    gname = ("gemv_chain" if "gemv_chain" in kinds else
             "gemv_bf16" if "gemv_bf16" in kinds else "gemm_bf16")
    roof_gemv = roofline(gname) if gname in kinds else None
    step_bytes = W.algorithmic_decode_bytes(w.shape, Bsz, ctx_total // Bsz)["total"]
    result = {
        "value": Bsz / (ms * 1e-3), "ms_per_step": ms, "wall_s": wall, "graph": use_graph,
        "steps_per_graph": chain_steps if use_graph else None,
        "roofline": roof, "roofline_attention": roof_attn, "roofline_gemv": roof_gemv,
        "kernels": breakdown, "roles_us_per_step": roles,
        "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "config": {"workload": w.name, "batch": Bsz, "context": int(inp.past_lens[0]) + 1,
                   "hidden": w.shape.hidden, "n_q": w.shape.n_q, "n_kv": w.shape.n_kv,
                   "head_dim": w.shape.head_dim, "ffn": w.shape.ffn,
                   "compression_pct": w.compression_pct, "ranks": dict(w.shape.ranks),
                   "weight_sets": nsets},
    }
    del sets
    torch.cuda.empty_cache()
    return result, weights, inp


def decode_leg(args, torch, binding, W, name, peaks):
    r, _, _ = decode_bench(args, torch, binding, W, name, args.leg_steps, args.leg_warmup,
                           args.leg_trace_steps, args.sets)
    return {"workload": name, "tokens_per_s": round(r["value"], 1),
            "ms_per_step": round(r["ms_per_step"], 5), "steps": args.leg_steps,
            "step_hbm_frac": r["step_hbm_frac"],
            "roofline_attention": with_measured(r["roofline_attention"], peaks),
            "roofline_gemv": with_measured(r["roofline_gemv"], peaks),
            "kernels": r["kernels"], "config": r["config"]}


def prefill_bench(args, torch, binding, W):
    w = W.by_name(args.prefill_workload)
    log(f"prefill workload {w.name}: drawing inputs")
    weights, inp = W.draw(w)
    sets = make_sets(torch, binding, weights, inp, 1)
    fn = lambda i: run_step(sets[0])
    ms, wall = timed(torch, fn, args.prefill_steps, 1)
    per = trace_breakdown(torch, binding, sets, 1)
    total, gemm, core = prefill_flops(w.shape, w.batch, w.prefill)
    gemm_ms = sum(sum(v) for (k, _), v in per.items() if k == "gemm_bf16")
    attn_ms = sum(sum(v) for (k, _), v in per.items() if k == "attn_prefill_bf16")
    tf = total / (ms * 1e-3) / 1e12
    gemm_tf = gemm / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None
    out = {"workload": w.name, "TFLOP_per_s": round(tf, 2),
           "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "ms_per_step": round(ms, 3),
           "algorithmic_TFLOP_per_step": round(total / 1e12, 3),
           "gemm_TFLOP_per_s": round(gemm_tf, 2) if gemm_tf else None,
           "gemm_mfma_frac": round(gemm_tf / MFMA_BF16_PEAK_TFLOPS, 4) if gemm_tf else None,
           "gemm_ms": round(gemm_ms, 3), "attention_ms": round(attn_ms, 3),
           "roles_ms": {f"{k}/{r}": round(sum(v), 3) for (k, r), v in sorted(per.items())},
           "steps": args.prefill_steps}
    del sets
    torch.cuda.empty_cache()
    return out, (w, weights, inp)


# ----------------------------------------------------------------------------
# Fused factor pair (decode-sized M): one persistent launch vs two launches
# ----------------------------------------------------------------------------
PAIR_SHAPES = (("llama3_8b_c40_o_pair", 16, 4096, 1216, 4096),
               ("llama3_70b_c50_o_pair", 32, 8192, 2048, 8192),
               ("llama3_70b_c50_gate_pair", 32, 8192, 3136, 28672))


def fused_pair_bench(torch, binding, calls=40):
    """dl_lowrank_linear y = (x A) B at decode sizes, timed from a captured
    graph of `calls` calls over enough independent weight copies that the
    Infinity Cache cannot hold them, with the pair fused into one launch
    (DL_FUSED_CHAIN=pair) and as two launches (none). Bytes are the factor
    bytes plus x and y."""
    out = []
    for name, M, m, k, n in PAIR_SHAPES:
        nbytes = 2 * (m * k + k * n)
        copies = max(2, -(-640_000_000 // nbytes))
        dev = "cuda:0"
        x = torch.randn(M, m, device=dev).to(torch.bfloat16)
        ws_list = [(torch.randn(k, m, device=dev).mul_(0.02).to(torch.bfloat16),
                    torch.randn(n, k, device=dev).mul_(0.02).to(torch.bfloat16)) for _ in range(copies)]
        y = torch.empty(M, n, dtype=torch.bfloat16, device=dev)
        res = {"pair": name, "M": M, "m": m, "k": k, "n": n, "weight_copies": copies}
        for mode in ("pair", "none"):
            os.environ["DL_FUSED_CHAIN"] = mode
            need = binding.load().dl_lowrank_linear_workspace(M, m, k, n, binding.DL_BF16)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                binding.lowrank_linear(x, *ws_list[0], y=y, ws=ws)
            torch.cuda.current_stream().wait_stream(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(calls):
                    binding.lowrank_linear(x, *ws_list[i % copies], y=y, ws=ws)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (3 * calls)
            gbs = (nbytes + 2 * M * (m + n)) / (us * 1e-6) / 1e9
            res["fused_us" if mode == "pair" else "separate_us"] = round(us, 2)
            res["fused_GB_per_s" if mode == "pair" else "separate_GB_per_s"] = round(gbs, 1)
            del g
        os.environ.pop("DL_FUSED_CHAIN", None)
        out.append(res)
        del ws_list
        torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------
# Measured peaks (denominators reported beside the published ones)
# ----------------------------------------------------------------------------
def measured_peaks(torch, binding):
    """Rates this GPU sustains: a 1 GiB device-to-device copy ((read + write)
    bytes per second, best of 5 after a warm-up) and the library's matrix-pipe
    probe (independent bf16 MFMA chains, best of 3 after a warm-up)."""
    dev = torch.device("cuda:0")
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best_ms(fn, reps):
        fn()
        best = float("inf")
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    copy_ms = best_ms(lambda: dst.copy_(src), 5)
    del src, dst
    blocks, iters = 256 * 4, 2048
    sink = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    flops = blocks * 8 * iters * 32 * 16384
    mfma_ms = best_ms(lambda: binding.probe_mfma_bf16(sink, blocks, iters), 3)
    return {"hbm_copy_GB_per_s": round(2 * n / (copy_ms * 1e-3) / 1e9, 1),
            "mfma_bf16_TFLOP_per_s": round(flops / (mfma_ms * 1e-3) / 1e12, 1),
            "method": "1 GiB device copy, (read + write) bytes / time, best of 5; "
                      "dl_probe_mfma_bf16 with 1024 workgroups x 8 waves x 2048 rounds of 12 "
                      "LDS operand reads and 32 independent 16x16x32 bf16 MFMAs (the prefill "
                      "GEMM's mix, random operands), best of 3"}


def with_measured(roof, peaks):
    """Adds the fraction of the measured peak to a roofline object."""
    if roof is None or peaks is None:
        return roof
    mp = peaks["hbm_copy_GB_per_s"] if roof["unit"] == "GB/s" else peaks["mfma_bf16_TFLOP_per_s"]
    roof["measured_peak"] = mp
    roof["frac_of_measured"] = round(roof["achieved"] / mp, 4)
    return roof


# ----------------------------------------------------------------------------
# CPU oracle baseline
# ----------------------------------------------------------------------------
def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(args, W, weights, inp, prefill):
    """The fp64 oracle as it stands, on the host cores: full decode steps of
    the headline workload for about --cpu-seconds, then one sequence of the
    prefill workload (a labelled subset)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import ref

    ncores = len(os.sched_getaffinity(0))
    f64 = lambda a: W.decode_array(a).astype(np.float64)
    F = {p: (f64(a), f64(b)) for p, (a, b) in weights.factors.items()}
    x, ck, cv = (f64(a) for a in (inp.x, inp.ck, inp.cv))
    shp = weights.shape
    out = {"kind": "oracle", "cpu_model": cpu_model(), "logical_cpus_available": ncores}
    with threadpool_limits(limits=ncores):
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        steps, t0 = 0, time.perf_counter()
        while True:
            ref.decomposed_layer(F, x, ck, cv, inp.past_lens, shp.n_q, shp.n_kv, shp.head_dim,
                                 shp.rope_theta, shp.rms_eps)
            steps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or steps >= 1000:
                break
        Bsz = inp.x.shape[0]
        out.update({"value": round(Bsz * steps / el, 3), "unit": "tokens/s", "cores": threads,
                    "sample": f"{steps} full decode steps of the headline workload (batch {Bsz}, "
                              f"context {int(inp.past_lens[0]) + 1}), fp64 numpy, {el:.1f} s"})
        del F, x, ck, cv
        if prefill is not None:
            w, pw, pin = prefill
            PF = {p: (f64(a), f64(b)) for p, (a, b) in pw.factors.items()}
            s1 = slice(0, 1)
            t0 = time.perf_counter()
            ref.decomposed_layer(PF, f64(pin.x)[s1], f64(pin.ck)[s1], f64(pin.cv)[s1],
                                 pin.past_lens[s1], w.shape.n_q, w.shape.n_kv, w.shape.head_dim,
                                 w.shape.rope_theta, w.shape.rms_eps)
            el = time.perf_counter() - t0
            total, _, _ = prefill_flops(w.shape, 1, w.prefill)
            out["prefill"] = {"value": round(total / el / 1e12, 5), "unit": "TFLOP/s",
                              "cores": threads,
                              "sample": f"sequence 0 of {w.name} ({w.prefill} tokens, 1 of "
                                        f"{w.batch} sequences), fp64 numpy, {el:.1f} s"}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(requested --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    from rank_decomposed_linear_amd import binding, workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        # one plain device-to-device copy of 1 GiB: the reference for the
        # FETCH_SIZE / WRITE_SIZE counter scale
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}), flush=True)
        return
    binding.load()
    peaks = measured_peaks(torch, binding)
    log(f"measured peaks: {peaks['hbm_copy_GB_per_s']} GB/s copy, "
        f"{peaks['mfma_bf16_TFLOP_per_s']} TFLOP/s bf16 MFMA")
    dec, weights, inp = decode_bench(args, torch, binding, W, args.workload, args.steps,
                                     args.warmup, args.trace_steps, args.sets)
    log(f"decode: {dec['value']:.0f} tokens/s, {dec['ms_per_step'] * 1e3:.1f} us/step")
    legs = []
    for name in [n for n in args.legs.split(",") if n]:
        legs.append(decode_leg(args, torch, binding, W, name, peaks))
        log(f"leg {name}: {legs[-1]['tokens_per_s']:.0f} tokens/s")
    pairs = None if args.no_pairs else fused_pair_bench(torch, binding)
    for p in pairs or []:
        log(f"factor pair {p['pair']}: fused {p['fused_us']} us, separate {p['separate_us']} us")
    pre = pre_inputs = None
    if not args.no_prefill:
        pre, pre_inputs = prefill_bench(args, torch, binding, W)
        pre["mfma_frac_of_measured"] = round(pre["TFLOP_per_s"] / peaks["mfma_bf16_TFLOP_per_s"], 4)
        if pre["gemm_TFLOP_per_s"]:
            pre["gemm_frac_of_measured"] = round(pre["gemm_TFLOP_per_s"] / peaks["mfma_bf16_TFLOP_per_s"], 4)
        log(f"prefill: {pre['TFLOP_per_s']} TFLOP/s")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(args, W, weights, inp, pre_inputs)
    line = {
        "metric": METRIC, "value": round(dec["value"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; random-init factors, pre-filled low-rank cache)",
        "config": dec["config"], "graph": dec["graph"], "steps_per_graph": dec["steps_per_graph"],
        "roofline": with_measured(dec["roofline"], peaks),
        "roofline_attention": with_measured(dec["roofline_attention"], peaks),
        "roofline_gemv": with_measured(dec["roofline_gemv"], peaks),
        "measured_peaks": peaks,
        "step_hbm_frac": dec["step_hbm_frac"], "kernel_source_hash": kernel_source_hash(),
        "cpu_baseline": cpu, "prefill": pre, "decode_legs": legs, "factor_pairs": pairs,
        "kernels": dec["kernels"],
        "roles_us_per_step": dec["roles_us_per_step"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
