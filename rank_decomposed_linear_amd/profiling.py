"""Summaries of rocprofv3 output for the library's kernels.

Reads the SQLite results that `rocprofv3 -d DIR -o run ...` writes and
prints short text tables (for profiles/) or the per-launch HBM traffic JSON
that bench.py reports in its roofline object.

  python -m rank_decomposed_linear_amd.profiling kernels DB --command CMD
      per-kernel dispatch count and duration statistics of a
      `rocprofv3 --kernel-trace --stats` run

  python -m rank_decomposed_linear_amd.profiling mfma --pmc DB --trace DB --measured TFLOPS
      --command CMD
      executed bf16 MFMA flops per kernel (`rocprofv3 --pmc
      SQ_INSTS_VALU_MFMA_MOPS_BF16`) over the kernel-trace durations

  python -m rank_decomposed_linear_amd.profiling traffic --fetch DB --write DB
      --cal-fetch DB --cal-write DB --copy-bytes N --workload NAME
      --command CMD [--json OUT]
      HBM bytes per launch from two `rocprofv3 --pmc FETCH_SIZE` /
      `--pmc WRITE_SIZE` runs, each scaled by what the same counter reads for
      a plain device copy of N bytes (`bench.py --calibrate-copy`)

Kernel kinds follow the names the library's launch trace uses.
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# device function name fragment -> kernel kind (the launch trace's names)
KINDS = (
    ("gemv_chain_kernel", "gemv_chain"),
    ("gemv_kernel", "gemv_bf16"),
    ("attn_decode_kernel", "attn_decode_bf16"),
    ("attn_decode_ws_kernel", "attn_decode_bf16"),
    ("attn_prefill_kernel", "attn_prefill_bf16"),
    ("attn_rebuild_kernel", "attn_prefill_bf16"),
    ("latent_query_kernel", "attn_latent"),
    ("latent_attn_kernel", "attn_latent"),
    ("latent_out_kernel", "attn_latent"),
    ("gemm_bf16_kernel", "gemm_bf16"),
    ("gemm_bf16_fixup_kernel", "gemm_bf16"),
    ("gemm_f32_kernel", "gemm_f32"),
    ("attn_f32_kernel", "attn_f32"),
    ("pack_up_factor_kernel", "pack_up_factor"),
    ("rmsnorm_kernel", "rmsnorm"),
    ("rmsnorm_vec_kernel", "rmsnorm"),
    ("norm_tiles_kernel", "rmsnorm"),
    ("fill_kernel", "fill"),
    ("convert_kernel", "convert"),
    ("store_cache_rows_kernel", "store_cache_rows"),
)

KERNEL_SOURCES = ("gemv_bf16.hip", "attn_decode_bf16.hip", "attn_bf16.hip", "attn_latent_bf16.hip",
                  "gemm_bf16.hip", "elementwise.hip", "common.h", "kernels.h")


def source_hash() -> str:
    """Hash of the kernel sources (bench.py compares it before trusting
    counter values taken on an earlier build)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rank_decomposed_linear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kind_of(name: str) -> str:
    for frag, kind in KINDS:
        if frag in name:
            return kind
    return "other:" + name.split("(")[0][:48]


def short_name(name: str) -> str:
    s = name.replace("void ", "").replace("dl::(anonymous namespace)::", "")
    return s.split("(dl::")[0].split("(")[0][:60]


def _db(path: str) -> sqlite3.Connection:
    if os.path.isdir(path):
        for dp, _, fs in os.walk(path):
            for f in fs:
                if f.endswith(".db"):
                    return sqlite3.connect(os.path.join(dp, f))
        raise FileNotFoundError(f"no .db under {path}")
    return sqlite3.connect(path)


def kernel_table(db: str, command: str) -> str:
    c = _db(db)
    rows = c.execute("select name, grid_x, grid_y, grid_z, workgroup_x, duration from kernels "
                     "order by start").fetchall()
    agg = collections.OrderedDict()
    for name, gx, gy, gz, wx, d in rows:
        key = (short_name(name), gx // max(wx, 1), gy, gz)
        agg.setdefault(key, []).append(d / 1000.0)
    out = [f"# rocprofv3 kernel trace: {command}",
           "# kernel (workgroups x, y, z): dispatches, average / median / min / max duration in us",
           ""]
    for (nm, wgx, gy, gz), v in agg.items():
        if not any(frag in nm for frag, _ in KINDS):
            continue
        v = sorted(v)
        out.append(f"{nm:52s} ({wgx}, {gy}, {gz})  n={len(v):4d}  avg={sum(v) / len(v):9.2f}  "
                   f"med={v[len(v) // 2]:9.2f}  min={v[0]:9.2f}  max={v[-1]:9.2f}")
    return "\n".join(out) + "\n"


def _counter(db: str, counter: str):
    c = _db(db)
    return [(n, v) for n, v in c.execute(
        "select kernel_name, value from counters_collection where counter_name = ? "
        "order by dispatch_id", (counter,))]


def _copy_kib(db: str, counter: str) -> float:
    vals = [v for n, v in _counter(db, counter) if "copyBuffer" in n or "copy" in n.lower()]
    if not vals:
        raise RuntimeError(f"no copy dispatch with {counter} in {db}")
    return max(vals)


def mfma_table(pmc_db: str, trace_db: str, command: str, peak_tflops: float,
               measured_tflops: float) -> str:
    """Executed bf16 MFMA work per kernel from a `rocprofv3 --pmc
    SQ_INSTS_VALU_MFMA_MOPS_BF16` run (the counter counts operations / 512),
    over the average duration of the same kernel and grid in a kernel-trace
    run: the counter-measured matrix-pipe rate."""
    c = _db(pmc_db)
    per = collections.OrderedDict()
    rows = c.execute("select dispatch_id, kernel_name, grid_size_x, grid_size_y, grid_size_z, "
                     "workgroup_size_x, value from counters_collection where counter_name = ? "
                     "order by dispatch_id", ("SQ_INSTS_VALU_MFMA_MOPS_BF16",)).fetchall()
    disp = collections.OrderedDict()
    for did, name, gx, gy, gz, wx, v in rows:
        key = (short_name(name), gx // max(wx, 1), gy, gz)
        disp.setdefault(did, [key, 0.0])[1] += v * 512.0
    for key, flops in disp.values():
        per.setdefault(key, []).append(flops)
    t = _db(trace_db)
    dur = collections.defaultdict(list)
    for name, gx, gy, gz, wx, d in t.execute("select name, grid_x, grid_y, grid_z, workgroup_x, duration "
                                             "from kernels").fetchall():
        dur[(short_name(name), gx // max(wx, 1), gy, gz)].append(d * 1e-9)
    out = [f"# bf16 MFMA work from counters: {command}",
           f"# rate = counter flops per launch / average duration of the same kernel and grid in the kernel trace;",
           f"# fractions of the published {peak_tflops:.0f} TFLOP/s and of the measured 16x16x32 GEMM-mix rate "
           f"{measured_tflops:.0f} TFLOP/s",
           "# kernel (workgroups x, y, z): launches, TFLOP per launch, average us, TFLOP/s, published, measured",
           ""]
    for (nm, wgx, gy, gz), fl in per.items():
        f = sum(fl) / len(fl)
        if f <= 0 or not any(frag in nm for frag, _ in KINDS):
            continue
        d = dur.get((nm, wgx, gy, gz))
        if not d:
            continue
        avg = sum(d) / len(d)
        rate = f / avg / 1e12
        out.append(f"{nm:40s} ({wgx}, {gy}, {gz})  n={len(fl):3d}  {f / 1e12:8.4f} TF  {avg * 1e6:9.2f} us  "
                   f"{rate:8.1f} TFLOP/s  {rate / peak_tflops:6.1%}  {rate / measured_tflops:6.1%}")
    return "\n".join(out) + "\n"


def traffic(fetch_db, write_db, cal_fetch_db, cal_write_db, copy_bytes, workload, command):
    fscale = copy_bytes / (_copy_kib(cal_fetch_db, "FETCH_SIZE") * 1024.0)
    wscale = copy_bytes / (_copy_kib(cal_write_db, "WRITE_SIZE") * 1024.0)
    per = {}
    for db, counter, scale, field in ((fetch_db, "FETCH_SIZE", fscale, "fetch"),
                                      (write_db, "WRITE_SIZE", wscale, "write")):
        for name, kib in _counter(db, counter):
            k = kind_of(name)
            if k.startswith("other:"):
                continue
            e = per.setdefault(k, {"fetch": [], "write": []})
            e[field].append(kib * 1024.0 * scale)
    kernels = {}
    for k, e in per.items():
        n = max(len(e["fetch"]), 1)
        f = sum(e["fetch"]) / n
        w = sum(e["write"]) / max(len(e["write"]), 1)
        kernels[k] = {"launches_profiled": n, "fetch_bytes_per_launch": int(f),
                      "write_bytes_per_launch": int(w), "hbm_bytes_per_launch": int(f + w)}
    return {"workload": workload, "source_hash": source_hash(), "command": command,
            "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
            "copy_bytes": copy_bytes, "kernels": kernels}


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = p.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("db")
    k.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--cal-fetch", "--cal-write", "--workload", "--command"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--json")
    m = sub.add_parser("mfma")
    for x in ("--pmc", "--trace", "--command"):
        m.add_argument(x, required=True)
    m.add_argument("--peak", type=float, default=2500.0)
    m.add_argument("--measured", type=float, required=True)
    a = p.parse_args(argv)
    if a.cmd == "kernels":
        sys.stdout.write(kernel_table(a.db, a.command))
        return
    if a.cmd == "mfma":
        sys.stdout.write(mfma_table(a.pmc, a.trace, a.command, a.peak, a.measured))
        return
    r = traffic(a.fetch, a.write, a.cal_fetch, a.cal_write, a.copy_bytes, a.workload, a.command)
    if a.json:
        with open(a.json, "w") as fh:
            json.dump(r, fh, indent=1)
            fh.write("\n")
    print(f"# HBM traffic per launch, {a.workload}: {a.command}")
    print(f"# FETCH_SIZE x {r['fetch_scale']}, WRITE_SIZE x {r['write_scale']} "
          f"(calibrated on a {a.copy_bytes}-byte device copy); kernel sources {r['source_hash']}")
    for kk, e in sorted(r["kernels"].items()):
        print(f"{kk:20s} launches={e['launches_profiled']:4d}  fetch={e['fetch_bytes_per_launch'] / 1e6:10.3f} MB"
              f"  write={e['write_bytes_per_launch'] / 1e6:9.3f} MB  total={e['hbm_bytes_per_launch'] / 1e6:10.3f} MB")


if __name__ == "__main__":
    main()
