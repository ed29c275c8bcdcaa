"""Benchmark of the windowed atom-attention block on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1]

A step is one call of the whole block (pack, [token projection], prep,
slot attention, post, [pool]) on one batch of synthetic input of the named
workload. Inputs are resident in HBM before the timed region; to keep the
256 MB Infinity Cache from serving them, the step cycles through enough
copies of the inputs that they do not fit in it. The timed region is exactly
K steps between two device synchronisations and gives the throughput. A
second timed region of the same K steps runs with the library's profiling
mode on: HIP events recorded around each launch on the stream it launches
on give every kernel's average duration (the roofline figures).

Prints ONE JSON line: metric entries/s (B*A*H*K per second), plus
atoms/s, the roofline of the dominant kernel and the fp64 oracle's rate on
the host cores.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}  # dense matrix peaks


def kernel_work(w, split=False):
    """Algorithmic work per launch of each kernel: ('hbm', bytes) for the
    bandwidth-bound slot attention, ('mfma', flops) for the projections.
    With the AF3 pair bias split off (`split`: the projection kernel's extra
    workgroups stream the pair rows and write 16 bytes of bias per slot),
    the slot kernel reads that bias instead of the pair rows."""
    d = w.dims
    B, A, T, K, C, S, H, D, V, M, U = (d[k] for k in "B A T K C S H D V M U".split())
    HD = H * D
    e = 2 if w.dtype.itemsize == 2 else 4
    N, E = B * A, B * A * K
    af3 = w.style == "af3"
    pair = (E * 16 if split else E * V * e) if af3 else 0
    slot_bytes = (3 * N * HD * e + 8 * E + E + N + pair
                  + E * H * e + N * HD * e)
    if af3:
        prep = N * 2 * (4 * S * C + 4 * C * HD)
        post = N * 2 * (HD * C + S * C + 2 * S * C + 2 * C * M + M * C + S * C)
    else:
        prep = N * 2 * (2 * S * C + 4 * C * HD)
        post = N * 2 * (HD * C + S * C + 2 * S * C + 2 * C * M + M * C + S * C)
    work = {"slot_attention": ("hbm", slot_bytes), "prep": ("mfma", prep),
            "post": ("mfma", post)}
    if w.stage == "encoder":
        # the pooled projection runs inside post; the pool kernel only joins
        # tokens that cross 32-row tiles (reads the tile records, writes at
        # most two token rows per tile)
        work["post"] = ("mfma", post + N * 2 * C * U)
        ntile = (N + 31) // 32
        work["pool"] = ("hbm", ntile * (2 * U * 4 + 32) + ntile * 2 * U * e)
    else:
        work["token_proj"] = ("mfma", B * T * 2 * U * C)
    return work


def _source_sha(kernel):
    files = {"slot_attention": ["slot.hip", "slot_kernel.hpp"], "prep": ["prep.hip"],
             "post": ["post.hip"], "pool": ["post.hip"], "token_proj": ["prep.hip"],
             "pack": ["pack.hip"], "vt": ["slot.hip"], "masks": ["prep.hip"]}
    h = hashlib.sha256()
    for f in files.get(kernel, []) + ["common.hpp", "kernels.hpp"]:
        p = os.path.join(ROOT, "windowed_atom_attention_amd", "csrc", f)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current source of this kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get("%s@%s" % (kernel, workload))
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != _source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


# Kernel symbols of libatomattn, as they appear in a rocprofv3 trace, and the
# names the library's own profiler gives them.
KERNEL_SYMBOLS = {"k_slot": "slot_attention", "k_prep": "prep", "k_post": "post",
                  "k_pool_fix": "pool", "k_pack": "pack", "k_token_proj": "token_proj",
                  "k_vt": "vt", "k_masks": "masks"}


def kernel_of(symbol):
    """Library kernel name of a trace symbol (demangled or mangled), else None."""
    import re
    m = re.search(r"k_(slot|prep|post|pool_fix|pack|token_proj|vt|masks)(?![a-z_])", symbol)
    return KERNEL_SYMBOLS["k_" + m.group(1)] if m else None


COPY_PROBE_BYTES = 1 << 30


def copy_probe(reps=5):
    """A plain elementwise copy (y = -x, fp32) of COPY_PROBE_BYTES read and
    the same written, the calibration kernel for the HBM byte counters."""
    import torch
    n = COPY_PROBE_BYTES // 4
    x = torch.ones(n, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(reps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe": "neg", "bytes_read": COPY_PROBE_BYTES,
                      "bytes_written": COPY_PROBE_BYTES, "launches": reps}))


def _counter_rows(directory):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", "*counter_collection.csv"),
                              recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit("no counter_collection.csv under %s" % directory)
    return rows


def _per_dispatch(rows, counter, select):
    """Mean over dispatches of `counter` (summed over its dimensions within
    a dispatch) for the rows whose kernel name `select` maps to a key."""
    per = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        key = select(r.get("Kernel_Name", ""))
        if key is None:
            continue
        did = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per.setdefault(key, {}).setdefault(did, 0.0)
        per[key][did] += float(r["Counter_Value"])
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in per.items()}


def traffic_summary(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """profiles/traffic.json entries from four rocprofv3 --pmc runs: FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch) over a bench run of `workload` and over
    the copy probe. Each counter is scaled by known bytes / what it reads for
    the copy probe."""
    neg = lambda name: "neg" if "neg" in name else None
    cf, _ = _per_dispatch(_counter_rows(copy_fetch_dir), "FETCH_SIZE", neg)["neg"]
    cw, _ = _per_dispatch(_counter_rows(copy_write_dir), "WRITE_SIZE", neg)["neg"]
    f_read = COPY_PROBE_BYTES / (cf * 1024.0)
    f_write = COPY_PROBE_BYTES / (cw * 1024.0)
    fetch = _per_dispatch(_counter_rows(fetch_dir), "FETCH_SIZE", kernel_of)
    write = _per_dispatch(_counter_rows(write_dir), "WRITE_SIZE", kernel_of)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    db = json.load(open(path)) if os.path.exists(path) else {}
    for k in sorted(set(fetch) & set(write)):
        rd = fetch[k][0] * 1024.0 * f_read
        wr = write[k][0] * 1024.0 * f_write
        db["%s@%s" % (k, workload)] = {
            "bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
            "fetch_kib_raw": fetch[k][0], "write_kib_raw": write[k][0],
            "dispatches": [fetch[k][1], write[k][1]],
            "copy_scale": {"fetch": f_read, "write": f_write},
            "source_sha": _source_sha(k)}
    with open(path, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
    print(json.dumps({k: v["bytes_per_launch"] for k, v in db.items()}))


def cpu_baseline(name, seconds=12.0):
    """The fp64 oracle, as it stands, on the host cores: repeated whole-block
    runs of the same workload (sampled atoms for workloads too large to run
    whole within the budget)."""
    import numpy as np
    import torch
    import oracle
    from windowed_atom_attention_amd.workloads import make_workload

    w = make_workload(name)
    d = w.dims
    entries_per_atom = d["H"] * d["K"]
    nthreads = oracle.threads(0)
    # one probe run on a bounded sample decides how much fits the budget
    sel = None
    if d["B"] * d["A"] > 8192:
        g = np.random.default_rng(0)
        sel = np.zeros((d["B"], d["A"]), bool)
        for b in range(d["B"]):
            start = int(g.integers(0, d["A"] - 1024))
            sel[b, start:start + 1024] = True
        sel = torch.from_numpy(sel)
    t0 = time.perf_counter()
    r = oracle.block(**w.kwargs(), select=sel)
    dt = time.perf_counter() - t0
    atoms = int(r["done_atom"].sum()) if sel is not None else d["B"] * d["A"]
    reps = max(1, min(50, int(seconds / max(dt, 1e-3))))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.block(**w.kwargs(), select=sel)
    dt = (time.perf_counter() - t0) / reps
    sample = ("%d whole-block run(s) of workload %s" % (reps, name) if sel is None else
              "%d run(s) of workload %s restricted to %d atoms (1024 consecutive query "
              "atoms per batch, their keys and tokens)" % (reps, name, atoms))
    return {"value": atoms * entries_per_atom / dt, "unit": "entries/s",
            "cores": nthreads, "kind": "oracle", "sample": sample,
            "atoms_per_s": atoms / dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="1",
                    help="workload: 0, 1, 2, 3, 4a, 4b (default 1)")
    ap.add_argument("--cache-bytes", type=float, default=768e6,
                    help="input copies are added until they exceed this")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of HIP graphs that capture one step each")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only the counter-calibration copy kernel")
    ap.add_argument("--traffic-summary", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/traffic.json entries for --config from "
                         "rocprofv3 --pmc output directories (no GPU work)")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args.config, *args.traffic_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return

    import torch
    from windowed_atom_attention_amd import (pair_bias_split, profile_enable, profile_read,
                                             windowed_atom_attention, workspace_bytes)
    from windowed_atom_attention_amd.workloads import make_workload

    dev = torch.device("cuda:0")
    w = make_workload(args.config)
    d = w.dims
    g = w.to(dev)
    in_bytes = sum(t.numel() * t.element_size() for grp in
                   (g.activations, g.masks, g.structure) for t in grp.values())
    copies = max(1, math.ceil(args.cache_bytes / max(in_bytes, 1)))
    sets = [g]
    for _ in range(copies - 1):
        sets.append(dataclasses.replace(
            g, activations={k: v.clone() for k, v in g.activations.items()},
            masks={k: v.clone() for k, v in g.masks.items()},
            structure={k: v.clone() for k, v in g.structure.items()}))
    ws = torch.empty(workspace_bytes(d, w.style, w.stage, w.dtype), dtype=torch.uint8, device=dev)
    out = None

    def eager(i):
        nonlocal out
        s = sets[i % len(sets)]
        out = windowed_atom_attention(**s.kwargs(), workspace=ws, out=out)

    graphs = []

    def step(i, instrumented=False):
        if graphs and not instrumented:
            graphs[i % len(graphs)].replay()
        else:
            eager(i)

    def timed(instrumented):
        if instrumented:
            profile_enable(True)
            profile_read()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, instrumented)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        kt = profile_read() if instrumented else None
        profile_enable(False)
        return t1 - t0, kt

    for i in range(args.warmup):
        eager(i)
    if args.graph:
        # one captured step per input copy (the library makes no allocation,
        # host synchronisation or memset inside a call)
        torch.cuda.synchronize()
        for s in sets:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                windowed_atom_attention(**s.kwargs(), workspace=ws, out=out)
            graphs.append(gr)
        for i in range(len(graphs)):
            step(i)
    # the throughput comes from an uninstrumented timed region; the kernel
    # durations from HIP events around every launch in a second timed region
    # of the same steps (the events add a little time between kernels)
    elapsed, _ = timed(False)
    elapsed_ev, kt = timed(True)
    ms_step = elapsed * 1e3 / args.steps
    entries = w.entries
    value = entries * args.steps / elapsed
    dtype = "bf16" if w.dtype == torch.bfloat16 else "f32"
    work = kernel_work(w, pair_bias_split(w.dims, w.style, w.stage, w.dtype))
    per_kernel = {k: {"avg_us": 1e3 * ms / n, "launches": n} for k, (ms, n) in kt.items()}
    dom = max((k for k in per_kernel if k in work), key=lambda k: per_kernel[k]["avg_us"])
    bound, amount = work[dom]
    avg_s = per_kernel[dom]["avg_us"] * 1e-6
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": amount / avg_s / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": amount / avg_s / 1e12,
                "peak": MFMA_PEAK_TFLOPS[dtype], "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = _traffic(dom, args.config)
    roof["kernel"] = dom
    roof["work_per_launch"] = amount
    for k, v in per_kernel.items():
        if k in work:
            b, a = work[k]
            if b == "hbm":
                v["GB_per_s"] = a / (v["avg_us"] * 1e-6) / 1e9
                v["frac_hbm"] = v["GB_per_s"] / HBM_PEAK_GBS
            else:
                v["TFLOP_per_s"] = a / (v["avg_us"] * 1e-6) / 1e12
                v["frac_mfma"] = v["TFLOP_per_s"] / MFMA_PEAK_TFLOPS[dtype]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.config)

    names = {"0": "tiny AF3 encoder fp32", "1": "AF3 encoder fp32",
             "2": "ESMFold2 encoder bf16 radius 48", "3": "AF3 decoder bf16",
             "4a": "large mixed AF3 encoder bf16", "4b": "large mixed ESMFold2 encoder bf16 radius 64"}
    line = {
        "metric": "atom-slot attention entries/sec (B*A*H*K) per block, 1xMI355X",
        "value": value, "unit": "entries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step,
        "ms_per_step_instrumented": elapsed_ev * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": "%s (config %s): B=%d A=%d T=%d K=%d C=%d S=%d H=%d D=%d "
                               "V=%d M=%d U=%d, %s, radius %d" % (
                                   names[args.config], args.config, d["B"], d["A"], d["T"],
                                   d["K"], d["C"], d["S"], d["H"], d["D"], d["V"], d["M"],
                                   d["U"], w.stage, w.radius),
                   "style": w.style, "stage": w.stage, "entries_per_step": entries,
                   "atoms_per_step": w.atoms, "input_copies": copies},
        "atoms_per_s": w.atoms * args.steps / elapsed,
        "kernels": per_kernel,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
