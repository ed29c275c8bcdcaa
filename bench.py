"""Benchmark of the windowed atom-attention block on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1]

A step is one call of the whole block ([token projection], prep, slot
attention, post, [pool]) on one batch of synthetic input of the named
workload; the weight matrices are packed into the matrix cores' operand
order once, before the timed region, as a caller that keeps one parameter
set would (--pack-per-call adds the packing kernel to every step). Inputs are resident in HBM before the timed region; to keep the
256 MB Infinity Cache from serving them, the step cycles through enough
copies of the inputs that they do not fit in it. The timed region is exactly
K steps between two device synchronisations and gives the throughput. A
second timed region of the same K steps runs with the library's profiling
mode on: HIP events recorded around each launch on the stream it launches
on give every kernel's average duration (the roofline figures).

Prints ONE JSON line: metric entries/s (B*A*H*K per second) of the
headline workload (--config, default config 1, the AF3 encoder in fp32),
plus atoms/s, every kernel's duration and roofline fraction, the roofline of
the dominant kernel, the fp64 oracle's rate on the host cores (all threads
and one thread, with the CPU model), and under "configs" the same figures
for the other full-size workloads (--also, default 2, 3, 4a, 4b) timed in
the same run, and under "ops" the per-kernel durations and roofline
fractions of the other operators (single-to-pair features, tied pair row
attention, the device window table).
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


def wide_block_fraction(w):
    """Fraction of 16-query blocks whose allowed key ids span more than eight
    128-row chunks (from the 8-aligned band start), i.e. the blocks the slot
    kernel hands to the gather kernel."""
    import torch
    ki = w.structure["key_index"]
    B, A, K = ki.shape
    T = w.masks["token_valid"].shape[-1]
    a2t = w.structure["atom_to_token"]
    usable = w.masks["valid"] & (a2t >= 0) & (a2t < T) & torch.gather(
        w.masks["token_valid"], 1, a2t.clamp(0, T - 1))
    jc = ki.clamp(0, A - 1)
    uk = torch.gather(usable, 1, jc.reshape(B, A * K)).reshape(B, A, K)
    ok = usable[..., None] & (ki >= 0) & (ki < A) & uk & w.masks["window_mask"]
    if w.radius >= 0:
        ok &= (jc - torch.arange(A)[None, :, None]).abs() <= w.radius
    nqb = (A + 15) // 16
    pad = nqb * 16 - A
    big = torch.iinfo(torch.int64).max
    lo = torch.where(ok, ki, torch.full_like(ki, big)).amin(-1)
    hi = torch.where(ok, ki, torch.full_like(ki, -1)).amax(-1)
    lo = torch.nn.functional.pad(lo, (0, pad), value=big).reshape(B, nqb, 16).amin(-1)
    hi = torch.nn.functional.pad(hi, (0, pad), value=-1).reshape(B, nqb, 16).amax(-1)
    has = hi >= 0
    span = hi + 1 - (lo.clamp(max=A) & ~7)
    nch = (span + 127) // 128
    return float(((nch > 8) & has).sum()) / float(B * nqb)


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
    # query blocks of 16 whose key band exceeds eight 128-row chunks take the
    # gather kernel, where every slot reads its key's K row (fp32) and V row
    wide = wide_block_fraction(w)
    gather_bytes = (N * HD * 4 + E * HD * (4 + e) + 8 * E + E + N + pair
                    + E * H * e + N * HD * e)
    work = {"slot_attention": ("hbm", slot_bytes * (1.0 - wide)), "prep": ("mfma", prep),
            "post": ("mfma", post)}
    if wide > 0:
        work["slot_gather"] = ("hbm", gather_bytes * wide)
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
             "pack": ["pack.hip"], "vt": ["slot.hip"], "masks": ["prep.hip"],
             "slot_gather": ["slot_gather.hip"]}
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
                  "k_vt": "vt", "k_masks": "masks", "k_slot_gather": "slot_gather"}


def kernel_of(symbol):
    """Library kernel name of a trace symbol (demangled or mangled), else None."""
    import re
    m = re.search(r"k_(slot_gather|slot|prep|post|pool_fix|pack|token_proj|vt|masks)(?![a-z_])",
                  symbol)
    return KERNEL_SYMBOLS["k_" + m.group(1)] if m else None


COPY_PROBE_BYTES = 1 << 30


def measured_peaks(reps=10):
    """Achievable ceilings on this GPU, beside the spec peaks: HBM from a
    1 GiB device-to-device copy (bytes read + written per second), the
    matrix cores from large square fp32 and bf16 products (torch.matmul,
    TF32 off; 2 n^3 flops each). The rooflines report their fraction of
    these as the secondary figure (the spec peak stays primary)."""
    import torch
    torch.backends.cuda.matmul.allow_tf32 = False
    dev = torch.device("cuda:0")

    def tavg(fn):
        for _ in range(3):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e-3 / reps

    n = 1 << 28  # fp32 elements: 1 GiB
    src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    t = tavg(lambda: dst.copy_(src))
    out = {"hbm_copy_GBps": 2.0 * 4 * n / t / 1e9, "copy_bytes": 4 * n}
    del src, dst
    for name, dt, m in (("fp32", torch.float32, 8192), ("bf16", torch.bfloat16, 8192)):
        a = torch.randn((m, m), device=dev).to(dt)
        b = torch.randn((m, m), device=dev).to(dt)
        t = tavg(lambda: torch.matmul(a, b))
        out["%s_matmul_TFLOPs" % name] = 2.0 * m ** 3 / t / 1e12
        del a, b
    out["matmul_n"] = 8192
    torch.cuda.empty_cache()
    return out


def _with_measured(roof, peaks, dtype):
    """Add the fraction of the measured ceiling to a roofline record."""
    if not peaks or not roof:
        return roof
    if roof["bound"] == "hbm":
        ref = peaks["hbm_copy_GBps"]
    else:
        ref = peaks["fp32_matmul_TFLOPs" if dtype == "f32" else "bf16_matmul_TFLOPs"]
    roof = dict(roof)
    roof["peak_measured"] = ref
    roof["frac_measured"] = roof["achieved"] / ref
    return roof


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


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(name, seconds=12.0, seconds_1t=4.0):
    """The fp64 oracle, as it stands, on the host cores: repeated whole-block
    runs of the same workload (sampled atoms for workloads too large to run
    whole within the budget), with every host thread the oracle uses and
    then with one thread on a smaller sample."""
    import numpy as np
    import torch
    import oracle
    from windowed_atom_attention_amd.workloads import make_workload

    w = make_workload(name)
    d = w.dims
    entries_per_atom = d["H"] * d["K"]
    nthreads = oracle.threads(0)

    def sample(n_per_batch):
        if d["B"] * d["A"] <= n_per_batch:
            return None
        g = np.random.default_rng(0)
        sel = np.zeros((d["B"], d["A"]), bool)
        n = min(n_per_batch, d["A"])
        for b in range(d["B"]):
            start = int(g.integers(0, d["A"] - n + 1))
            sel[b, start:start + n] = True
        return torch.from_numpy(sel)

    def rate(sel, nt, budget):
        # one probe run decides how many repetitions fit the budget
        t0 = time.perf_counter()
        r = oracle.block(**w.kwargs(), select=sel, nthreads=nt)
        dt = time.perf_counter() - t0
        atoms = int(r["done_atom"].sum()) if sel is not None else d["B"] * d["A"]
        reps = max(1, min(50, int(budget / max(dt, 1e-3))))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.block(**w.kwargs(), select=sel, nthreads=nt)
        dt = (time.perf_counter() - t0) / reps
        return atoms, reps, dt

    sel = sample(1024) if d["B"] * d["A"] > 8192 else None
    atoms, reps, dt = rate(sel, 0, seconds)
    desc = ("%d whole-block run(s) of workload %s" % (reps, name) if sel is None else
            "%d run(s) of workload %s restricted to %d atoms (1024 consecutive query "
            "atoms per batch, their keys and tokens)" % (reps, name, atoms))
    sel1 = sample(256)
    atoms1, reps1, dt1 = rate(sel1, 1, seconds_1t)
    return {"value": atoms * entries_per_atom / dt, "unit": "entries/s",
            "cores": nthreads, "kind": "oracle", "sample": desc,
            "atoms_per_s": atoms / dt, "cpu_model": _cpu_model(),
            "host_cpus": os.cpu_count(),
            "one_thread": {"value": atoms1 * entries_per_atom / dt1, "unit": "entries/s",
                           "cores": 1, "atoms_per_s": atoms1 / dt1,
                           "sample": "%d run(s) of workload %s restricted to %d atoms "
                                     "(256 consecutive query atoms per batch, their keys "
                                     "and tokens)" % (reps1, name, atoms1)}}


NAMES = {"0": "tiny AF3 encoder fp32", "1": "AF3 encoder fp32",
         "2": "ESMFold2 encoder bf16 radius 48", "3": "AF3 decoder bf16",
         "4a": "large mixed AF3 encoder bf16",
         "4b": "large mixed ESMFold2 encoder bf16 radius 64",
         "1r": "AF3 encoder fp32, scattered key ids",
         "4r": "large AF3 encoder bf16, scattered key ids"}


def measure(config, steps, warmup, cache_bytes, graph=False, pack_per_call=False):
    """Time `steps` block calls of workload `config` on cuda:0 (inputs
    resident in HBM, cycled over enough copies to defeat the Infinity Cache)
    and return throughput, per-kernel durations and the dominant kernel's
    roofline. The weight matrices are packed once before the timed region
    (a parameter set is reused across calls) unless `pack_per_call`."""
    import torch
    from windowed_atom_attention_amd import (pack_params, pair_bias_split, profile_enable,
                                             profile_read, windowed_atom_attention,
                                             workspace_bytes)
    from windowed_atom_attention_amd.workloads import make_workload

    dev = torch.device("cuda:0")
    w = make_workload(config)
    d = w.dims
    g = w.to(dev)
    in_bytes = sum(t.numel() * t.element_size() for grp in
                   (g.activations, g.masks, g.structure) for t in grp.values())
    copies = max(1, math.ceil(cache_bytes / max(in_bytes, 1)))
    sets = [g]
    for _ in range(copies - 1):
        sets.append(dataclasses.replace(
            g, activations={k: v.clone() for k, v in g.activations.items()},
            masks={k: v.clone() for k, v in g.masks.items()},
            structure={k: v.clone() for k, v in g.structure.items()}))
    ws = torch.empty(workspace_bytes(d, w.style, w.stage, w.dtype), dtype=torch.uint8, device=dev)
    out = None
    packed = None if pack_per_call else pack_params(g.parameters, d, w.style, w.stage)

    def eager(i):
        nonlocal out
        s = sets[i % len(sets)]
        out = windowed_atom_attention(**s.kwargs(), workspace=ws, out=out, packed=packed)

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
        for i in range(steps):
            step(i, instrumented)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        kt = profile_read() if instrumented else None
        profile_enable(False)
        return t1 - t0, kt

    for i in range(warmup):
        eager(i)
    if graph:
        # one captured step per input copy (the library makes no allocation,
        # host synchronisation or memset inside a call)
        torch.cuda.synchronize()
        for s in sets:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                windowed_atom_attention(**s.kwargs(), workspace=ws, out=out, packed=packed)
            graphs.append(gr)
        for i in range(len(graphs)):
            step(i)
    # the throughput comes from an uninstrumented timed region; the kernel
    # durations from HIP events around every launch in a second timed region
    # of the same steps (the events add a little time between kernels)
    elapsed, _ = timed(False)
    elapsed_ev, kt = timed(True)
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
    roof["traffic"] = _traffic(dom, config)
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
            v["traffic"] = _traffic(k, config)
    # the slot step's rate on its own kernel time: entries (B*A*H*K) per
    # second of the slot kernel (and of the gather kernel, which takes the
    # blocks of scattered key ids)
    slot_us = sum(per_kernel[k]["avg_us"] for k in ("slot_attention", "slot_gather")
                  if k in per_kernel)
    if slot_us > 0:
        per_kernel["slot_attention"]["entries_per_s_slot_step"] = w.entries / (slot_us * 1e-6)
    res = {
        "workload": "%s (config %s): B=%d A=%d T=%d K=%d C=%d S=%d H=%d D=%d V=%d M=%d "
                    "U=%d, %s, radius %d" % (NAMES[config], config, d["B"], d["A"], d["T"],
                                            d["K"], d["C"], d["S"], d["H"], d["D"], d["V"],
                                            d["M"], d["U"], w.stage, w.radius),
        "style": w.style, "stage": w.stage, "dtype": dtype,
        "entries_per_step": w.entries, "atoms_per_step": w.atoms, "input_copies": copies,
        "weights": "packed per call" if pack_per_call else "packed once before timing",
        "steps": steps, "ms_per_step": elapsed * 1e3 / steps,
        "ms_per_step_instrumented": elapsed_ev * 1e3 / steps,
        "entries_per_s": w.entries * steps / elapsed,
        "atoms_per_s": w.atoms * steps / elapsed,
        "kernels": per_kernel, "roofline": roof,
    }
    del sets, ws, out, graphs, g, packed
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def _time_op(call, nbuf, steps, warmup):
    """Average wall time per call (uninstrumented, between device
    synchronisations) and per-kernel HIP-event durations of `call(i)`,
    cycling over `nbuf` output buffers."""
    import torch
    from windowed_atom_attention_amd import profile_enable, profile_read
    for i in range(warmup):
        call(i % nbuf)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(i % nbuf)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    profile_enable(True)
    profile_read()
    for i in range(steps):
        call(i % nbuf)
    torch.cuda.synchronize()
    kt = profile_read()
    profile_enable(False)
    return wall, {k: {"avg_us": 1e3 * ms / n, "launches": n} for k, (ms, n) in kt.items()}


def _roof(v, bound, amount, dtype):
    sec = v["avg_us"] * 1e-6
    if bound == "hbm":
        v["GB_per_s"] = amount / sec / 1e9
        v["frac_hbm"] = v["GB_per_s"] / HBM_PEAK_GBS
    else:
        v["TFLOP_per_s"] = amount / sec / 1e12
        v["frac_mfma"] = v["TFLOP_per_s"] / MFMA_PEAK_TFLOPS[dtype]
    v["work_per_launch"] = amount


def measure_ops(steps=50, warmup=5, cache_bytes=768e6):
    """The other operators at their benchmark sizes: single-to-pair features
    (ESMFold-like trunk: B=1, N=512, C=1024, H=64, D=128, bf16) and the
    device window table (the decoder workload's [4,12288,128], int64 and
    int32). Outputs cycle over enough buffers to exceed the Infinity Cache."""
    import torch
    from windowed_atom_attention_amd import single_to_pair, window_table
    from windowed_atom_attention_amd.workloads import make_s2p_workload

    res = {}
    acts, par, masks, on = make_s2p_workload()
    B, Ntok, C = acts["x"].shape
    H2, D = par["weight"].shape[-1], par["out_weight"].shape[-1]
    cu = lambda d: {k: v.cuda() for k, v in d.items()}
    a, p_, m = cu(acts), cu(par), cu(masks)
    e = 2
    per = B * Ntok * Ntok * (H2 + D) * e
    nbuf = max(2, math.ceil(cache_bytes / per))
    outs = [(torch.empty((B, Ntok, Ntok, H2), dtype=torch.bfloat16, device="cuda"),
             torch.empty((B, Ntok, Ntok, D), dtype=torch.bfloat16, device="cuda"))
            for _ in range(nbuf)]
    wall, kt = _time_op(lambda i: single_to_pair(a, p_, m, output_norm=on, out=outs[i]),
                        nbuf, steps, warmup)
    # algorithmic bytes: the two output tensors written once, the q|k rows
    # (fp32) read once, the mask; the token kernel: x, its weight and q|k
    pair_bytes = per + B * Ntok * H2 * 4 + B * Ntok
    tok_bytes = B * Ntok * C * e + C * H2 * e + B * Ntok * H2 * 4 + B * Ntok
    _roof(kt["s2p_pair"], "hbm", pair_bytes, "bf16")
    _roof(kt["s2p_token"], "hbm", tok_bytes, "bf16")
    kt["s2p_pair"]["flops_per_launch"] = B * Ntok * Ntok * H2 * D * 2
    res["single_to_pair"] = {
        "workload": "B=%d N=%d C=%d H=%d D=%d bf16, output_norm %s, %d%% absent tokens" % (
            B, Ntok, C, H2 // 2, D, on, 5),
        "ms_per_call": wall * 1e3, "pairs_per_s": B * Ntok * Ntok / wall,
        "kernels": kt, "output_buffers": nbuf}
    del outs
    from windowed_atom_attention_amd import tied_row_attention, tied_workspace_bytes
    from windowed_atom_attention_amd.workloads import make_tied_workload
    acts, par = make_tied_workload()
    B, L, _, C = acts["features"].shape
    CB, H = acts["bias_features"].shape[-1], par["w_bias"].shape[-1]
    HD = par["w_q"].shape[-1]
    a, p_ = cu(acts), cu(par)
    ws = torch.empty(tied_workspace_bytes(B, L, C, CB, H, HD // H, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    per = B * L * L * C * 2
    nbuf = max(2, math.ceil(cache_bytes / per))
    outs = [torch.empty((B, L, L, C), dtype=torch.bfloat16, device="cuda") for _ in range(nbuf)]
    wall, kt = _time_op(lambda i: tied_row_attention(a, p_, out=outs[i], workspace=ws), nbuf,
                        steps, warmup)
    # algorithmic work per kernel: flops of its matrix products (the bf16
    # path forms some of them from hi + lo pairs; counted once here)
    LL = B * L * L
    flops = {"tied_proj": LL * 2 * C * 4 * HD, "tied_logits": B * H * L * L * L * (HD // H) * 2,
             "tied_out": B * H * L * L * L * (HD // H) * 2 + LL * 2 * HD * C}
    for k, f in flops.items():
        _roof(kt[k], "mfma", f, "bf16")
    _roof(kt["tied_softmax"], "hbm", B * H * L * L * (4 + 4 + 2), "bf16")
    if "tied_bias" in kt:   # beta is formed inside k_tied_proj for most Cb
        _roof(kt["tied_bias"], "hbm", LL * CB * 2 + B * H * L * L * 4, "bf16")
    res["tied_row_attention"] = {
        "workload": "B=%d L=%d C=%d CB=%d H=%d D=%d bf16" % (B, L, C, CB, H, HD // H),
        "ms_per_call": wall * 1e3, "pair_entries_per_s": LL / wall, "kernels": kt,
        "flops_per_call": sum(flops.values())}
    del outs, ws
    Bw, Aw, Kw = 4, 12288, 128
    for dt, esz in ((torch.int64, 8), (torch.int32, 4)):
        nb = max(2, math.ceil(cache_bytes / (Bw * Aw * Kw * esz)))
        bufs = [torch.empty((Bw, Aw, Kw), dtype=dt, device="cuda") for _ in range(nb)]
        wall, kt = _time_op(lambda i: window_table(Bw, Aw, Kw, dtype=dt, out=bufs[i]), nb,
                            steps, warmup)
        _roof(kt["window"], "hbm", Bw * Aw * Kw * esz, "bf16")
        res["window_table_%s" % ("int64" if esz == 8 else "int32")] = {
            "workload": "B=%d A=%d K=%d, blocks of 32 queries" % (Bw, Aw, Kw),
            "ms_per_call": wall * 1e3, "ids_per_s": Bw * Aw * Kw / wall, "kernels": kt}
        del bufs
    torch.cuda.empty_cache()
    return res


def _dense_flops(d, style, stage):
    """Flops of the block's dense products for one call (forward)."""
    N = d["B"] * d["A"]
    C, S, HD, M, U = d["C"], d["S"], d["H"] * d["D"], d["M"], d["U"]
    per = 2 * C * HD * 4 + 2 * HD * C + 2 * C * M * 2 + 2 * M * C
    per += 2 * S * C * 8 if style == "af3" else 2 * S * 6 * C
    per += 2 * C * U if stage == "encoder" else 2 * C * 3
    tok = 2 * d["B"] * d["T"] * U * C if stage == "decoder" else 0
    return N * per + tok


def measure_backward(names=("1", "4a"), steps=20, warmup=3):
    """The backward pass (atom_attn_backward) on whole workloads: wall time per
    call with every upstream gradient given, and the per-phase HIP-event
    spans with their rooflines: the forward recomputation and the chain
    rule's dense products against the fp32 matrix-core peak (they run in
    fp32 whatever the storage), the slot-step kernels against HBM."""
    import torch
    from windowed_atom_attention_amd import backward_workspace_bytes, block_backward
    from windowed_atom_attention_amd.workloads import make_workload
    res = {}
    for name in names:
        w = make_workload(name).to("cuda")
        d = w.dims
        B, A, T, K, C, H, D, U, V = (d[k] for k in "B A T K C H D U V".split())
        g = torch.Generator(device="cuda").manual_seed(0)
        up = {"hidden": torch.randn((B, A, C), generator=g, device="cuda"),
              "attention": torch.randn((B, H, A, K), generator=g, device="cuda")}
        if w.stage == "encoder":
            up["token_output"] = torch.randn((B, T, U), generator=g, device="cuda")
        else:
            up["position_update"] = torch.randn((B, A, 3), generator=g, device="cuda")
        ws = torch.empty(backward_workspace_bytes(d, w.style, w.stage, w.dtype),
                         dtype=torch.uint8, device="cuda")
        call = lambda i: block_backward(w.activations, w.parameters, w.masks, w.structure, up,
                                        eps=w.eps, style=w.style, stage=w.stage,
                                        radius=w.radius, workspace=ws)
        wall, kt = _time_op(call, 1, steps, warmup)
        N, E, HD = B * A, B * A * K, H * D
        e = 2 if w.dtype == torch.bfloat16 else 4
        pair = E * V * e if w.style == "af3" else 0
        dpair = E * V * 4 if w.style == "af3" else 0
        f32 = 4
        work = {
            # Q, K, V rows, key ids, window mask, usable, pair rows; weights,
            # o, slot -> key map written
            "bwd_slot_fwd": ("hbm", 3 * N * HD * f32 + 9 * E + N + pair + E * H * f32 +
                             N * HD * f32 + 4 * E),
            # weights, upstream weights, d_o, K and V rows, slot -> key map,
            # pair rows read; logit gradients, dq, d_pair written
            "bwd_slot_q": ("hbm", 2 * E * H * f32 + 3 * N * HD * f32 + 4 * E + pair +
                           E * H * f32 + N * HD * f32 + dpair),
            # reverse index (map read twice, list written and read), weights
            # and logit gradients, Q and d_o rows read; dk, dv written
            "bwd_slot_kv": ("hbm", 16 * E + 2 * E * H * f32 + 4 * N * HD * f32),
            "bwd_recompute": ("mfma", _dense_flops(d, w.style, w.stage)),
            "bwd_chain": ("mfma", 2 * _dense_flops(d, w.style, w.stage)),
        }
        for k, (bound, amount) in work.items():
            if k in kt:
                _roof(kt[k], bound, amount, "f32")
        res[name] = {"workload": "%s (config %s), B=%d A=%d K=%d, every upstream gradient"
                                 % (NAMES[name], name, B, A, K),
                     "storage_dtype": str(w.dtype).replace("torch.", ""), "compute_dtype": "f32",
                     "ms_per_call": wall * 1e3, "atoms_per_s": N / wall,
                     "entries_per_s": N * H * K / wall, "kernels": kt, "steps": steps,
                     "workspace_bytes": ws.numel()}
        print("bench: backward %s %.3f ms/call" % (name, wall * 1e3), file=sys.stderr,
              flush=True)
        del ws, w, up
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="1",
                    help="workload of the headline line: 0, 1, 2, 3, 4a, 4b (default 1)")
    ap.add_argument("--also", default="2,3,4a,4b,1r,4r",
                    help="further workloads timed in the same run and reported under "
                         "'configs' (comma separated; empty for none)")
    ap.add_argument("--also-steps", type=int, default=50)
    ap.add_argument("--no-ops", action="store_true",
                    help="skip the other operators (single-to-pair, tied attention, window table)")
    ap.add_argument("--only-ops", action="store_true",
                    help="time only the other operators (for profiler runs); prints their record")
    ap.add_argument("--backward", default="1,4a",
                    help="workloads whose backward pass is timed and reported under "
                         "'backward' (comma separated; empty for none)")
    ap.add_argument("--only-backward", action="store_true",
                    help="time only the backward pass of --backward (for profiler runs)")
    ap.add_argument("--cache-bytes", type=float, default=768e6,
                    help="input copies are added until they exceed this")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU baseline and the measured ceilings (profiler runs)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured ceilings (copy and matrix-product microbenchmarks)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of HIP graphs that capture one step each")
    ap.add_argument("--pack-per-call", action="store_true",
                    help="pack the weight matrices inside every call (default: once, "
                         "before the timed region)")
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

    if args.only_ops:
        print(json.dumps({"ops": measure_ops(args.steps, args.warmup)}))
        return
    bwd_names = [x for x in args.backward.split(",") if x]
    if args.only_backward:
        print(json.dumps({"backward": measure_backward(bwd_names, args.steps, args.warmup)}))
        return
    head = measure(args.config, args.steps, args.warmup, args.cache_bytes, args.graph,
                   args.pack_per_call)
    print("bench: config %s %.4f ms/step" % (args.config, head["ms_per_step"]),
          file=sys.stderr, flush=True)
    others = {}
    for c in [x for x in args.also.split(",") if x and x != args.config]:
        r = measure(c, args.also_steps, min(args.warmup, 5), args.cache_bytes, args.graph,
                    args.pack_per_call)
        others[c] = {k: r[k] for k in ("workload", "dtype", "ms_per_step", "entries_per_s",
                                       "atoms_per_s", "kernels", "roofline", "steps")}
        print("bench: config %s %.4f ms/step" % (c, r["ms_per_step"]), file=sys.stderr,
              flush=True)

    ops = None if args.no_ops else measure_ops(args.also_steps)
    bwd = measure_backward(bwd_names, 20, 3) if bwd_names else None

    peaks = None if (args.no_peaks or args.no_cpu_baseline) else measured_peaks()
    if peaks:
        head["roofline"] = _with_measured(head["roofline"], peaks, head["dtype"])
        for r in others.values():
            r["roofline"] = _with_measured(r["roofline"], peaks, r["dtype"])
        print("bench: measured ceilings %s" % json.dumps({k: round(v, 1) for k, v in peaks.items()}),
              file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.config)

    line = {
        "metric": "atom-slot attention entries/sec (B*A*H*K) per block, 1xMI355X",
        "value": head["entries_per_s"], "unit": "entries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "ms_per_step_instrumented": head["ms_per_step_instrumented"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"], "data": "synthetic",
        "config": {"workload": head["workload"], "style": head["style"],
                   "stage": head["stage"], "weights": head["weights"],
                   "entries_per_step": head["entries_per_step"],
                   "atoms_per_step": head["atoms_per_step"],
                   "input_copies": head["input_copies"]},
        "atoms_per_s": head["atoms_per_s"],
        "kernels": head["kernels"],
        "roofline": head["roofline"],
        "peaks_measured": peaks,
        "cpu_baseline": cpu,
        "configs": others,
        "ops": ops,
        "backward": bwd,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
