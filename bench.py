#!/usr/bin/env python3
"""Benchmark of the multi-LoRA hot path on one MI355X.

One step = one pass of the whole path over one batch: lora_build_segments,
lora_shrink, and lora_expand / lora_expand_slice for every output of the
workload.  Inputs live in HBM before timing starts.  Following the kernel
micro-benchmark PR's method, a pool of distinct argument sets (>= 1 GiB, four
times the 256 MB Infinity Cache) is cycled so that no step finds its data in
cache, and the K timed steps are captured in one HIP graph (launch overhead
of the Python binding stays out of the measurement) and replayed once between
two events.

Output: one JSON line on stdout.  value = algorithmic shrink + expand bytes of
a step / step time (GB/s).  roofline = the dominant kernel, timed alone (a
graph of K launches of that op over the pool, events on its stream) against
the 8 TB/s HBM peak.  cpu_baseline = the fp64 oracle on the host cores on the
same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config k]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "shrink+expand achieved HBM GB/s (BGMV) / MFMA TFLOP/s (SGMV), % roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _set_layout(w):
    """(key, element bytes, shape) of every device tensor of one argument set,
    in allocation order."""
    items = [("ids", 4, (w.T,)), ("x", 2, (w.T, w.H)), ("A", 2, (w.L, w.r, w.H))]
    for oi, o in enumerate(w.outputs):
        for si, q in enumerate(o.slices):
            items.append((f"B{oi}.{si}", 2, (w.L, q.n, w.r)))
    for oi, o in enumerate(w.outputs):
        items.append((f"y{oi}", 2, (w.T, o.ldy)))
    items.append(("v", 4, (w.T, w.r)))
    # segment metadata: built once on set 0, then copied with everything else
    items += [("meta.st", 4, (max(w.T, 1),)), ("meta.sl", 4, (w.L,)), ("meta.ss", 4, (w.L + 1,)),
              ("meta.cn", 4, (4,))]
    return items


def _host_bits(w, key):
    import numpy as np
    if key == "ids":
        return np.ascontiguousarray(w.ids, np.int32)
    if key == "x":
        return w.x
    if key == "A":
        return w.A
    if key == "v":
        return np.zeros((w.T, w.r), np.float32)
    if key.startswith("meta."):
        return None
    if key[0] == "B":
        oi, si = map(int, key[1:].split("."))
        return w.outputs[oi].slices[si].B
    return w.outputs[int(key[1:])].y0


class ArgSet:
    """One step's device buffers: views into a pool allocation."""

    def __init__(self, w, torch, lsb, flat, base, layout, offs):
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        t = {}
        for (key, eb, shape), off in zip(layout, offs):
            n = math.prod(shape)
            view = flat[base + off: base + off + n * eb]
            dt = torch.int32 if (key == "ids" or key.startswith("meta.")) else (
                torch.float32 if key == "v" else tdt)
            t[key] = view.view(dt).view(shape)
        self.ids, self.x, self.A, self.v = t["ids"], t["x"], t["A"], t["v"]
        self.Bs = [[t[f"B{oi}.{si}"] for si in range(len(o.slices))] for oi, o in enumerate(w.outputs)]
        self.ys = [t[f"y{oi}"] for oi in range(len(w.outputs))]
        self.seg = lsb.Segments(self.ids, w.L,
                                buffers=(t["meta.st"], t["meta.sl"], t["meta.ss"], t["meta.cn"]))


def set_bytes(w):
    return sum(((math.prod(shape) * eb + 255) // 256) * 256 for _, eb, shape in _set_layout(w))


def make_pool(w, torch, lsb, P):
    """P argument sets of the workload, carved from one device allocation.
    Set 0 is copied from the host tensor by tensor; the others are filled by
    doubling copies of the sets already filled, so the pool costs about
    log2(P) + a few copy dispatches whatever its size (thousands of small
    per-tensor copies under a counter profiler are avoided)."""
    import numpy as np
    layout = _set_layout(w)
    offs, off = [], 0
    for _, eb, shape in layout:
        offs.append(off)
        off += ((math.prod(shape) * eb + 255) // 256) * 256
    S = max(off, 256)
    flat = torch.empty(P * S, dtype=torch.uint8, device="cuda")
    for (key, eb, shape), o in zip(layout, offs):
        nb = math.prod(shape) * eb
        bits = _host_bits(w, key)
        if nb and bits is not None:
            src = torch.from_numpy(np.ascontiguousarray(bits).reshape(-1).view(np.uint8))
            flat[o:o + nb].copy_(src)
    first = ArgSet(w, torch, lsb, flat, 0, layout, offs)
    # Every set carries valid metadata before anything is timed (a call timed
    # alone, without the build, reads the set's metadata as it stands).
    lsb.lora_build_segments(first.ids, w.L, seg=first.seg)
    k = 1
    while k < P:
        m = min(k, P - k)
        flat[k * S:(k + m) * S].copy_(flat[0:m * S])
        k += m
    return [first] + [ArgSet(w, torch, lsb, flat, i * S, layout, offs) for i in range(1, P)]


def op_build(w, lsb, s, ws):
    lsb.lora_build_segments(s.ids, w.L, seg=s.seg)


def op_shrink(w, lsb, s, ws):
    lsb.lora_shrink(s.x, s.A, s.seg, s.v, workspace=ws)


def op_expand_output(w, lsb, s, oi):
    o = w.outputs[oi]
    if len(o.slices) == 1 and o.slices[0].col_off == 0:
        lsb.lora_expand(s.v, s.Bs[oi][0], s.seg, s.ys[oi], w.add)
    else:
        lsb.lora_expand_slice(s.v, s.Bs[oi], [q.col_off for q in o.slices], s.seg, s.ys[oi], w.add)


def op_expand(w, lsb, s, ws):
    for oi in range(len(w.outputs)):
        op_expand_output(w, lsb, s, oi)


def step(w, lsb, s, ws):
    op_build(w, lsb, s, ws)
    op_shrink(w, lsb, s, ws)
    op_expand(w, lsb, s, ws)


def fused_applies(w):
    """Whether lora_shrink_expand (shrink and expand in one launch) takes the
    workload: one output, r in 8..64 by powers of two, aligned sizes, a
    decode-sized batch."""
    if len(w.outputs) != 1 or w.r not in (8, 16, 32, 64) or w.H % 8 or w.T > 1024:
        return False
    o = w.outputs[0]
    return o.ldy % 8 == 0 and all(q.n % 8 == 0 and q.col_off % 8 == 0 for q in o.slices)


def op_fused(w, lsb, s, ws):
    o = w.outputs[0]
    lsb.lora_shrink_expand(s.x, s.A, s.Bs[0], [q.col_off for q in o.slices], s.seg, s.v, s.ys[0], w.add)


def fused_step(w, lsb, s, ws):
    op_build(w, lsb, s, ws)
    op_fused(w, lsb, s, ws)


_evict = None


def graph_time(torch, fn, sets, first, count, evict=True):
    """Captures `count` calls of fn over consecutive pool sets in one graph,
    replays it once untimed, then once between two events.  Returns ms.

    When `count` sets fit in the 256 MB Infinity Cache, one replay would
    leave them there for the next.  So before each replay the stream sums a
    512 MiB buffer: a read-only sweep that replaces the cache's contents with
    clean lines (nothing to write back later), and the calls find their
    inputs in HBM.  Before the timed replay the sweep also keeps the GPU busy
    while the host queues the replay."""
    global _evict
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(count):
            fn(sets[(first + i) % len(sets)])
    if evict and _evict is None:
        _evict = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
    if evict:
        _evict.sum()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if evict:
        _evict.sum()
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    del g
    return ms


def tol_ratio(got, ref):
    """max |got - ref| / (1e-2 (1 + |ref|)) over all elements; <= 1 passes.
    Any NaN in the errors (a NaN or infinite output where the oracle is
    finite, or the reverse) makes the ratio infinite."""
    import numpy as np
    if got.size == 0:
        return 0.0
    err = np.abs(got - ref) / (1e-2 * (1.0 + np.abs(ref)))
    if np.isnan(err).any():
        return float("inf")
    return float(err.max())


def parity_check(w, torch, lsb, ws, stepfn=step):
    """Checks one fresh step against the oracle before anything is timed:
    metadata bit for bit, every active row of v and of every output in full
    (streamed through the oracle in row blocks, so no fp64 copy of a whole
    output is held), and rows without an adapter untouched."""
    import numpy as np
    import oracle
    import workloads as W
    s = make_pool(w, torch, lsb, 1)[0]
    stepfn(w, lsb, s, ws)
    torch.cuda.synchronize()
    meta = (s.seg.sorted_token[:w.T].cpu().numpy(), s.seg.seg_lora.cpu().numpy(),
            s.seg.seg_start.cpu().numpy(), s.seg.counts.cpu().numpy())
    for g_, r_ in zip(meta, oracle.build_segments(w.ids, w.L)):
        if not np.array_equal(g_, r_):
            return float("inf")
    act = np.nonzero(w.active)[0].astype(np.int32)
    inact = np.nonzero(~w.active)[0]
    v_ref = oracle.shrink(w.dtype, w.x, w.A, w.ids, rows=act)
    vg = s.v.cpu().numpy().astype(np.float64)[act]
    worst = tol_ratio(vg, v_ref)
    v_full = np.zeros((w.T, w.r))
    v_full[act] = v_ref
    for o, y in zip(w.outputs, s.ys):
        cols = np.concatenate([np.arange(q.col_off, q.col_off + q.n) for q in o.slices])
        block = max(1, (32 << 20) // o.ldy)
        for b in range(0, act.size, block):
            rows = act[b:b + block]
            ref = oracle.expand_slice(w.dtype, v_full, [q.B for q in o.slices],
                                      [q.col_off for q in o.slices], w.ids, o.y0, w.add, rows=rows)
            yb = y.index_select(0, torch.from_numpy(rows).long().cuda()).view(torch.int16)
            got = W.bits_to_f32(yb.cpu().numpy().view(np.uint16)[:, cols], w.dtype).astype(np.float64)
            worst = max(worst, tol_ratio(got, ref))
        if inact.size:
            yb = y.index_select(0, torch.from_numpy(inact).long().cuda()).view(torch.int16)
            if not np.array_equal(yb.cpu().numpy().view(np.uint16), o.y0[inact]):
                return float("inf")
    del s
    torch.cuda.empty_cache()
    return worst


def run_oracle_step(w):
    """The whole workload through the oracle: metadata, shrink, every expand."""
    import numpy as np
    import oracle
    oracle.build_segments(w.ids, w.L)
    v = np.nan_to_num(oracle.shrink(w.dtype, w.x, w.A, w.ids))
    for o in w.outputs:
        oracle.expand_slice(w.dtype, v, [q.B for q in o.slices], [q.col_off for q in o.slices],
                            w.ids, o.y0, w.add)


def _time_oracle(w, target_s, max_s):
    t0 = time.perf_counter()
    run_oracle_step(w)
    t1 = time.perf_counter() - t0
    reps = 1 if t1 >= target_s else max(1, min(100000, int(math.ceil(target_s / max(t1, 1e-6)))))
    reps = min(reps, max(1, int(max_s / max(t1, 1e-6))))
    t0 = time.perf_counter()
    for _ in range(reps - 1):
        run_oracle_step(w)
    el = time.perf_counter() - t0 + t1
    return reps, el


def cpu_baseline(w, step_bytes):
    """The fp64 oracle (as it is) on the host cores, over the same workload,
    repeated to about 12 s of CPU work; then, on one thread, the three
    smallest named workloads (about 1.5 s each)."""
    import oracle
    import workloads as W
    reps, el = _time_oracle(w, 12.0, 30.0)
    out = {
        "value": round(step_bytes * reps / el / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"the whole workload (metadata, shrink, expand of every output, every row) run "
                  f"{reps}x in {el:.1f} s, OpenMP over tokens",
        "tokens_per_s": round(w.T * reps / el, 2),
        "host_cpus": os.cpu_count(),
        "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"),
    }
    single = {}
    prev = oracle.set_num_threads(1)
    try:
        for k in (1, 2, 3):
            wk = W.config(k)
            r1, e1 = _time_oracle(wk, 1.5, 5.0)
            b = wk.shrink_bytes() + wk.expand_bytes()
            single[wk.name] = {"GB_s": round(b * r1 / e1 / 1e9, 4),
                               "tokens_per_s": round(wk.T * r1 / e1, 1), "runs": r1,
                               "seconds": round(e1, 2)}
    finally:
        oracle.set_num_threads(prev)
    out["one_thread"] = single
    return out


OP_KERNELS = {  # kernel-name fragments of each op (rocprofv3 names)
    "build": ("build_segments",),
    "shrink": ("shrink",),
    "expand": ("expand",),
}
COPY_PROBE_BYTES = 256 << 20


def op_of(kernel_name):
    for op, frags in OP_KERNELS.items():
        if any(f in kernel_name for f in frags):
            return op
    return None


def short_name(kn):
    return kn.replace("void ", "").replace("lora::(anonymous namespace)::", "").split("(")[0]


def assign_units(rows, n_outputs, with_step=False):
    """Unit of every library dispatch of a --profile run, in dispatch order:
    each step is build, shrink (one or two kernels), then one expand call per
    output (one or two kernels each: the tile launch, and the per-token launch
    when the expand splits a decode + prefill mix), so the expand kernels after
    a build are numbered by output in order.  Returns [(unit, row)], or
    [(unit, step, row)] with with_step; other kernels (the copy probe, torch's
    fills) get unit None.  A build not followed by a shrink (the argument
    pool's one-time metadata) forms no step of its own."""
    out = []
    k = 0
    step = -1
    prev = None
    for r in sorted(rows, key=lambda r: int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0)):
        kn = r["Kernel_Name"]
        op = op_of(kn)
        if op == "build":
            k = 0
            step += 1
            unit = "build"
        elif op == "shrink":
            unit = "shrink"
        elif op == "expand":
            # A per-token launch right after the tile launch of the same call.
            if prev is not None and prev[0].startswith("expand") and "bgmv" in kn and "bgmv" not in prev[1]:
                unit = prev[0]
            else:
                unit = f"expand[{k}]" if n_outputs > 1 else "expand"
                k += 1
        else:
            unit = None
        if unit:
            prev = (unit, kn)
        out.append((unit, step, r) if with_step else (unit, r))
    return out


def steps_of(assigned):
    """Per unit, the number of distinct steps it occurs in."""
    import collections
    seen = collections.defaultdict(set)
    for unit, step, _ in assigned:
        if unit:
            seen[unit].add(step)
    return {u: len(v) for u, v in seen.items()}


def unit_bytes(w, unit):
    if unit == "shrink":
        return w.shrink_bytes()
    if unit == "expand":
        return w.expand_bytes()
    if unit.startswith("expand["):
        return w.output_bytes(w.outputs[int(unit[7:-1])])
    return None


COUNTER_SET = ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_INSTS_MFMA",
               "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def summarize_counters(args, name, out_dir):
    """Per-kernel LDS and matrix-core counters of one --pmc pass (summed over
    dispatches): the share of LDS cycles lost to bank conflicts, and
    matrix-core busy cycles per CU and active GPU cycle (256 CUs)."""
    import csv
    import collections
    tot = collections.defaultdict(lambda: collections.defaultdict(float))
    calls = collections.defaultdict(set)
    for r in csv.DictReader(open(args.counters)):
        kn = r["Kernel_Name"]
        if op_of(kn) is None:
            continue
        short = short_name(kn)
        tot[short][r["Counter_Name"]] += float(r["Counter_Value"])
        calls[short].add(r.get("Dispatch_Id", r.get("Correlation_Id", "")))
    lines = [f"# rocprofv3 LDS and matrix-core counters: {name}", "",
             "command (from the repository root, on one MI355X):",
             f"  rocprofv3 --pmc {' '.join(COUNTER_SET)} -d <dir> -o run --output-format csv -- "
             f"python bench.py --config {args.config} --profile",
             "",
             "Sums over all dispatches of each kernel.  LDS conflict share = SQ_LDS_BANK_CONFLICT / "
             "SQ_LDS_IDX_ACTIVE (cycles).  Matrix-core busy = SQ_VALU_MFMA_BUSY_CYCLES / "
             "(GRBM_GUI_ACTIVE x 256 CUs).", "",
             "| kernel | dispatches | LDS instructions | LDS conflict share | MFMA instructions | "
             "matrix-core busy |", "|---|---|---|---|---|---|"]
    for k in sorted(tot):
        c = tot[k]
        lds_active = c.get("SQ_LDS_IDX_ACTIVE", 0.0)
        conflict = c.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds_active if lds_active else 0.0
        gui = c.get("GRBM_GUI_ACTIVE", 0.0)
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * 256) if gui else 0.0
        lines.append(f"| {k} | {len(calls[k])} | {c.get('SQ_INSTS_LDS', 0.0):.3g} | {100 * conflict:.2f}% | "
                     f"{c.get('SQ_INSTS_MFMA', 0.0):.3g} | {100 * busy:.2f}% |")
    path = os.path.join(out_dir, f"counters_{name}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", path)


def summarize_profiles(args):
    """Turns rocprofv3 CSV output of `bench.py --profile` into the short
    summaries kept under profiles/: a kernel-trace table (per kernel, and per
    call of the step: build, shrink, each expand), and per-call HBM traffic from
    the FETCH_SIZE / WRITE_SIZE runs scaled by a copy of known size."""
    import csv
    import collections
    import statistics
    import workloads as W
    w = W.config(args.config)
    name = w.name
    nout = len(w.outputs)
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    pool = f" --pool-gib {args.pool_gib:g}" if args.pool_gib != 1.0 else ""
    if args.trace:
        lines = [f"# rocprofv3 kernel trace: {name}", "",
                 "command (from the repository root, on one MI355X):",
                 f"  rocprofv3 --kernel-trace --stats -d <dir> -o run --output-format csv -- "
                 f"python bench.py --config {args.config} --profile{pool}",
                 "",
                 "Every launch of the run: the parity step, the warm-up steps and both replays of "
                 "the K-step graph (inputs in HBM for the replays).  Durations are each kernel's "
                 "own (end - start).", "",
                 "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        rows = list(csv.DictReader(open(args.trace)))
        per_kernel = collections.defaultdict(list)
        per_unit = collections.defaultdict(list)
        assigned = assign_units(rows, nout, with_step=True)
        nsteps = steps_of(assigned)
        for unit, _, r in assigned:
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            if unit is None and "copy" not in r["Kernel_Name"].lower():
                continue
            per_kernel[short_name(r["Kernel_Name"])].append(d)
            if unit:
                per_unit[unit].append(d)
        for k in sorted(per_kernel):
            v = per_kernel[k]
            lines.append(f"| {k} | {len(v)} | {statistics.fmean(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
        lines += ["", f"Per call of the step ({nsteps.get('shrink', 0)} steps traced; a call's kernels "
                  "summed; algorithmic bytes of the call; fraction of the 8 TB/s HBM peak):", "",
                  "| call | us per step | algorithmic MiB | GB/s | of 8 TB/s |", "|---|---|---|---|---|"]
        for unit in sorted(per_unit):
            per_step = sum(per_unit[unit]) / max(1, nsteps.get(unit, 1))
            nb = unit_bytes(w, unit)
            if nb:
                gbs = nb / (per_step * 1e-6) / 1e9
                lines.append(f"| {unit} | {per_step:.2f} | {nb / 2**20:.3f} | {gbs:.1f} | "
                             f"{gbs / HBM_PEAK_GBS:.4f} |")
            else:
                lines.append(f"| {unit} | {per_step:.2f} | | | |")
        path = os.path.join(out_dir, f"trace_{name}.md")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print("wrote", path)
    if args.counters:
        summarize_counters(args, name, out_dir)
    if not (args.fetch and args.write):
        return

    def per_unit(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        tot = collections.defaultdict(float)
        copy_vals = []
        assigned = assign_units(rows, nout, with_step=True)
        nsteps = steps_of(assigned)
        for unit, _, r in assigned:
            val = float(r["Counter_Value"])  # KiB per dispatch
            if unit:
                tot[unit] += val
            elif "neg_kernel" in r["Kernel_Name"]:
                copy_vals.append(val)
        return ({k: v / max(1, nsteps.get(k, 1)) for k, v in tot.items()}, copy_vals,
                nsteps.get("shrink", 0))

    fetch, fcopy, steps = per_unit(args.fetch, "FETCH_SIZE")
    write, wcopy, _ = per_unit(args.write, "WRITE_SIZE")
    if not fcopy or not wcopy:
        raise SystemExit("no copy probe dispatch found: run the --pmc passes with --traffic-probe")
    f_fetch = max(fcopy) * 1024 / COPY_PROBE_BYTES
    f_write = max(wcopy) * 1024 / COPY_PROBE_BYTES
    rec = {"workload": name, "steps_profiled": steps,
           "copy_probe_bytes": COPY_PROBE_BYTES,
           "fetch_scale": round(f_fetch, 4), "write_scale": round(f_write, 4),
           "ops": {}}
    for unit in sorted(set(fetch) | set(write)):
        b = fetch.get(unit, 0.0) * 1024 / f_fetch + write.get(unit, 0.0) * 1024 / f_write
        alg = unit_bytes(w, unit)
        fam = "build" if unit == "build" else ("shrink" if unit == "shrink" else "expand")
        rec["ops"][unit] = {"bytes_per_call": int(b), "fetch_kib": round(fetch.get(unit, 0.0), 1),
                            "write_kib": round(write.get(unit, 0.0), 1),
                            "algorithmic_bytes": alg,
                            "ratio": round(b / alg, 3) if alg else None,
                            "source_hash": source_hash(KERNEL_SOURCES[fam])}
    rec["commands"] = [
        f"rocprofv3 --pmc FETCH_SIZE -d <dir> -o run --output-format csv -- python bench.py "
        f"--config {args.config} --profile --traffic-probe{pool}",
        f"rocprofv3 --pmc WRITE_SIZE -d <dir> -o run --output-format csv -- python bench.py "
        f"--config {args.config} --profile --traffic-probe{pool}"]
    path = os.path.join(out_dir, f"traffic_{name}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print("wrote", path)


def golden_shapes():
    """The problem shapes the micro-benchmark PR prints (tests/golden/
    microbench_shapes.txt): its console table's SGMV expand and the review
    thread's bs 8192 x seq 8 example."""
    out = []
    with open(os.path.join(ROOT, "tests", "golden", "microbench_shapes.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                src, bs, sl, m, k, n, L, srt, ns = line.split()
                out.append(dict(source=src, bs=int(bs), sl=int(sl), m=int(m), rank=int(k), n=int(n),
                                num_loras=int(L), sort=bool(int(srt)), num_slices=int(ns)))
    return out


SWEEP_TOKENS = (16, 128, 256, 512, 1024, 2048, 8192)
SWEEP_HIDDEN = (1024, 2048, 4096, 8192, 16384)
SWEEP_RANKS = (8, 16, 32, 64, 128)


def sweep_points(grid="full"):
    """(kind, tokens, hidden, rank, out_cols, adapters, seq_len, add) of the
    sweep.  kind bgmv / sgmv: the micro-benchmark PR's grid (batches,
    hidden sizes, 4 adapters, sorted by id; one token per sequence or eight)
    widened to ranks 8-128; single: one adapter for every token, beside
    torch.mm of the same shapes; logits: expand r -> 128256 columns; golden:
    the shapes the PR prints (expand with add_inputs off, as its table)."""
    pts = []
    if grid == "full":
        for kind in ("bgmv", "sgmv"):
            for T in SWEEP_TOKENS:
                for H in SWEEP_HIDDEN:
                    for r in SWEEP_RANKS:
                        pts.append((kind, T, H, r, H, 4, 1 if kind == "bgmv" else 8, True))
    else:
        for kind in ("bgmv", "sgmv"):
            for T in (16, 256, 2048, 8192):
                for H in (4096, 16384):
                    for r in (16, 64):
                        pts.append((kind, T, H, r, H, 4, 1 if kind == "bgmv" else 8, True))
    pts += [("single", T, H, r, H, 1, 8, True) for T in (256, 2048, 8192) for H in (4096, 16384)
            for r in (16, 64)]
    pts += [("logits", T, 4096, 16, 128256, 4, 1, True) for T in (16, 256, 2048)]
    for g in golden_shapes():
        pts.append((f"golden:{g['source']}", g["m"], g["n"], g["rank"], g["n"], g["num_loras"], g["sl"],
                    g["source"] != "console_table"))
    return pts


def sweep(args):
    """Shrink and expand alone on the sweep shapes (fp16).  Before a point is
    timed, one set of its inputs runs build -> shrink -> expand and a sample
    of rows (the first and last of every segment, plus random ones) is
    checked against the oracle; a point that fails is reported and not
    timed.  Ids come from the shared generator; the tensors are drawn on the
    GPU (seeded), because host generation of the large points takes longer
    than timing them.  One JSON line per point and op."""
    import numpy as np
    import torch
    import lora_serving_build_amd as lsb
    import oracle
    import workloads as W
    torch.cuda.set_device(0)
    dt = torch.float16
    gen = torch.Generator(device="cuda")
    kinds = [k for k in args.sweep_kinds.split(",") if k] if args.sweep_kinds else None
    for kind, T, H, r, n, L, sl, add in sweep_points(args.sweep_grid):
        if kinds and not any(kind.startswith(k) for k in kinds):
            continue
        base_kind = "sgmv" if kind in ("single",) or kind.startswith("golden") else \
            ("bgmv" if kind == "logits" else kind)
        ids_w = W.make(f"{kind}_T{T}", "f16", T, 8, 8, L, [[8]], seed=7, seq_len=sl, sort_by_id=True) \
            if kind.startswith("golden") or kind == "single" else \
            W.sweep_point(base_kind, T, 8, 8, L=L)  # the same id draw at every size
        ids_np = ids_w.ids
        ids = torch.from_numpy(ids_np).cuda()
        per_set = T * H * 2 + T * n * 2 + L * r * H * 2 + L * r * n * 2 + T * r * 4
        P = max(2, min(64, int(math.ceil(args.pool_gib * 2**30 / per_set))))
        gen.manual_seed(T * 131 + H * 7 + r)
        sets = []
        for _ in range(P):
            sets.append(dict(
                x=torch.randn(T, H, generator=gen, device="cuda").to(dt),
                A=(torch.randn(L, r, H, generator=gen, device="cuda") / math.sqrt(H)).to(dt),
                B=(torch.randn(L, n, r, generator=gen, device="cuda") / math.sqrt(r)).to(dt),
                y=torch.randn(T, n, generator=gen, device="cuda").to(dt),
                v=torch.zeros(T, r, device="cuda"),
                seg=lsb.lora_build_segments(ids, L)))
        need = lsb.lora_shrink_workspace_bytes(T, L, H, r)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        head = {"sweep": kind, "tokens": T, "hidden": H, "out_cols": n, "rank": r, "num_loras": L,
                "seq_len": sl, "add_inputs": add}
        if kind == "single":
            # The single-adapter entry points: no metadata, token index = row.
            f_shrink = lambda s: lsb.lora_shrink_single(s["x"], s["A"][0], s["v"], workspace=ws)
            f_expand = lambda s, y=None: lsb.lora_expand_single(s["v"], s["B"][0], s["y"] if y is None else y,
                                                                add)
        else:
            f_shrink = lambda s: lsb.lora_shrink(s["x"], s["A"], s["seg"], s["v"], workspace=ws)
            f_expand = lambda s, y=None: lsb.lora_expand(s["v"], s["B"], s["seg"], s["y"] if y is None else y,
                                                         add)

        # Correctness first: one step on set 0 (y on a copy), sampled rows
        # against the oracle.
        s0 = sets[0]
        y_chk = s0["y"].clone()
        lsb.lora_build_segments(ids, L, seg=s0["seg"])
        f_shrink(s0)
        f_expand(s0, y_chk)
        torch.cuda.synchronize()
        st = s0["seg"].sorted_token[:T].cpu().numpy()
        ss = s0["seg"].seg_start.cpu().numpy()
        S = int(s0["seg"].counts[0].item())
        rng = np.random.default_rng(T + H + r)
        rows = np.unique(np.concatenate([st[ss[:S]], st[np.maximum(ss[1:S + 1] - 1, 0)],
                                         rng.integers(0, T, 16)])).astype(np.int64)
        ri = torch.from_numpy(rows).cuda()
        bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
        x_s = bits(s0["x"].index_select(0, ri))
        y0_s = bits(s0["y"].index_select(0, ri))
        ids_s = ids_np[rows]
        v_ref = oracle.shrink("f16", x_s, bits(s0["A"]), ids_s)
        y_ref = oracle.expand("f16", v_ref, bits(s0["B"]), ids_s, y0_s, 0, add)
        v_got = s0["v"].index_select(0, ri).cpu().numpy().astype(np.float64)
        y_got = y_chk.index_select(0, ri).float().cpu().numpy().astype(np.float64)
        ratio = max(tol_ratio(v_got, v_ref), tol_ratio(y_got, y_ref))
        head["parity_rows"] = int(rows.size)
        head["parity_ratio"] = round(ratio, 4)
        del y_chk
        if not ratio <= 1.0:
            print(json.dumps(dict(head, error="parity check failed")), flush=True)
            del sets, ws
            torch.cuda.empty_cache()
            continue

        K = min(P, 20) if T * H < 2**27 else 8
        shrink_b = T * H * 2 + L * r * H * 2 + T * r * 4
        expand_b = T * r * 4 + L * r * n * 2 + (2 if add else 1) * T * n * 2
        ref = {}
        if kind == "single":
            # The same products as one dense GEMM each (fp16 in, fp16 out):
            # x . A0^T and y + v16 . B0^T, with the transposed weights made
            # contiguous beforehand.
            for s in sets:
                s["At"] = s["A"][0].t().contiguous()
                s["Bt"] = s["B"][0].t().contiguous()
                s["v16"] = torch.zeros(T, r, dtype=dt, device="cuda")
                s["vo"] = torch.empty(T, r, dtype=dt, device="cuda")
            # The GEMM library does not allow stream capture here, so these are
            # timed eagerly: K calls over the pool between two events, after
            # one untimed pass (launch overhead is included).
            mm = {"shrink": lambda s: torch.mm(s["x"], s["At"], out=s["vo"]),
                  "expand": lambda s: s["y"].addmm_(s["v16"], s["Bt"])}
            for op, fn in mm.items():
                for i in range(K):
                    fn(sets[i % P])
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(K):
                    fn(sets[i % P])
                e1.record()
                torch.cuda.synchronize()
                ref[op] = e0.elapsed_time(e1) / K * 1e3
        for op, fn, nb in (("shrink", f_shrink, shrink_b), ("expand", f_expand, expand_b)):
            us = graph_time(torch, fn, sets, 0, K) / K * 1e3
            gbs = nb / (us * 1e-6) / 1e9
            rec = dict(head, op=op, us=round(us, 2), GB_s=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                       algorithmic_MiB=round(nb / 2**20, 2), pool_sets=P)
            if op in ref:
                rec["torch_mm_us_eager"] = round(ref[op], 2)
            print(json.dumps(rec), flush=True)
        del sets, ws
        torch.cuda.empty_cache()


def summarize_sweep(path):
    """profiles/sweep_shrink_expand_f16.md from the JSON lines of a --sweep run."""
    import collections
    recs = [json.loads(l) for l in open(path) if l.startswith("{")]
    by = collections.OrderedDict()
    fails = []
    for r in recs:
        if "error" in r:
            fails.append(r)
            continue
        key = (r["sweep"], r["tokens"], r["hidden"], r["out_cols"], r["rank"])
        by.setdefault(key, {})[r["op"]] = r
    lines = ["# Sweep: shrink and expand alone, fp16 (MI355X, one GPU)", "",
             "command (from the repository root):",
             "  python bench.py --sweep > sweep.jsonl; python bench.py --summarize-sweep sweep.jsonl", "",
             "Each op timed alone: K launches over a pool of argument sets (>= 1 GiB, or 64 sets) "
             "captured in one graph, inputs in HBM.  bgmv = one token per sequence, sgmv = eight, "
             "4 adapters sorted by id, expand with add_inputs unless noted; single = one adapter "
             "(torch.mm / addmm_ of the same shapes beside it, eager); logits = expand to 128256 "
             "columns; golden = shapes the micro-benchmark PR prints.  Before timing, each point "
             "checks sampled rows against the oracle (ratio <= 1 passes).  GB/s = algorithmic bytes "
             "/ time; frac = of 8 TB/s.", "",
             "| kind | T | H | n | r | parity | shrink us | GB/s | frac | expand us | GB/s | frac | torch.mm us | torch.addmm us |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for key, ops in by.items():
        sh, ex = ops.get("shrink", {}), ops.get("expand", {})
        any_ = sh or ex
        lines.append(f"| {key[0]} | {key[1]} | {key[2]} | {key[3]} | {key[4]} | {any_.get('parity_ratio', '')} | "
                     f"{sh.get('us', '')} | {sh.get('GB_s', '')} | {sh.get('hbm_frac', '')} | "
                     f"{ex.get('us', '')} | {ex.get('GB_s', '')} | {ex.get('hbm_frac', '')} | "
                     f"{sh.get('torch_mm_us_eager', '')} | {ex.get('torch_mm_us_eager', '')} |")
    if fails:
        lines += ["", "Points that failed the parity check (not timed):", ""]
        lines += [f"- {json.dumps(f)}" for f in fails]
    out = os.path.join(ROOT, "profiles", "sweep_shrink_expand_f16.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", out)


def _graph_us(torch, fn, sets, K):
    return graph_time(torch, fn, sets, 0, K) / K * 1e3


def plan_sweep(args):
    """The launch-plan measurements the design notes quote, each call alone
    over a pool of argument sets far beyond the Infinity Cache (bf16 unless
    noted; one JSON line per measurement):
      shrink_split  -- the tile shrink over H-split counts 1..8 (LORA_SHRINK_KSPLIT)
      expand_plan   -- the tile expand over token-tile size x run length
                       (LORA_EXPAND_TB x LORA_EXPAND_CPR)
      path          -- forced per-token, forced tile and automatic path, fp16,
                       4 adapters, one token per sequence
      mixed         -- decode + prefill mixes, and a prefill of a few adapters
                       of a large pool: the automatic path (the per-segment
                       split) against tiles only and per-token only
    Inputs are drawn on the GPU (seeded); ids from the shared generator."""
    import numpy as np
    import torch
    import lora_serving_build_amd as lsb
    import workloads as W
    torch.cuda.set_device(0)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    parts = [p for p in args.plans.split(",") if p]

    def emit(**kw):
        print(json.dumps(kw), flush=True)

    def with_env(env):
        for k in [k for k in os.environ if k.startswith("LORA_")]:
            del os.environ[k]
        os.environ.update(env)
        lsb.lora_reload_tuning()

    def ids_of(name):
        if name == "llama3_70b_layer":
            return W.make("p", "bf16", 8192, 8, 8, 64, [[8]], seed=1005, seq_len=(1, 512), id_dist="zipf",
                          zipf_s=1.1, neg_frac=0.05).ids, 64
        if name == "prefill_T2048":
            return W.make("p", "bf16", 2048, 8, 8, 4, [[8]], seed=1003, seq_len=8, sort_by_id=True).ids, 4
        T = int(name.split("_T")[1])
        return W.sweep_point("sgmv", T, 8, 8, L=4).ids, 4

    if "shrink_split" in parts:
        for name, H, r in (("llama3_70b_layer", 8192, 64), ("seq8_T8192", 16384, 16), ("seq8_T8192", 16384, 64),
                           ("prefill_T2048", 4096, 16)):
            ids_np, L = ids_of(name)
            T = ids_np.size
            ids = torch.from_numpy(ids_np).cuda()
            P = max(3, math.ceil(1.5 * 2**30 / (T * H * 2)))
            sets = [dict(x=torch.randn(T, H, generator=gen, device="cuda").to(torch.bfloat16),
                         A=(torch.randn(L, r, H, generator=gen, device="cuda") / math.sqrt(H)).to(torch.bfloat16),
                         v=torch.zeros(T, r, device="cuda"), seg=lsb.lora_build_segments(ids, L))
                    for _ in range(P)]
            ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
            for ks in ("", "1", "2", "3", "4", "5", "6", "7", "8"):
                with_env({"LORA_SHRINK_KSPLIT": ks} if ks else {})
                need = lsb.lora_shrink_workspace_bytes(T, L, H, r)
                us = _graph_us(torch, lambda s: lsb.lora_shrink(s["x"], s["A"], s["seg"], s["v"], workspace=ws),
                               sets, 2 * P)
                emit(plan="shrink_split", shape=name, H=H, r=r, ksplit=ks or "auto",
                     workspace_MB=round(need / 1e6, 2), us=round(us, 2))
            del sets, ws
            torch.cuda.empty_cache()

    if "expand_plan" in parts:
        shapes = (("llama3_70b_layer", [8192, 1024, 1024], 64), ("llama3_70b_layer", [28672, 28672], 64),
                  ("seq8_T8192", [16384], 16), ("seq8_T8192", [16384], 64), ("seq8_T8192", [4096], 64),
                  ("seq8_T2048", [16384], 64), ("seq8_T2048", [4096], 64))
        plans = ("", "1:2", "1:4", "2:2", "2:3", "2:4", "2:6", "2:8")
        for name, widths, r in shapes:
            ids_np, L = ids_of(name)
            T = ids_np.size
            n = sum(widths)
            ids = torch.from_numpy(ids_np).cuda()
            offs = [int(o) for o in np.cumsum([0] + widths[:-1])]
            P = max(3, math.ceil(2.0 * 2**30 / (T * n * 2)))
            sets = [dict(v=torch.randn(T, r, generator=gen, device="cuda"),
                         Bs=[(torch.randn(L, wd, r, generator=gen, device="cuda") / 8).to(torch.bfloat16)
                             for wd in widths],
                         y=torch.randn(T, n, generator=gen, device="cuda").to(torch.bfloat16),
                         seg=lsb.lora_build_segments(ids, L)) for _ in range(P)]
            for plan in plans:
                env = {}
                if plan:
                    tb, cpr = plan.split(":")
                    env = {"LORA_EXPAND_TB": tb, "LORA_EXPAND_CPR": cpr}
                with_env(env)
                us = _graph_us(torch, lambda s: lsb.lora_expand_slice(s["v"], s["Bs"], offs, s["seg"], s["y"], True),
                               sets, 3 * P)
                emit(plan="expand_plan", shape=name, slices=widths, r=r, tile_blocks_cpr=plan or "auto",
                     us=round(us, 2))
            del sets
            torch.cuda.empty_cache()
    with_env({})

    if "path" in parts:
        L = 4
        for T in (16, 64, 256, 512):
            ids = torch.from_numpy(W.sweep_point("bgmv", T, 8, 8, L=L).ids).cuda()
            for H in (1024, 4096, 16384):
                for r in (32, 64, 128):
                    P = max(4, min(64, math.ceil(2**30 / (T * H * 4 + L * r * H * 4))))
                    sets = [dict(x=torch.randn(T, H, generator=gen, device="cuda").half(),
                                 A=(torch.randn(L, r, H, generator=gen, device="cuda") / 64).half(),
                                 B=(torch.randn(L, H, r, generator=gen, device="cuda") / 8).half(),
                                 y=torch.randn(T, H, generator=gen, device="cuda").half(),
                                 v=torch.randn(T, r, generator=gen, device="cuda"),
                                 seg=lsb.lora_build_segments(ids, L)) for _ in range(P)]
                    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
                    rec = {}
                    for label, mode in (("per_token", lsb.PATH_BGMV), ("tiles", lsb.PATH_SGMV),
                                        ("auto", lsb.PATH_AUTO)):
                        lsb.lora_set_path(mode)
                        rec["shrink_" + label] = round(_graph_us(
                            torch, lambda s: lsb.lora_shrink(s["x"], s["A"], s["seg"], s["v"], workspace=ws),
                            sets, 2 * P), 2)
                        try:
                            rec["expand_" + label] = round(_graph_us(
                                torch, lambda s: lsb.lora_expand(s["v"], s["B"], s["seg"], s["y"], True),
                                sets, 2 * P), 2)
                        except lsb.LoraError:
                            rec["expand_" + label] = None
                    lsb.lora_set_path(lsb.PATH_AUTO)
                    emit(plan="path", T=T, H=H, r=r, **rec)
                    del sets, ws
                    torch.cuda.empty_cache()

    if "mixed" in parts:
        H = n = 4096
        for n_pre, pre_l, n_dec, L in ((7168, 16, 1024, 1040), (3072, 16, 1024, 1040), (7936, 16, 256, 300),
                                       (4096, 8, 0, 1024)):
            w = W.make_mixed("m", "bf16", n_pre, pre_l, n_dec, L, 8, 8, [[8]], seed=5)
            ids = torch.from_numpy(w.ids).cuda()
            T = w.T
            for r in (16, 32, 64):
                P = 6
                sets = [dict(x=torch.randn(T, H, generator=gen, device="cuda").to(torch.bfloat16),
                             A=(torch.randn(L, r, H, generator=gen, device="cuda") / 64).to(torch.bfloat16),
                             B=(torch.randn(L, n, r, generator=gen, device="cuda") / 8).to(torch.bfloat16),
                             y=torch.randn(T, n, generator=gen, device="cuda").to(torch.bfloat16),
                             v=torch.randn(T, r, generator=gen, device="cuda"),
                             seg=lsb.lora_build_segments(ids, L)) for _ in range(P)]
                ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
                rec = {}
                for label, mode in (("auto", lsb.PATH_AUTO), ("tiles", lsb.PATH_SGMV), ("per_token", lsb.PATH_BGMV)):
                    lsb.lora_set_path(mode)
                    rec["shrink_" + label] = round(_graph_us(
                        torch, lambda s: lsb.lora_shrink(s["x"], s["A"], s["seg"], s["v"], workspace=ws),
                        sets, 2 * P), 2)
                    rec["expand_" + label] = round(_graph_us(
                        torch, lambda s: lsb.lora_expand(s["v"], s["B"], s["seg"], s["y"], True), sets, 2 * P), 2)
                lsb.lora_set_path(lsb.PATH_AUTO)
                emit(plan="mixed", prefill=n_pre, prefill_loras=pre_l, decode=n_dec, L=L, H=H, r=r, **rec)
                del sets, ws
                torch.cuda.empty_cache()


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(unit, workload_name, src_hash):
    """HBM bytes of one call (build, shrink, expand or expand[k]) from the
    committed rocprofv3 counter summary, if the kernel sources of its op have
    not changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("ops", {}).get(unit)
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec["bytes_per_call"]


_COMMON = ["lora_serving_build_amd/csrc/lora_device.h", "lora_serving_build_amd/csrc/tiles.h",
           "lora_serving_build_amd/csrc/lora_kernels.h", "lora_serving_build_amd/csrc/lora_api.hip"]
KERNEL_SOURCES = {
    "build": ["lora_serving_build_amd/csrc/segments.hip"] + _COMMON,
    "shrink": ["lora_serving_build_amd/csrc/shrink.hip", "lora_serving_build_amd/csrc/bgmv.hip"] + _COMMON,
    "expand": ["lora_serving_build_amd/csrc/expand.hip", "lora_serving_build_amd/csrc/bgmv.hip"] + _COMMON,
}


def _output_label(o):
    return "+".join(str(q.n) for q in o.slices)


def measure(w, args, torch, lsb, check=True):
    """Times one workload: the K-step graph, then every op and every expand
    call alone.  Returns the fields of the JSON line that depend on it."""
    need = lsb.lora_shrink_workspace_bytes(w.T, w.L, w.H, w.r)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda") if need else None

    worst = None
    if check:
        log(f"{w.name}: parity check of one fresh step against the oracle (every row)")
        worst = parity_check(w, torch, lsb, ws)
        log(f"worst tolerance ratio {worst:.3g}")
        if not worst <= 1.0:
            print(json.dumps({"error": "parity check failed", "workload": w.name, "ratio": worst}))
            sys.exit(1)

    # Enough sets that every call timed alone cycles >= pool_gib of its own
    # operands (a shrink alone touches only x and A: with too few sets they
    # would stay in the 256 MB Infinity Cache), within 24 GiB of HBM.
    per_set = set_bytes(w)
    op_min = min([w.shrink_bytes()] + [w.output_bytes(o) for o in w.outputs])
    P = max(2, int(math.ceil(args.pool_gib * 2**30 / max(1, op_min))))
    P = max(2, min(P, int((24 << 30) // per_set)))
    log(f"argument pool: {P} sets of {per_set / 2**20:.1f} MiB")
    sets = make_pool(w, torch, lsb, P)
    torch.cuda.synchronize()

    fstep = lambda s: step(w, lsb, s, ws)
    for i in range(args.warmup):
        fstep(sets[i % P])
    torch.cuda.synchronize()

    K = args.steps
    log(f"timing {K} steps in one graph")
    ms = graph_time(torch, fstep, sets, args.warmup, K)
    ms_per_step = ms / K
    res = {"ms_per_step": ms_per_step, "pool_sets": P, "parity_ratio": worst}
    if args.profile:
        # Profiler runs: the steps only, so that every dispatch belongs to a
        # step in order (build, shrink, one expand per output).
        if args.traffic_probe:
            # A plain streaming kernel of known size (reads and writes 256 MiB
            # once each): the yardstick for the FETCH_SIZE / WRITE_SIZE counters.
            src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.int32, device="cuda")
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            torch.neg(src, out=dst)
            torch.cuda.synchronize()
            del src, dst
        return res, sets

    # Each op alone, K launches over the pool in one graph; every expand
    # call (one per output) also alone.
    units = [("build", lambda s: op_build(w, lsb, s, ws), 8 * w.T + 8 * (w.L + 1) + 16, 0, 1),
             ("shrink", lambda s: op_shrink(w, lsb, s, ws), w.shrink_bytes(), w.shrink_flops(), 1),
             ("expand", lambda s: op_expand(w, lsb, s, ws), w.expand_bytes(), w.expand_flops(),
              len(w.outputs))]
    if len(w.outputs) > 1:
        for oi, o in enumerate(w.outputs):
            n = sum(q.n for q in o.slices)
            units.append((f"expand[{oi}]", lambda s, oi=oi: op_expand_output(w, lsb, s, oi),
                          w.output_bytes(o), 2 * w.T_a * w.r * n, 1))
    ops = {}
    first = args.warmup + K
    for name, fn, nbytes, flops, launches in units:
        t = graph_time(torch, fn, sets, first, K) / K
        ops[name] = {"us_per_op": round(t * 1e3, 3), "launches": launches, "bytes": nbytes,
                     "GB_s": round(nbytes / (t * 1e-3) / 1e9, 1),
                     "TFLOP_s": round(flops / (t * 1e-3) / 1e12, 2)}
        if name.startswith("expand["):
            ops[name]["slices"] = _output_label(w.outputs[int(name[7:-1])])
        log(f"{name}: {t * 1e3:.2f} us/op, {ops[name]['GB_s']} GB/s, {ops[name]['TFLOP_s']} TFLOP/s")
        first += K

    # The roofline names one call, the longest single launch: the shrink, or
    # one expand call (with several outputs, each is timed alone above).
    cands = ["shrink"] + ([k for k in ops if k.startswith("expand[")] if len(w.outputs) > 1 else ["expand"])
    dom = max(cands, key=lambda k: ops[k]["us_per_op"])
    op_family = "shrink" if dom == "shrink" else "expand"
    src_hash = source_hash(KERNEL_SOURCES[op_family])
    traffic = measured_traffic(dom, w.name, src_hash)
    achieved = ops[dom]["bytes"] / (ops[dom]["us_per_op"] * 1e-6) / 1e9
    desc = {"shrink": "lora_shrink (segment tiles; with an H split, plus its reduce kernel)"
            if w.T > 512 else "lora_shrink", "expand": "lora_expand"}
    if dom.startswith("expand["):
        kdesc = f"lora_expand_slice into output {dom[7:-1]} (slices {ops[dom]['slices']})"
    else:
        kdesc = desc[dom]
    roofline = {"bound": "hbm", "kernel": kdesc, "op": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "bytes_per_launch": ops[dom]["bytes"],
                "us_per_launch": ops[dom]["us_per_op"], "source_hash": src_hash}
    res.update(ops=ops, roofline=roofline)

    # Mixed-rank workloads: the same step with each adapter's live rank handed
    # to the segment kernels (they then skip the zero padding).  Bytes count
    # the live ranks; the padded step above stays the workload's number.
    live = None
    if w.ranks is not None and bool((w.ranks < w.r).any()):
        import numpy as np
        rk = torch.from_numpy(np.ascontiguousarray(w.ranks, np.int32)).cuda()
        for s in sets:
            s.seg.c.lora_rank = rk.data_ptr()
        ms_live = graph_time(torch, fstep, sets, args.warmup, K) / K
        for s in sets:
            s.seg.c.lora_rank = None
        present = np.unique(w.ids[w.ids >= 0])
        live_sum = int(w.ranks[present].sum())
        n_tot = sum(q.n for o in w.outputs for q in o.slices)
        e = 2
        live_bytes = (w.T_a * w.H * e + live_sum * w.H * e + w.T_a * w.r * 4
                      + len(w.outputs) * w.T_a * w.r * 4 + live_sum * n_tot * e
                      + (2 if w.add else 1) * w.T_a * n_tot * e)
        live = {"ms_per_step": round(ms_live, 6), "speedup": round(ms_per_step / ms_live, 3),
                "bytes_live_ranks": live_bytes,
                "value": round(live_bytes / (ms_live * 1e-3) / 1e9, 2)}
        log(f"live ranks: {ms_live * 1e3:.2f} us/step ({live['speedup']}x)")
    res["live_ranks"] = live

    # Decode batches: the same step with shrink and expand in one launch
    # (lora_shrink_expand), checked against the oracle first.
    fused = None
    if fused_applies(w):
        ratio = parity_check(w, torch, lsb, ws, stepfn=fused_step) if check else None
        if ratio is not None and not ratio <= 1.0:
            print(json.dumps({"error": "parity check failed (fused step)", "workload": w.name, "ratio": ratio}))
            sys.exit(1)
        ms_f = graph_time(torch, lambda s: fused_step(w, lsb, s, ws), sets, args.warmup, K) / K
        t_op = graph_time(torch, lambda s: op_fused(w, lsb, s, ws), sets, args.warmup + K, K) / K
        fb = w.shrink_bytes() + w.expand_bytes()
        fused = {"ms_per_step": round(ms_f, 6), "speedup": round(ms_per_step / ms_f, 3),
                 "value": round(fb / (ms_f * 1e-3) / 1e9, 2), "us_per_op": round(t_op * 1e3, 3),
                 "parity_ratio": ratio}
        log(f"fused step: {ms_f * 1e3:.2f} us/step ({fused['speedup']}x), shrink+expand {t_op * 1e3:.2f} us")
    res["fused"] = fused
    return res, sets


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5,
                    help="named workload 1..5 (default 5, the largest: the 8192-token 70B layer)")
    ap.add_argument("--also", default="2",
                    help="comma-separated named workloads also timed, reported under "
                         "'other_workloads' (default 2, the 256-token decode; '' for none)")
    ap.add_argument("--pool-gib", type=float, default=1.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--no-context", action="store_true", help="skip the torch streaming-rate context")
    ap.add_argument("--profile", action="store_true",
                    help="profiler run: warm-up and the timed steps only, no per-op graphs, no "
                         "other workloads, no context, no CPU baseline")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="with --profile: also run one plain copy of 256 MiB (calibrates "
                         "FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize-profiles", action="store_true",
                    help="write profiles/ summaries from rocprofv3 CSVs (--trace, --fetch, --write)")
    ap.add_argument("--sweep", action="store_true",
                    help="time shrink and expand alone on the micro-benchmark sweep shapes")
    ap.add_argument("--sweep-grid", default="full", choices=("full", "thin"))
    ap.add_argument("--sweep-kinds", default="",
                    help="comma-separated sweep kinds to run (bgmv, sgmv, single, logits, golden)")
    ap.add_argument("--plans", default="",
                    help="comma-separated launch-plan measurements: shrink_split, expand_plan, path, mixed")
    ap.add_argument("--summarize-sweep", metavar="JSONL",
                    help="write profiles/sweep_shrink_expand_f16.md from a --sweep run's output")
    ap.add_argument("--trace", help="kernel_trace.csv of a --kernel-trace run")
    ap.add_argument("--stats", help="kernel_stats.csv of the same run")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--counters", help="CSV of a --pmc pass over the LDS / matrix-core counter set")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args)
        return
    if args.summarize_sweep:
        summarize_sweep(args.summarize_sweep)
        return
    if args.sweep:
        sweep(args)
        return
    if args.plans:
        plan_sweep(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the multi-LoRA path here has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    import torch
    import lora_serving_build_amd as lsb
    import workloads as W

    lsb.lib()
    torch.cuda.set_device(0)
    log(f"generating workload {args.config}")
    w = W.config(args.config)
    res, sets = measure(w, args, torch, lsb, check=not args.no_check)
    del sets
    torch.cuda.empty_cache()
    ms_per_step = res["ms_per_step"]
    step_bytes = w.shrink_bytes() + w.expand_bytes()
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    if args.profile:
        log(f"{w.name}: {ms_per_step * 1e3:.2f} us/step")
        return

    others = {}
    for k in [int(c) for c in args.also.split(",") if c.strip()]:
        if k == args.config:
            continue
        wk = W.config(k)
        rk, sk = measure(wk, args, torch, lsb, check=not args.no_check)
        del sk
        torch.cuda.empty_cache()
        bk = wk.shrink_bytes() + wk.expand_bytes()
        others[wk.name] = {"value": round(bk / (rk["ms_per_step"] * 1e-3) / 1e9, 2), "unit": "GB/s",
                           "ms_per_step": round(rk["ms_per_step"], 6), "ops": rk["ops"],
                           "roofline": rk["roofline"], "parity_ratio": rk["parity_ratio"],
                           "pool_sets": rk["pool_sets"], "live_ranks": rk["live_ranks"], "fused": rk["fused"]}

    # Context for the roofline fraction: what plain torch streaming kernels
    # reach on this GPU (a copy and an in-place add over 512 MiB each, twice
    # the Infinity Cache), timed eagerly over 10 calls between two events.
    hbm_context = None
    if not args.no_context:
        src = torch.ones((512 << 20) // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        rates = {}
        for name, fn in (("copy", lambda: dst.copy_(src)), ("rmw", lambda: src.add_(1))):
            fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                fn()
            e1.record()
            torch.cuda.synchronize()
            rates[name] = round(2 * (512 << 20) * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        del src, dst
        torch.cuda.empty_cache()
        # The launch floor the decode-sized ops sit on: 64 launches of a
        # one-element add (an empty kernel in all but name) captured in one
        # graph, replayed once untimed and once between two events.
        tiny = torch.zeros(1, dtype=torch.int32, device="cuda")
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(64):
                tiny.add_(1)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        floor_us = round(e0.elapsed_time(e1) * 1e3 / 64, 2)
        del g, tiny
        hbm_context = {"copy_GB_s": rates["copy"], "rmw_GB_s": rates["rmw"],
                       "how": "torch copy_ and in-place add_ over 512 MiB int32, read + write bytes",
                       "launch_floor_us": floor_us,
                       "launch_floor_how": "graph replay of 64 one-element torch add_ launches, per launch"}
        log(f"torch streaming context: copy {rates['copy']} GB/s, rmw {rates['rmw']} GB/s; "
            f"launch floor {floor_us} us per launch in a graph")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        cpu = cpu_baseline(w, step_bytes)

    flops = w.shrink_flops() + w.expand_flops()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.T, "active_tokens": w.T_a, "hidden": w.H,
                   "rank": w.r, "num_loras": w.L, "distinct_loras": w.distinct,
                   "outputs": [[q.n for q in o.slices] for o in w.outputs], "add_inputs": w.add,
                   "pool_sets": res["pool_sets"], "parallelism": "none"},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "mfma_frac": round(flops / (ms_per_step * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype], 5),
        "tokens_per_s": round(w.T / (ms_per_step * 1e-3), 1),
        "ops": res["ops"],
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "parity_ratio": res["parity_ratio"],
        "live_ranks": res["live_ranks"],
        "fused": res["fused"],
        "other_workloads": others,
        "hbm_context": hbm_context,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
