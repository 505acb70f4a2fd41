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


class ArgSet:
    """One set of device buffers for one step."""

    def __init__(self, w, torch, lsb, src=None):
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        import numpy as np

        def dev(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(tdt)

        if src is None:
            self.ids = torch.from_numpy(w.ids).cuda()
            self.x = dev(w.x)
            self.A = dev(w.A)
            self.Bs = [[dev(s.B) for s in o.slices] for o in w.outputs]
            self.ys = [dev(o.y0) for o in w.outputs]
        else:
            self.ids = src.ids.clone()
            self.x = src.x.clone()
            self.A = src.A.clone()
            self.Bs = [[b.clone() for b in bl] for bl in src.Bs]
            self.ys = [y.clone() for y in src.ys]
        self.v = torch.zeros(w.T, w.r, dtype=torch.float32, device="cuda")
        self.seg = lsb.Segments(self.ids, w.L)

    def nbytes(self):
        t = [self.ids, self.x, self.A, self.v] + [b for bl in self.Bs for b in bl] + self.ys
        return sum(x.numel() * x.element_size() for x in t)


def op_build(w, lsb, s, ws):
    lsb.lora_build_segments(s.ids, w.L, seg=s.seg)


def op_shrink(w, lsb, s, ws):
    lsb.lora_shrink(s.x, s.A, s.seg, s.v, workspace=ws)


def op_expand(w, lsb, s, ws):
    for o, Bs, y in zip(w.outputs, s.Bs, s.ys):
        if len(o.slices) == 1 and o.slices[0].col_off == 0:
            lsb.lora_expand(s.v, Bs[0], s.seg, y, w.add)
        else:
            lsb.lora_expand_slice(s.v, Bs, [q.col_off for q in o.slices], s.seg, y, w.add)


def step(w, lsb, s, ws):
    op_build(w, lsb, s, ws)
    op_shrink(w, lsb, s, ws)
    op_expand(w, lsb, s, ws)


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


def parity_check(w, torch, lsb, ws):
    """Checks one fresh step against the oracle before anything is timed."""
    import numpy as np
    import oracle
    import workloads as W
    s = ArgSet(w, torch, lsb)
    step(w, lsb, s, ws)
    torch.cuda.synchronize()
    act = np.nonzero(w.active)[0].astype(np.int32)
    v_ref = oracle.shrink(w.dtype, w.x, w.A, w.ids, rows=act)
    vg = s.v.cpu().numpy().astype(np.float64)[act]
    worst = float(np.max(np.abs(vg - v_ref) / (1e-2 * (1 + np.abs(v_ref))))) if act.size else 0.0
    v_full = np.zeros((w.T, w.r))
    v_full[act] = v_ref
    for o, y in zip(w.outputs, s.ys):
        cols = np.concatenate([np.arange(q.col_off, q.col_off + q.n) for q in o.slices])
        ref = oracle.expand_slice(w.dtype, v_full, [q.B for q in o.slices], [q.col_off for q in o.slices],
                                  w.ids, o.y0, w.add, rows=act)
        yb = y.view(torch.int16).cpu().numpy().view(np.uint16)[act][:, cols]
        got = W.bits_to_f32(yb, w.dtype).astype(np.float64)
        if act.size:
            worst = max(worst, float(np.max(np.abs(got - ref) / (1e-2 * (1 + np.abs(ref))))))
    return worst


def cpu_baseline(w, step_bytes):
    """The fp64 oracle (as it is) on the host cores, over the same workload,
    repeated to about 10 s of CPU work."""
    import numpy as np
    import oracle

    def run():
        oracle.build_segments(w.ids, w.L)
        v = oracle.shrink(w.dtype, w.x, w.A, w.ids)
        v = np.nan_to_num(v)
        for o in w.outputs:
            oracle.expand_slice(w.dtype, v, [q.B for q in o.slices], [q.col_off for q in o.slices],
                                w.ids, o.y0, w.add)

    t0 = time.perf_counter()
    run()
    t1 = time.perf_counter() - t0
    reps = max(1, min(100000, int(math.ceil(12.0 / max(t1, 1e-6)))))
    if t1 > 30.0:
        reps = 1
    t0 = time.perf_counter()
    for _ in range(reps - 1):
        run()
    el = time.perf_counter() - t0 + (t1 if reps >= 1 else 0.0)
    return {
        "value": round(step_bytes * reps / el / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"the whole workload (metadata, shrink, expand of every output) run {reps}x "
                  f"in {el:.1f} s, OpenMP over tokens",
        "tokens_per_s": round(w.T * reps / el, 2),
    }


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
        short = kn.replace("void ", "").replace("lora::(anonymous namespace)::", "").split("(")[0]
        tot[short][r["Counter_Name"]] += float(r["Counter_Value"])
        calls[short].add(r.get("Dispatch_Id", r.get("Correlation_Id", "")))
    lines = [f"# rocprofv3 LDS and matrix-core counters: {name}", "",
             "command (from the repository root, on one MI355X):",
             f"  rocprofv3 --pmc {' '.join(COUNTER_SET)} -d <dir> -o run --output-format csv -- "
             f"python bench.py --config {args.config} --no-cpu-baseline --no-context",
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
    """Turns rocprofv3 CSV output of this script into the short summaries kept
    under profiles/: a kernel-trace table, and per-op HBM traffic from the
    FETCH_SIZE / WRITE_SIZE runs scaled by a copy of known size."""
    import csv
    import collections
    import workloads as W
    w = W.config(args.config)
    name = w.name
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    lines = [f"# rocprofv3 kernel trace: {name}", "",
             "command (from the repository root, on one MI355X):",
             f"  rocprofv3 --kernel-trace --stats -d <dir> -o run --output-format csv -- "
             f"python bench.py --config {args.config} --no-cpu-baseline",
             "", "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    stats = list(csv.DictReader(open(args.trace)))
    op_avg = {}
    for r in stats:
        kn = r["Name"]
        op = op_of(kn)
        if op is None and "copy" not in kn.lower():
            continue
        short = kn.replace("void ", "").replace("lora::(anonymous namespace)::", "").split("(")[0]
        lines.append(f"| {short} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                     f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} |")
        if op:
            op_avg.setdefault(op, []).append((kn, float(r["AverageNs"]) / 1e3, int(r["Calls"])))
    steps = sum(c for _, _, c in op_avg.get("build", [])) or 1
    lines += ["", f"Per op and step ({steps} steps traced; every kernel of the op counted, "
              "algorithmic bytes of the op):"]
    nbytes = {"shrink": w.shrink_bytes(), "expand": w.expand_bytes()}
    for op, rows in sorted(op_avg.items()):
        per_step = sum(a * c for _, a, c in rows) / steps
        line = f"- {op}: {per_step:.2f} us per step"
        if op in nbytes:
            line += (f"; {nbytes[op] / 2**20:.3f} MiB -> "
                     f"{nbytes[op] / (per_step * 1e-6) / 1e9:.1f} GB/s")
        lines.append(line)
    with open(os.path.join(out_dir, f"trace_{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", os.path.join(out_dir, f"trace_{name}.md"))
    if args.counters:
        summarize_counters(args, name, out_dir)
    if not (args.fetch and args.write):
        return

    def per_op(path, counter):
        rows = list(csv.DictReader(open(path)))
        tot = collections.defaultdict(float)
        steps = 0
        copy_vals = []
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            kn = r["Kernel_Name"]
            val = float(r["Counter_Value"])  # KiB per dispatch
            op = op_of(kn)
            if op == "build":
                steps += 1
            if op:
                tot[op] += val
            elif "neg_kernel" in kn:
                copy_vals.append(val)
        return {k: v / max(1, steps) for k, v in tot.items()}, copy_vals, steps

    fetch, fcopy, steps = per_op(args.fetch, "FETCH_SIZE")
    write, wcopy, _ = per_op(args.write, "WRITE_SIZE")
    if not fcopy or not wcopy:
        raise SystemExit("no copy probe dispatch found: run the --pmc passes with --traffic-probe")
    f_fetch = max(fcopy) * 1024 / COPY_PROBE_BYTES
    f_write = max(wcopy) * 1024 / COPY_PROBE_BYTES
    rec = {"workload": name, "steps_profiled": steps,
           "copy_probe_bytes": COPY_PROBE_BYTES,
           "fetch_scale": round(f_fetch, 4), "write_scale": round(f_write, 4),
           "ops": {}}
    for op in sorted(set(fetch) | set(write)):
        b = fetch.get(op, 0.0) * 1024 / f_fetch + write.get(op, 0.0) * 1024 / f_write
        alg = {"shrink": w.shrink_bytes(), "expand": w.expand_bytes()}.get(op)
        rec["ops"][op] = {"bytes_per_call": int(b), "fetch_kib": round(fetch.get(op, 0.0), 1),
                          "write_kib": round(write.get(op, 0.0), 1),
                          "algorithmic_bytes": alg,
                          "source_hash": source_hash(KERNEL_SOURCES[op])}
    pool = f" --pool-gib {args.pool_gib:g}" if args.pool_gib != 1.0 else ""
    rec["commands"] = [
        f"rocprofv3 --pmc FETCH_SIZE -d <dir> -o run --output-format csv -- python bench.py "
        f"--config {args.config} --no-cpu-baseline --traffic-probe{pool}",
        f"rocprofv3 --pmc WRITE_SIZE -d <dir> -o run --output-format csv -- python bench.py "
        f"--config {args.config} --no-cpu-baseline --traffic-probe{pool}"]
    path = os.path.join(out_dir, f"traffic_{name}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print("wrote", path)


SWEEP_POINTS = (  # (kind, tokens, hidden, rank): the micro-benchmark grid, thinned
    [(k, T, H, r) for k in ("bgmv", "sgmv") for T in (16, 256, 2048, 8192)
     for H in (4096, 16384) for r in (16, 64)]
    + [("sgmv", 65536, 16384, 16)]   # the review thread's bs 8192 x seq 8 example
    # one adapter for every token (the TPU PR's unmasked single-adapter case):
    # torch.mm of the same shapes (hipBLASLt) is timed beside it
    + [("single", T, H, r) for T in (256, 2048, 8192) for H in (4096, 16384) for r in (16, 64)]
    # LoRA on the logits layer (TPU PR): expand r -> vocabulary, 128256 columns
    + [("logits", T, 4096, 16) for T in (16, 256, 2048)])


def sweep(args):
    """Shrink and expand alone on the micro-benchmark sweep shapes: 4 adapters,
    ids sorted, one token per sequence (bgmv) or eight (sgmv), expand r -> H
    with add_inputs; then one adapter for every token beside torch.mm of the
    same shapes, and the logits layer (expand r -> 128256 columns).  Ids come from the shared generator; the tensors are drawn
    on the GPU (seeded) because host generation of the large points takes
    longer than timing them.  One JSON line per point and op."""
    import torch
    import lora_serving_build_amd as lsb
    import workloads as W
    torch.cuda.set_device(0)
    dt = torch.float16
    gen = torch.Generator(device="cuda")
    for kind, T, H, r in SWEEP_POINTS:
        L = 1 if kind == "single" else 4
        n = 128256 if kind == "logits" else H
        ids_w = W.sweep_point("bgmv" if kind == "logits" else ("sgmv" if kind == "single" else kind),
                              T, 8, 8, L=L)  # same id draw as the full-size point
        ids = torch.from_numpy(ids_w.ids).cuda()
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
        K = min(P, 20) if T * H < 2**27 else 8
        shrink_b = T * H * 2 + L * r * H * 2 + T * r * 4
        expand_b = T * r * 4 + L * r * n * 2 + 2 * T * n * 2
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
        for op, fn, nb in (
                ("shrink", lambda s: lsb.lora_shrink(s["x"], s["A"], s["seg"], s["v"], workspace=ws), shrink_b),
                ("expand", lambda s: lsb.lora_expand(s["v"], s["B"], s["seg"], s["y"], True), expand_b)):
            us = graph_time(torch, fn, sets, 0, K) / K * 1e3
            gbs = nb / (us * 1e-6) / 1e9
            rec = {"sweep": kind, "tokens": T, "hidden": H, "out_cols": n, "rank": r, "num_loras": L,
                   "op": op, "us": round(us, 2), "GB_s": round(gbs, 1),
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                   "algorithmic_MiB": round(nb / 2**20, 2), "pool_sets": P}
            if op in ref:
                rec["torch_mm_us_eager"] = round(ref[op], 2)
            print(json.dumps(rec), flush=True)
        del sets, ws
        torch.cuda.empty_cache()


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(op, workload_name, src_hash, launches):
    """HBM bytes per launch of an op from the committed rocprofv3 counter
    summary, if the op's kernel sources have not changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("ops", {}).get(op)
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec["bytes_per_call"] // launches


_COMMON = ["lora_serving_build_amd/csrc/lora_device.h", "lora_serving_build_amd/csrc/tiles.h",
           "lora_serving_build_amd/csrc/lora_kernels.h", "lora_serving_build_amd/csrc/lora_api.hip"]
KERNEL_SOURCES = {
    "build": ["lora_serving_build_amd/csrc/segments.hip"] + _COMMON,
    "shrink": ["lora_serving_build_amd/csrc/shrink.hip", "lora_serving_build_amd/csrc/bgmv.hip"] + _COMMON,
    "expand": ["lora_serving_build_amd/csrc/expand.hip", "lora_serving_build_amd/csrc/bgmv.hip"] + _COMMON,
}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="named workload 1..5 (default 2)")
    ap.add_argument("--pool-gib", type=float, default=1.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--no-context", action="store_true", help="skip the torch streaming-rate context")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="also run one plain copy of 256 MiB (calibrates FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize-profiles", action="store_true",
                    help="write profiles/ summaries from rocprofv3 CSVs (--trace, --fetch, --write)")
    ap.add_argument("--sweep", action="store_true",
                    help="time shrink and expand alone on the micro-benchmark sweep shapes")
    ap.add_argument("--trace")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--counters", help="CSV of a --pmc pass over the LDS / matrix-core counter set")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args)
        return
    if args.sweep:
        sweep(args)
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
    need = lsb.lora_shrink_workspace_bytes(w.T, w.L, w.H, w.r)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda") if need else None

    worst = None
    if not args.no_check:
        log("parity check of one fresh step against the oracle")
        worst = parity_check(w, torch, lsb, ws)
        log(f"worst tolerance ratio {worst:.3g}")
        if not worst <= 1.0:
            print(json.dumps({"error": "parity check failed", "ratio": worst}))
            sys.exit(1)

    base = ArgSet(w, torch, lsb)
    per_set = base.nbytes()
    P = max(2, int(math.ceil(args.pool_gib * 2**30 / per_set)))
    log(f"argument pool: {P} sets of {per_set / 2**20:.1f} MiB")
    sets = [base] + [ArgSet(w, torch, lsb, src=base) for _ in range(P - 1)]
    torch.cuda.synchronize()

    fstep = lambda s: step(w, lsb, s, ws)
    for i in range(args.warmup):
        fstep(sets[i % P])
    torch.cuda.synchronize()

    K = args.steps
    log(f"timing {K} steps in one graph")
    ms = graph_time(torch, fstep, sets, args.warmup, K)
    ms_per_step = ms / K

    shrink_b = w.shrink_bytes()
    expand_b = w.expand_bytes()
    step_bytes = shrink_b + expand_b
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # Per-op timing: each op alone, K launches over the pool in one graph.
    ops = {}
    for name, fn, nbytes, flops in (
            ("build", op_build, 8 * w.T + 8 * (w.L + 1) + 16, 0),
            ("shrink", op_shrink, shrink_b, w.shrink_flops()),
            ("expand", op_expand, expand_b, w.expand_flops())):
        t = graph_time(torch, lambda s, fn=fn: fn(w, lsb, s, ws), sets, args.warmup + K, K) / K
        launches = 1 if name != "expand" else len(w.outputs)
        ops[name] = {"us_per_op": round(t * 1e3, 3), "launches": launches, "bytes": nbytes,
                     "GB_s": round(nbytes / (t * 1e-3) / 1e9, 1),
                     "TFLOP_s": round(flops / (t * 1e-3) / 1e12, 2)}
        log(f"{name}: {t * 1e3:.2f} us/op, {ops[name]['GB_s']} GB/s, {ops[name]['TFLOP_s']} TFLOP/s")
    if args.traffic_probe:
        # A plain streaming kernel of known size (reads and writes 256 MiB
        # once each): the yardstick for the FETCH_SIZE / WRITE_SIZE counters.
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    dom = max(("shrink", "expand"), key=lambda k: ops[k]["us_per_op"])
    src_hash = source_hash(KERNEL_SOURCES[dom])
    traffic = measured_traffic(dom, w.name, src_hash, ops[dom]["launches"])
    achieved = ops[dom]["bytes"] / (ops[dom]["us_per_op"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "bytes_per_launch": ops[dom]["bytes"] // ops[dom]["launches"],
                "us_per_launch": round(ops[dom]["us_per_op"] / ops[dom]["launches"], 3),
                "source_hash": src_hash}

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
        hbm_context = {"copy_GB_s": rates["copy"], "rmw_GB_s": rates["rmw"],
                       "how": "torch copy_ and in-place add_ over 512 MiB int32, read + write bytes"}
        log(f"torch streaming context: copy {rates['copy']} GB/s, rmw {rates['rmw']} GB/s")

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
        "steps": K,
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
                   "pool_sets": P, "parallelism": "none"},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "mfma_frac": round(flops / (ms_per_step * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype], 5),
        "tokens_per_s": round(w.T / (ms_per_step * 1e-3), 1),
        "ops": ops,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity_ratio": worst,
        "live_ranks": live,
        "hbm_context": hbm_context,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
