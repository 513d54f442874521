#!/usr/bin/env python3
"""Decode-attention benchmark: achieved HBM GB/s and attention calls/s.

One step = one split-KV decode attention call (split kernel + merge kernel)
over one batch of seeded synthetic inputs already resident in HBM.  The
default workload is the Qwen3-8B-shaped decode batch (B=64, qLen=1, Hq=32,
Hkv=8, D=128, bf16, KV cache of 16384 with per-sequence lengths uniform in
[1024, 16384], two K channels per head scaled x8).  Prints one JSON line.

  value      algorithmic bytes per call / wall time per call (GB/s), where the
             algorithmic bytes are Q + every visible K/V row once + out + lse
             + cache_seqlens (nothing for scratch, the unread cache tail or
             masked work);
  roofline   the split kernel alone: its algorithmic bytes (K/V rows + Q) per
             launch / its mean duration from HIP events recorded around it on
             the stream it runs on, against the 8 TB/s HBM peak; traffic from
             a committed rocprofv3 counter summary when it matches the current kernel sources;
  cpu_baseline  the fp64 CPU oracle timed on this host on the same inputs
             (median of up to 3 runs with every core it may use, and a
             one-thread figure on a sample of the batch);
  read_ceiling  the library's streaming-read probe over 2 GiB (nt and default
             cache policy): the practical HBM read rate on this GPU;
  mfma_util  for the matrix-core path: attention flops (4 D per visible
             (row, key) pair) per split-kernel launch and per call against the
             2.5 PFLOP/s dense bf16/fp16 peak;
  dispatch_check  a few calls under the profiler must have dispatched
             exactly one split kernel each, plus one merge kernel when the
             plan has a merge, and nothing else (the run fails otherwise);
  configs    the same figures for every other named decode workload (the
             tiny causal case, the 12 SmallQ cases, the Qwen3-4B and
             Llama-70B batches), each over its own 1000 timed calls.

Caches smaller than 1 GiB are timed over rotating copies (enough that the
copies together hold at least 1 GiB of K/V, at most 64), so that no call
finds its K/V in the last-level cache left there by the previous one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "qwen3_8b_decode"
# the sources each split kernel is compiled from, plus the planner that
# chooses its launch (grid, partial results): a counter record is valid only
# while none of them has changed
_COMMON = ["split_kv_decode_amd/csrc/schedule.h", "split_kv_decode_amd/csrc/device_common.h",
           "split_kv_decode_amd/csrc/launch.h", "split_kv_decode_amd/csrc/api.hip",
           "include/mxfa.h"]
KERNEL_SOURCES = {
    "split_kv_valu_kernel": ["split_kv_decode_amd/csrc/split_valu.hip"] + _COMMON,
    "split_kv_mfma_kernel": ["split_kv_decode_amd/csrc/split_mfma.hip",
                             "split_kv_decode_amd/csrc/split_mfma_wide.hip",
                             "split_kv_decode_amd/csrc/mfma_kernel.h"] + _COMMON,
}
SPLIT_KERNEL = {"valu": "split_kv_valu_kernel", "mfma": "split_kv_mfma_kernel"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def code_text(src: str) -> str:
    """C/C++ source without its comments, blank lines and runs of spaces:
    what the compiler sees, so that an edit of comments or layout leaves a
    kernel's digest (and the counters recorded against it) valid.  String
    and character literals are kept as they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c == "/" and src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif c == "/" and src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    lines = (" ".join(line.split()) for line in "".join(out).splitlines())
    return "\n".join(line for line in lines if line)


def kernel_digest(kernel: str) -> str:
    """Digest of the code (comments and layout left out) of the sources
    `kernel` is built and planned from."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def traffic_for(workload: str, kernel: str):
    """HBM bytes per split-kernel launch from the committed counter summary,
    or None when there is none for this workload and kernel, or when the
    kernel's sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel") != kernel or rec.get("kernel_digest") != kernel_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


def _kernel_rows(csv_path):
    import csv
    with open(csv_path) as f:
        return list(csv.DictReader(f))


def summarize_profiles(trace_dir, fetch_dir, write_dir, workload, commands, mfma_dir=None,
                       page_size=0, out_dir=None, traffic_file=None):
    """Turn rocprofv3 outputs (kernel-trace stats, FETCH_SIZE pass, WRITE_SIZE
    pass, each of a bench run with --copy-calibration, and for the matrix-core
    kernel a MfmaUtil / MfmaFlopsBF16 / MfmaFlopsF16 pass) into a short
    summary under profiles/ and the per-launch traffic record bench.py
    reports.  The traffic counters are scaled by what they read for the 1 GiB
    device copy.  With page_size P the run read a paged cache: the record is
    the workload's paged one (NAME_pagedP) and the algorithmic bytes add one
    block-table entry per page touched.  out_dir / traffic_file: where the
    summary and the record go (profiles/ and its traffic.json by default).
    Returns the record."""
    import statistics
    stats = _kernel_rows(os.path.join(trace_dir, "run_kernel_stats.csv"))
    fetch = _kernel_rows(os.path.join(fetch_dir, "run_counter_collection.csv"))
    write = _kernel_rows(os.path.join(write_dir, "run_counter_collection.csv"))
    copy_bytes = float(1 << 30)

    def per_kernel(rows, counter):
        out = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return out

    f_by, w_by = per_kernel(fetch, "FETCH_SIZE"), per_kernel(write, "WRITE_SIZE")
    copy_name = [k for k in f_by if "copyBuffer" in k or "copy" in k.lower()]
    big = lambda xs: [x for x in xs if x > copy_bytes / 4]
    f_copy = statistics.median(big(f_by[copy_name[0]]))
    w_copy = statistics.median(big(w_by[copy_name[0]]))
    f_scale, w_scale = copy_bytes / f_copy, copy_bytes / w_copy
    split = [k for k in f_by if "split_kv_" in k][0]
    merge = [k for k in f_by if "combine_kernel" in k]
    f_raw, w_raw = statistics.median(f_by[split]), statistics.median(w_by[split])
    f_split, w_split = f_raw * f_scale, w_raw * w_scale

    import workloads as wl
    packed = workload in wl.VARLEN_WORKLOADS
    if packed:
        # a packed batch: distinct K/V + Q bytes once; attention flops
        w = wl.VARLEN_WORKLOADS[workload]
        lens = list(w.klens)
        alg = 2 * sum(w.klens) * w.Hkv * w.D * 2 + sum(w.qlens) * w.Hq * w.D * 2
    else:
        w = wl.WORKLOADS[workload]
        lens = wl.make_inputs(w).lengths() if w.len_range else [w.kv_cap] * w.B
        alg = wl.kv_bytes(w, lens) + w.B * w.qLen * w.Hq * w.D * w.elt
    if page_size:
        alg += sum(-(-max(0, min(n, w.kv_cap)) // page_size) for n in lens) * 4
        workload = f"{workload}_paged{page_size}"
    kname = "split_kv_mfma_kernel" if "mfma" in split else "split_kv_valu_kernel"
    trace_rows = [r for r in stats if "split_kv_" in r["Name"] or "combine_kernel" in r["Name"]]
    lines = [f"# {kname} on {workload}", "",
             f"Workload: {w.describe()}"
             f"{f', K/V in pages of {page_size} tokens' if page_size else ''}.", "",
             "Commands (run from the repository root on one MI355X, after "
             "`cd /tmp && export TMPDIR=/tmp`):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
              "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in trace_rows:
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    avg_ns = float([r for r in trace_rows if "split_kv_" in r["Name"]][0]["AverageNs"])
    lines += ["", "## HBM traffic per split-kernel launch (rocprofv3 --pmc)", "",
              f"- copy calibration: a 1 GiB device copy reads as {f_copy / 2**20:.1f} MiB of "
              f"FETCH_SIZE and {w_copy / 2**20:.1f} MiB of WRITE_SIZE; scale factors "
              f"{f_scale:.3f} (fetch) and {w_scale:.3f} (write)",
              f"- split kernel, raw counters (medians over {len(f_by[split])} launches): "
              f"FETCH_SIZE {f_raw / 1024:.0f} KiB ({f_raw / 1e9:.4f} GB), WRITE_SIZE "
              f"{w_raw / 1024:.0f} KiB ({w_raw / 1e9:.4f} GB) per launch",
              f"- split kernel, scaled: fetch {f_split / 1e9:.4f} GB (x{f_scale:.3f}), write "
              f"{w_split / 1e9:.4f} GB (x{w_scale:.3f})",
              f"- algorithmic bytes per launch (K/V rows read once + Q): {alg / 1e9:.4f} GB; "
              f"fetched / algorithmic = {f_split / alg:.4f}",
              f"- achieved from the trace average: {alg / (avg_ns * 1e-9) / 1e9:.1f} GB/s "
              f"({100 * alg / (avg_ns * 1e-9) / 1e9 / HBM_PEAK_GBS:.1f}% of 8 TB/s)"]
    if packed:
        fl_alg = wl.varlen_flops(w)
        lines.append(f"- attention flops per launch {fl_alg / 1e9:.1f} GFLOP: "
                     f"{fl_alg / (avg_ns * 1e-9) / 1e12:.1f} TFLOP/s from the trace average "
                     f"({100 * fl_alg / (avg_ns * 1e-9) / 2.5e15:.1f}% of 2.5 PFLOP/s); the "
                     f"fetched bytes are {f_split / alg:.2f}x the distinct K/V + Q bytes "
                     f"(every row block of a kv head reads its K/V; this counts the reads "
                     f"that miss the L2s)")
    if merge:
        fmr, wmr = statistics.median(f_by[merge[0]]), statistics.median(w_by[merge[0]])
        lines.append(f"- merge kernel: raw FETCH_SIZE {fmr / 1024:.0f} KiB, WRITE_SIZE "
                     f"{wmr / 1024:.0f} KiB; scaled fetch {fmr * f_scale / 1e6:.2f} MB, write "
                     f"{wmr * w_scale / 1e6:.2f} MB per launch")
    mfma_rec = None
    if mfma_dir:
        rows = _kernel_rows(os.path.join(mfma_dir, "run_counter_collection.csv"))
        by = {}
        for r in rows:
            if "split_kv_" in r["Kernel_Name"]:
                by.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        util = statistics.median(by["MfmaUtil"]) if "MfmaUtil" in by else None
        fl = sum(statistics.median(by[k]) for k in ("MfmaFlopsBF16", "MfmaFlopsF16") if k in by)
        alg_fl = wl.varlen_flops(w) if packed else 4 * w.D * wl.visible_pairs(w, lens)
        lines += ["", "## Matrix cores (rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 MfmaFlopsF16)", "",
                  f"- MfmaUtil (MFMA busy cycles / (GPU active cycles x SIMDs)): {util:.2f}%"
                  if util is not None else "- MfmaUtil: not reported",
                  f"- MFMA flops per launch from the counters: {fl / 1e9:.2f} GFLOP; the "
                  f"attention's algorithmic flops (4 D per visible (row, key) pair): "
                  f"{alg_fl / 1e9:.2f} GFLOP (the counters also count padded rows and keys)",
                  f"- algorithmic flops / trace average / 2.5 PFLOP/s: "
                  f"{100 * alg_fl / (avg_ns * 1e-9) / 2.5e15:.2f}%"]
        mfma_rec = {"mfma_util_pct": util, "mfma_flops": fl, "algorithmic_flops": alg_fl}
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    traffic_file = traffic_file or TRAFFIC_FILE
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, f"{kname}_{workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    try:
        with open(traffic_file) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec[workload] = {"kernel": kname, "kernel_digest": kernel_digest(kname),
                     "bytes_per_launch": int(round(f_split + w_split)),
                     "fetch_bytes": int(round(f_split)), "write_bytes": int(round(w_split)),
                     "fetch_raw_kib": round(f_raw / 1024, 1), "write_raw_kib": round(w_raw / 1024, 1),
                     "mfma": mfma_rec,
                     "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)}
    with open(traffic_file, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(path)
    return rec[workload]


MFMA_BF16_PEAK_TFLOPS = 2500.0


def time_calls(call, steps, warmup, torch, np, mx, stream):
    """(ms per whole call over exactly `steps` calls, mean split-kernel ms from
    HIP events recorded around it on its stream)."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t_start) * 1e3 / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for a, b in evs:
        mx.set_timing_events(a.cuda_event, b.cuda_event)
        call()
    mx.set_timing_events(None, None)
    torch.cuda.synchronize()
    return ms, float(np.mean([a.elapsed_time(b) for a, b in evs]))


def bench_varlen(args):
    """A packed (varlen) workload: attention TFLOP/s of the whole call; the
    split kernel against the dense bf16/fp16 matrix-core peak."""
    import numpy as np
    import torch

    import split_kv_decode_amd as mx
    import workloads as wl

    w = wl.VARLEN_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, cq, ck = wl.make_varlen_inputs(w)
    gq, gk, gv, gcq, gck = (t.to(dev) for t in (q, k, v, cq, ck))
    mq, mk = max(w.qlens), max(w.klens)
    dt = mx.MXFA_BF16 if w.dtype == "bf16" else mx.MXFA_FP16
    need = mx.workspace_size(w.B, w.Hq, w.Hkv, w.D, mq, mk, w.causal, dt, args.num_splits)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    out = torch.empty_like(gq)
    lse = torch.empty((w.Hq, gq.shape[0]), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        mx.fwd_varlen(gq, gk, gv, gcq, gck, mq, mk, w.causal, out=out, lse=lse,
                      num_splits=args.num_splits, workspace=ws, stream=stream.cuda_stream)

    ms, split_ms = time_calls(call, args.steps, args.warmup, torch, np, mx, stream)
    plan = mx.last_plan().as_dict()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    fl = wl.varlen_flops(w)
    tflops = fl / (ms * 1e-3) / 1e12
    split_tflops = fl / (split_ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # bounded sample: sequence 2 alone (its q chunk against its keys)
        b = 2
        sub = wl.VarlenWorkload(w.name, (w.qlens[b],), (w.klens[b],), w.Hq, w.Hkv, w.D,
                                w.dtype, w.causal, w.sigma, w.seed)
        q0, q1 = int(cq[b]), int(cq[b + 1])
        k0, k1 = int(ck[b]), int(ck[b + 1])
        threads = args.cpu_threads or len(os.sched_getaffinity(0))
        tc = time.perf_counter()
        oracle.attention_varlen(q[q0:q1], k[k0:k1], v[k0:k1],
                                [0, q1 - q0], [0, k1 - k0], q1 - q0, k1 - k0, w.causal,
                                w.dtype, nthreads=threads)
        cpu_s = time.perf_counter() - tc
        cpu = {"value": round(wl.varlen_flops(sub) / cpu_s / 1e12, 6), "unit": "TFLOP/s",
               "cores": threads, "kind": "oracle",
               "sample": (f"sequence {b} alone ({w.qlens[b]} queries x {w.klens[b]} keys, "
                          f"{wl.varlen_flops(sub) / 1e9:.1f} GFLOP, {cpu_s:.2f} s)")}
    rec = {
        "metric": "packed chunked-prefill attention TFLOP/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "qlens": list(w.qlens),
                   "klens": list(w.klens), "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "causal": w.causal, "kv_layout": "packed", "parallelism": "single GPU"},
        "gb_per_s": round(wl.varlen_bytes(w) / (ms * 1e-3) / 1e9, 2),
        "plan": plan,
        "roofline": {"bound": "mfma", "kernel": SPLIT_KERNEL[plan["path"]],
                     "achieved": round(split_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(split_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_for(w.name, SPLIT_KERNEL[plan["path"]]),
                     "flops_per_launch": fl,
                     "mean_launch_us": round(split_ms * 1e3, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # 1000 back-to-back calls (0.1-0.4 s on the long workloads): with 100 the
    # start of the timed loop (the GPU leaving idle) shows in the wall clock
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--page-size", type=int, default=0,
                    help="run on a paged copy of the cache with this page size "
                         "(0 = the contiguous cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0,
                    help="rotating copies of the inputs (0 = enough for 1 GiB of K/V, <= 64)")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the 2 GiB streaming-read probe")
    ap.add_argument("--no-dispatch-check", action="store_true",
                    help="skip the profiler count of the kernels each call dispatches "
                         "(for runs under an external profiler)")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure only the chosen workload (by default the other named "
                         "decode workloads are measured too and summarised under 'configs')")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    ap.add_argument("--summarize-profiles", nargs="+", metavar="DIR",
                    help="summarize rocprofv3 output directories TRACE FETCH WRITE [MFMA] "
                         "into profiles/ (no GPU)")
    ap.add_argument("--profile-command", action="append", default=[],
                    help="command line recorded in the profile summary")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_profiles:
        d = args.summarize_profiles
        if len(d) not in (3, 4):
            sys.exit("--summarize-profiles takes TRACE FETCH WRITE [MFMA]")
        summarize_profiles(d[0], d[1], d[2], args.workload, args.profile_command,
                           d[3] if len(d) == 4 else None, args.page_size)
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {args.gpus} is not supported "
              "(the split-KV path shards by batch or kv head with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import split_kv_decode_amd as mx
    import workloads as wl

    if args.workload in wl.VARLEN_WORKLOADS:
        bench_varlen(args)
        return
    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = measure_decode(w, args.steps, args.warmup, args.page_size, args.num_splits,
                       args.copies, torch, np, mx, wl, dev, not args.no_dispatch_check)
    ceiling = (read_ceiling(torch, mx, dev, m["stream"], m["kv"])
               if not args.no_read_ceiling else None)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    P = args.page_size
    traffic = traffic_for(f"{w.name}_paged{P}" if P else w.name, m["kernel"])
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, w, m["inp"], m["paged_cpu"], m["lens"], m["alg_bytes"])
    configs = None
    if not args.no_configs and not P and args.num_splits == 0:
        del m["inp"], m["paged_cpu"]
        configs = other_configs(w.name, args, torch, np, mx, wl, dev)
    split_gbs = m["split_gbs"]
    rec = {
        "metric": "decode attention achieved HBM GB/s (% of peak) and attn-calls/s at B x KV len",
        "value": round(m["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "qLen": w.qLen, "Hq": w.Hq, "Hkv": w.Hkv,
                   "D": w.D, "kv_cap": w.kv_cap, "sum_kv_len": int(sum(m["lens"])),
                   "causal": w.causal, "kv_layout": f"paged{P}" if P else "contiguous",
                   "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * m["gbs"] / HBM_PEAK_GBS, 2),
        # one over the median event-timed call (split + merge kernels)
        "attn_calls_per_s": round(1e3 / m["call_ms_median"], 1),
        "median_call_us": round(m["call_ms_median"] * 1e3, 2),
        "wall_calls_per_s": round(1e3 / m["ms_per_step"], 1),
        "rotating_copies": m["n_copies"],
        "plan": m["plan"],
        "dispatch_check": m["dispatch"],
        "roofline": {"bound": "hbm", "kernel": m["kernel"],
                     "achieved": round(split_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(split_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "bytes_per_launch": m["split_bytes"],
                     "mean_launch_us": round(m["split_ms_mean"] * 1e3, 2),
                     "median_launch_us": round(m["split_ms_median"] * 1e3, 2),
                     "frac_of_read_ceiling": (round(split_gbs / ceiling["nt_gbs"], 4)
                                              if ceiling else None),
                     "frac_of_size_matched_ceiling": (
                         round(split_gbs / ceiling["nt_gbs_at_workload_size"], 4)
                         if ceiling and "nt_gbs_at_workload_size" in ceiling else None)},
        "mfma_util": m["mfma_util"],
        "read_ceiling": ceiling,
        "cpu_baseline": cpu,
        "configs": configs,
    }
    print(json.dumps(rec), flush=True)


def measure_decode(w, steps, warmup, page_size, num_splits, copies, torch, np, mx, wl, dev,
                   dispatch_check=True):
    """Time one decode workload: exactly `steps` whole calls (after `warmup`)
    by the wall clock, the split kernel alone by HIP events recorded around it
    on its stream, and whole calls between event pairs; check the dispatch
    count of a few calls in a profiler trace.  Returns a dict of figures."""
    t0 = time.time()
    inp = wl.make_inputs(w)
    lens = inp.lengths()
    P = page_size
    paged_cpu = wl.to_paged(inp, P) if P else None
    paged = paged_cpu.to(dev) if P else None
    g = inp.to(dev) if not P else None
    q = inp.q.to(dev)
    print(f"# inputs {w.name} ({w.describe()}{f', pages of {P}' if P else ''}) "
          f"generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    dt = mx.MXFA_BF16 if w.dtype == "bf16" else mx.MXFA_FP16
    if P:
        need = mx.workspace_size_paged(w.B, w.Hq, w.Hkv, w.D, w.qLen, P,
                                       paged.block_table.shape[1], w.causal, dt, num_splits)
    else:
        need = mx.workspace_size(w.B, w.Hq, w.Hkv, w.D, w.qLen, w.kv_cap, w.causal, dt,
                                 num_splits)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    # rotating copies of q / K / V / out / lse (the block table and the
    # lengths are shared)
    kv = wl.kv_bytes(w, lens)
    n_copies = (copies if copies > 0
                else max(1, min(MAX_COPIES, -(-ROTATE_BYTES // max(kv, 1)))))
    k0, v0 = (paged.k_pages, paged.v_pages) if P else (g.k_cache, g.v_cache)
    sets = []
    for c in range(n_copies):
        kc, vc = (k0, v0) if c == 0 else (k0.clone(), v0.clone())
        qc = q if c == 0 else q.clone()
        sets.append((qc, kc, vc, torch.empty_like(q),
                     torch.empty((w.B, w.Hq, w.qLen), dtype=torch.float32, device=dev)))
    # each copy's call checked and marshalled once (PreparedCall); a step
    # enqueues the next copy's call
    if P:
        calls = [mx.fwd_kvcache_paged(qc, kc, vc, paged.block_table, paged.cache_seqlens,
                                      w.causal, out=oc, lse=lc, num_splits=num_splits,
                                      workspace=ws, stream=stream.cuda_stream, prepare=True)
                 for qc, kc, vc, oc, lc in sets]
    else:
        calls = [mx.fwd_kvcache(qc, kc, vc, g.cache_seqlens, w.causal, out=oc, lse=lc,
                                num_splits=num_splits, workspace=ws,
                                stream=stream.cuda_stream, prepare=True)
                 for qc, kc, vc, oc, lc in sets]
    counter = [0]

    def call():
        calls[counter[0] % n_copies].run()
        counter[0] += 1

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    plan = mx.last_plan().as_dict()

    # whole calls, wall clock over exactly `steps` calls
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / steps

    new_events = lambda: [(torch.cuda.Event(enable_timing=True),
                           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    # split kernel alone: HIP events recorded around it on its stream
    evs = new_events()
    for a, b in evs:          # create the underlying HIP events
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for a, b in evs:
        mx.set_timing_events(a.cuda_event, b.cuda_event)
        call()
    mx.set_timing_events(None, None)
    torch.cuda.synchronize()
    split_ms = [a.elapsed_time(b) for a, b in evs]
    split_ms_mean = float(np.mean(split_ms))
    # whole calls (split + merge), each between two events on the stream
    cevs = new_events()
    for a, b in cevs:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    call_ms_median = statistics.median(a.elapsed_time(b) for a, b in cevs)
    dispatch = (check_dispatch(call, plan, torch) if dispatch_check
                else {"checked": False, "reason": "--no-dispatch-check"})

    alg_bytes = wl.algorithmic_bytes(w, lens)
    q_bytes = w.B * w.qLen * w.Hq * w.D * w.elt
    # a paged cache also reads one block-table entry per page touched
    bt_bytes = sum(-(-max(0, min(n, w.kv_cap)) // P) for n in lens) * 4 if P else 0
    alg_bytes += bt_bytes
    split_bytes = kv + q_bytes + bt_bytes
    flops = wl.flops(w, lens)
    mfma_util = None
    if plan["path"] == "mfma":
        # attention flops (4 D per visible (row, key) pair) against the dense
        # matrix-core peak of the input type
        mfma_util = {"flops_per_call": flops,
                     "split_tflops": round(flops / (split_ms_mean * 1e-3) / 1e12, 2),
                     "split_frac_of_peak": round(flops / (split_ms_mean * 1e-3) / 1e12
                                                 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "call_frac_of_peak": round(flops / (ms_per_step * 1e-3) / 1e12
                                                / MFMA_BF16_PEAK_TFLOPS, 4),
                     "peak_tflops": MFMA_BF16_PEAK_TFLOPS}
    kernel = SPLIT_KERNEL[plan["path"]]
    out = {"inp": inp, "paged_cpu": paged_cpu, "lens": lens, "kv": kv, "stream": stream,
           "plan": plan, "kernel": kernel, "n_copies": n_copies,
           "ms_per_step": ms_per_step, "split_ms_mean": split_ms_mean,
           "split_ms_median": statistics.median(split_ms), "call_ms_median": call_ms_median,
           "alg_bytes": alg_bytes, "split_bytes": split_bytes,
           "gbs": alg_bytes / (ms_per_step * 1e-3) / 1e9,
           "split_gbs": split_bytes / (split_ms_mean * 1e-3) / 1e9,
           "mfma_util": mfma_util, "dispatch": dispatch}
    del calls, sets, ws, g, paged, q
    return out


DISPATCH_CALLS = 4


def check_dispatch(call, plan, torch):
    """Enqueue DISPATCH_CALLS calls under the profiler and count the kernels
    the GPU ran: each call must dispatch exactly one split kernel, plus one
    merge kernel when the plan has a merge, and nothing else.  Raises on a
    mismatch; returns the counts.  Without device events in the trace (no
    kernel tracing on this system) the check is reported as not run."""
    from torch.profiler import ProfilerActivity, profile
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        for _ in range(DISPATCH_CALLS):
            call()
        torch.cuda.synchronize()
    counts = {}
    for e in prof.events():
        dt = str(getattr(e, "device_type", ""))
        if "CUDA" in dt or "HIP" in dt:
            counts[e.name] = counts.get(e.name, 0) + 1
    if not counts:
        return {"checked": False, "reason": "the profiler recorded no device kernels"}
    split = sum(c for n, c in counts.items() if "split_kv_" in n)
    merge = sum(c for n, c in counts.items() if "combine_kernel" in n)
    other = sum(counts.values()) - split - merge
    want_merge = DISPATCH_CALLS if plan["combine"] else 0
    ok = split == DISPATCH_CALLS and merge == want_merge and other == 0
    rec = {"checked": True, "calls": DISPATCH_CALLS, "split_launches": split,
           "merge_launches": merge, "other_kernels": other, "ok": ok}
    if not ok:
        raise RuntimeError(f"dispatch check failed: {rec}; kernels {counts}")
    return rec


CONFIG_STEPS, CONFIG_WARMUP = 1000, 50


def other_configs(headline, args, torch, np, mx, wl, dev):
    """Every other named decode workload, each measured like the headline
    (its own CONFIG_STEPS calls after CONFIG_WARMUP, rotating copies, event
    timings, dispatch check) and summarised in one record."""
    recs = []
    for name, w in wl.WORKLOADS.items():
        if name == headline:
            continue
        m = measure_decode(w, CONFIG_STEPS, CONFIG_WARMUP, 0, 0, 0, torch, np, mx, wl, dev,
                           not args.no_dispatch_check)
        gbs = m["gbs"]
        ceil_gbs = None
        if not args.no_read_ceiling:
            c = read_ceiling(torch, mx, dev, m["stream"], m["kv"], full=False)
            ceil_gbs = c.get("nt_gbs_at_workload_size")
        recs.append({
            "workload": name, "B": w.B, "qLen": w.qLen, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
            "kv_cap": w.kv_cap, "sum_kv_len": int(sum(m["lens"])), "dtype": w.dtype,
            "causal": w.causal, "steps": CONFIG_STEPS, "warmup": CONFIG_WARMUP,
            "wall_us_per_call": round(m["ms_per_step"] * 1e3, 2),
            "median_call_us": round(m["call_ms_median"] * 1e3, 2),
            "gb_per_s": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "attn_calls_per_s": round(1e3 / m["call_ms_median"], 1),
            "rotating_copies": m["n_copies"],
            "path": m["plan"]["path"], "combine": m["plan"]["combine"],
            "split": {"kernel": m["kernel"], "mean_launch_us": round(m["split_ms_mean"] * 1e3, 2),
                      "gb_per_s": round(m["split_gbs"], 1),
                      "frac": round(m["split_gbs"] / HBM_PEAK_GBS, 4),
                      # the read probe over reads of this workload's K/V size
                      "size_matched_ceiling_gbs": ceil_gbs,
                      "frac_of_size_matched_ceiling": (round(m["split_gbs"] / ceil_gbs, 4)
                                                       if ceil_gbs else None)},
            "mfma_util": m["mfma_util"], "dispatch_check": m["dispatch"]})
        print(f"# {name}: {recs[-1]['wall_us_per_call']} us/call, "
              f"{recs[-1]['pct_of_hbm_peak']}% of peak", file=sys.stderr, flush=True)
        del m
        torch.cuda.empty_cache()
    return recs


ROTATE_BYTES = 1 << 30
MAX_COPIES = 64
READ_PROBE_BYTES = 1 << 31


def read_ceiling(torch, mx, dev, stream, size_bytes=0, reps=10, full=True):
    """Median rate of the library's streaming-read probe over 2 GiB, with the
    attention kernels' nt load policy and with the default policy (full=True);
    and, when size_bytes is given (the workload's K/V bytes), with the nt
    policy over reads of that size taken from consecutive windows of the 2 GiB
    buffer (so that no read finds its bytes in the last-level cache): the
    ceiling at the workload's own size, where the ramp and tail of one pass
    weigh more."""
    src = torch.ones(READ_PROBE_BYTES, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = {"kernel": "read_probe_kernel", "bytes": READ_PROBE_BYTES}

    def median_ms(views, nt):
        for v in views[:3]:
            mx.read_probe(v, nt, sink, cus, stream.cuda_stream)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for k, (a, b) in enumerate(evs):
            a.record(stream)
            mx.read_probe(views[k % len(views)], nt, sink, cus, stream.cuda_stream)
            b.record(stream)
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in evs)

    for nt in ((True, False) if full else ()):
        ms = median_ms([src], nt)
        out["nt_gbs" if nt else "default_gbs"] = round(READ_PROBE_BYTES / (ms * 1e-3) / 1e9, 1)
    size = min(int(size_bytes) // 16 * 16, READ_PROBE_BYTES)
    if size >= 1 << 20:
        n = READ_PROBE_BYTES // size
        views = [src[k * size:(k + 1) * size] for k in range(n)]
        ms = median_ms(views, True)
        out["workload_bytes"] = size
        out["nt_gbs_at_workload_size"] = round(size / (ms * 1e-3) / 1e9, 1)
    del src
    return out


def time_oracle(fn, runs=3, long_s=5.0):
    """Median wall time of up to `runs` calls (one if the first takes longer
    than long_s seconds)."""
    ts = []
    for _ in range(runs):
        t = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t)
        if ts[0] > long_s:
            break
    return statistics.median(ts), len(ts)


ONE_THREAD_SECONDS = 4.0


def cpu_baseline(args, w, inp, paged_cpu, lens, alg_bytes):
    """The fp64 oracle on this host: the whole batch with every core this
    process may use (median of up to 3 runs), and one thread on a leading
    part of the batch sized to about ONE_THREAD_SECONDS of work."""
    import oracle
    import workloads as wl
    threads = args.cpu_threads or len(os.sched_getaffinity(0))
    if paged_cpu is not None:
        whole = lambda: oracle.attention_paged(inp.q, paged_cpu.k_pages, paged_cpu.v_pages,
                                               paged_cpu.block_table, paged_cpu.cache_seqlens,
                                               w.causal, w.dtype, nthreads=threads)
    else:
        whole = lambda: oracle.attention(inp.q, inp.k_cache, inp.v_cache, inp.cache_seqlens,
                                         w.causal, w.dtype, nthreads=threads)
    cpu_s, runs = time_oracle(whole)
    # one thread on about 4 s of work: the first k sequences, and of those the
    # first nh kv heads (with their query heads) when one sequence is too much
    frac = min(1.0, ONE_THREAD_SECONDS / max(cpu_s * threads, 1e-9))
    total = sum(max(0, min(n, w.kv_cap)) for n in lens)
    k, acc = 0, 0
    while k < w.B and (k == 0 or acc < frac * total):
        acc += max(0, min(lens[k], w.kv_cap))
        k += 1
    nh = w.Hkv if acc == 0 else max(1, min(w.Hkv, -(-int(w.Hkv * frac * total) // acc)))
    G = w.Hq // w.Hkv
    sl = None if inp.cache_seqlens is None else inp.cache_seqlens[:k]
    sub = wl.Workload(w.name, B=k, qLen=w.qLen, Hq=nh * G, Hkv=nh, D=w.D, kv_cap=w.kv_cap,
                      dtype=w.dtype, causal=w.causal, sigma=w.sigma, seed=w.seed,
                      len_range=w.len_range)
    sub_bytes = wl.algorithmic_bytes(sub, lens[:k])
    q1 = inp.q[:k, :, :nh * G].contiguous()
    k1 = inp.k_cache[:k, :, :nh].contiguous()
    v1 = inp.v_cache[:k, :, :nh].contiguous()
    one_s, one_runs = time_oracle(lambda: oracle.attention(q1, k1, v1, sl, w.causal, w.dtype,
                                                           nthreads=1))
    return {"value": round(alg_bytes / cpu_s / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"the whole {w.name} batch, one call per run, median of {runs} "
                       f"({cpu_s:.2f} s; {alg_bytes / 1e9:.3f} GB algorithmic)"),
            "one_thread": {"value": round(sub_bytes / one_s / 1e9, 4), "unit": "GB/s",
                           "sample": (f"sequences 0..{k - 1} of the batch, kv heads "
                                      f"0..{nh - 1} (with their query heads), contiguous "
                                      f"cache, median of {one_runs} ({one_s:.2f} s; "
                                      f"{sub_bytes / 1e9:.3f} GB algorithmic)")}}


if __name__ == "__main__":
    main()
