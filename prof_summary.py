#!/usr/bin/env python3
"""Turn rocprofv3 CSV output of a bench.py run into the short text summaries
kept under profiles/.

    python prof_summary.py kernels STATS_CSV --command CMD [--title T] [--top N]
    python prof_summary.py traffic --fetch CSV --write CSV --probe-fetch CSV --probe-write CSV
                                   --probe-mib MIB --kernel-class CLASS --command CMD...
    python prof_summary.py calls TRACE_CSV --bench-json JSON --command CMD [--title T]
    python prof_summary.py rowbench --json JSON --dir DIR --workload W --launches N --probe-mib MIB

`kernels` reads `<prefix>_kernel_stats.csv` (rocprofv3 --kernel-trace --stats)
and prints the per-kernel table plus, for every GEMM class, the calls-weighted
average launch duration over the kernels of that class (the tile is chosen per
pass size, so a class can span several kernels).

`calls` reads `<prefix>_kernel_trace.csv` of bench.py --fixed-length-only
(tinybert) and splits the library's dispatches into es_score_batch calls at
each embedding kernel: per shape (200 timed calls after 10 warm-up calls,
shapes in bench.py's order) the kernels per call, the median summed kernel
time and the median per-kernel time, next to the plain run's wall clock.

`rowbench` combines rowbench.py's JSON line (event-timed launches, warm and
cold) with four --pmc runs of rowbench.py (FETCH_SIZE / WRITE_SIZE, --mode
warm / cold, directories DIR/pmc_rb_<workload>_<mode>_<counter>) and the
copy calibration (DIR/pmc_probe_<counter>): counter bytes per launch and the
bandwidth they give over the event-timed launch.

`traffic` reads the `counter_collection.csv` files of two --pmc runs of the
same command (FETCH_SIZE, then WRITE_SIZE) and of two runs over hbm_probe.py
(a plain device copy of PROBE_MIB MiB), scales the counters by what they read
for that copy (bytes moved / counter KiB), and prints the HBM bytes per launch
of the class's kernels, with the SHA-256 of the kernel source so bench.py can
tell whether the figure still describes the current source.
"""
import argparse
import csv
import hashlib
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "encoder_scoring_amd", "csrc")

# GEMM kernel name -> epilogue id (the template argument after the tile config)
GEMM_RE = re.compile(r"gemm_\w+_kernel<[^<>]*<[^<>]*>,\s*(\d+)")
EPI_CLASS = {0: "qkv_gemm", 1: "ffn1_gemm", 2: "oproj_gemm", 3: "ffn2_gemm", 4: "ffn2_gemm"}
CLASS_PATTERNS = {  # kernel classes that are not GEMMs, by kernel name
    "softmax": r"softmax_kernel",
    "layernorm": r"layernorm_kernel",
    "attn_fused": r"attn_fused",
    "scores": r"scores_(mfma_)?kernel",
    "pv": r"pv_(mfma_)?kernel",
    "embed": r"embed_kernel",
    "refine": r"gemm_split_kernel|layernorm_split_kernel|attn_last_kernel",
}
CLASS_SOURCE = {"softmax": "rowops.hip", "layernorm": "rowops.hip", "attn_fused": "attn.hip",
                "embed": "rowops.hip"}


def short(name):
    name = name.replace("es::(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*$", "", name)                 # drop the argument list


def class_of(name):
    m = GEMM_RE.search(name)
    if m:
        return EPI_CLASS.get(int(m.group(1)))
    for cls, pat in CLASS_PATTERNS.items():
        if re.search(pat, name):
            return cls
    return None


def kernels(a):
    rows = list(csv.DictReader(open(a.stats)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    print(f"# rocprofv3 kernel-trace summary: {a.title}")
    print("# command (after `cd /tmp && export TMPDIR=/tmp`, from the repository root):")
    print(f"#   {a.command}")
    print("# columns: kernel, calls, average duration (us), total (ms), share of GPU kernel time")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    for r in rows[:a.top]:
        print(f"{short(r['Name'])[:62]:62s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:9.2f} "
              f"{float(r['TotalDurationNs']) / 1e6:9.2f} {100 * float(r['TotalDurationNs']) / total:6.1f}%")
    agg = defaultdict(lambda: [0, 0.0, []])
    for r in rows:
        c = class_of(r["Name"])
        if c:
            agg[c][0] += int(r["Calls"])
            agg[c][1] += float(r["TotalDurationNs"])
            agg[c][2].append(f"{short(r['Name'])} x{r['Calls']}")
    print()
    print("# kernel classes (calls-weighted average launch over the class's kernels):")
    for c, (calls, ns, names) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        print(f"#   {c:11s} {calls:6d} launches  avg {ns / calls / 1e3:9.2f} us  total {ns / 1e6:9.2f} ms"
              f"  [{'; '.join(names)}]")
    if a.bench_log:  # the JSON line bench.py printed under the profiler
        import json
        line = [l for l in open(a.bench_log) if l.startswith('{"metric"')][-1]
        d = json.loads(line)
        r = d["roofline"]
        cls = r["kernel"]
        print()
        print("# bench.py's roofline reading in the same run (HIP events around every launch, one pass in flight):")
        print(f"#   dominant class {cls}: avg {r['avg_launch_ms'] * 1e3:.2f} us per launch, {r['achieved']} "
              f"{r['unit']} = {100 * r['frac']:.1f}% of {r['peak']} {r['unit']}")
        if cls in agg:
            calls, ns, _ = agg[cls]
            print(f"#   rocprof class average above: {ns / calls / 1e3:.2f} us per launch")
        print(f"#   value line of that run: {d['value']} {d['unit']}, {d['ms_per_step']} ms/step "
              f"({d['config']['passes_in_flight']} pass(es) in flight)")


def calls(a):
    import json
    import statistics
    rows = sorted(csv.DictReader(open(a.trace)), key=lambda r: int(r["Dispatch_Id"]))
    per_call, cur = [], None
    for r in rows:
        if "embed_kernel" in r["Kernel_Name"]:
            cur = []
            per_call.append(cur)
        if cur is not None and "es::" in r["Kernel_Name"]:
            cur.append(r)
    walls = json.loads([l for l in open(a.bench_json) if l.startswith("{")][-1])["fixed_length_calls"]
    shapes = list(walls)
    warm, timed = 10, 200
    want = len(shapes) * (warm + timed)
    if len(per_call) < want:
        sys.exit(f"{len(per_call)} calls in the trace, expected at least {want}")
    per_call = per_call[len(per_call) - want:]  # calls made before the timed shapes (warm-up) dropped
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    print(f"# rocprofv3 kernel trace: {a.title}")
    print("# command (after `cd /tmp && export TMPDIR=/tmp`, from the repository root):")
    print(f"#   {a.command}")
    print("# per shape: 200 timed calls (after 10 warm-up calls) split at each embedding kernel; medians over")
    print("# the calls; the library's kernels only.  'wall clock' = bench.py's fixed_length_calls figure of the")
    print("# same command run plainly (host-synchronised call, median and 99th percentile).")
    for i, shape in enumerate(shapes):
        cs = per_call[i * (warm + timed) + warm:(i + 1) * (warm + timed)]
        ksum = statistics.median(sum(dur(r) for r in c) for c in cs)
        w = walls[shape]
        print()
        print(f"{shape}: {statistics.median(len(c) for c in cs):.0f} kernels per call, kernel sum {ksum:.1f} us; "
              f"wall clock {w['ms_median'] * 1e3:.1f} us (p99 {w['ms_p99'] * 1e3:.1f} us) per call")
        agg = defaultdict(list)
        for c in cs:
            d = defaultdict(float)
            for r in c:
                d[short(r["Kernel_Name"])] += dur(r)
            for k, v in d.items():
                agg[k].append(v)
        for k, v in sorted(agg.items(), key=lambda kv: -statistics.median(kv[1])):
            n = statistics.median(sum(1 for r in c if short(r["Kernel_Name"]) == k) for c in cs[:5])
            print(f"  {k[:64]:64s} {n:3.0f} per call  {statistics.median(v):8.2f} us per call")


def rowbench(a):
    import json
    rb = json.loads([l for l in open(a.json) if l.startswith("{")][-1])
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        n, kib = counter_kib(os.path.join(a.dir, f"pmc_probe_{c}", "p_counter_collection.csv"), r"copyBuffer")
        cal[c] = a.probe_mib * 1024.0 / (kib / n)
    ps = rb["pass"]
    print(f"# Softmax and LayerNorm on one pass of {a.workload} ({ps['sequences']} sequences, {ps['tokens']} tokens, "
          f"{ps['heads']} heads, {'causal' if ps['causal'] else 'bidirectional'}), warm and cold cache")
    print("# commands (after `cd /tmp && export TMPDIR=/tmp`, from the repository root):")
    print(f"#   python3 rowbench.py --workload {a.workload}")
    print(f"#   rocprofv3 --pmc {{FETCH_SIZE|WRITE_SIZE}} --output-format csv -d <dir> -o p -- python3 rowbench.py "
          f"--workload {a.workload} --mode {{warm|cold}} --reps 10")
    print("#   rocprofv3 --pmc {FETCH_SIZE|WRITE_SIZE} --output-format csv -d <dir> -o p -- python3 hbm_probe.py 256 5")
    print(f"# cold: {rb['flush_mib_between_cold_launches']} MiB device copy between launches (the MALL holds 256 MB);"
          f" counter scale from the copy: FETCH_SIZE x {cal['FETCH_SIZE']:.4f}, WRITE_SIZE x {cal['WRITE_SIZE']:.4f}")
    print("# columns: kernel, mode, event-timed launch (us), algorithmic GB/s, counter bytes per launch (MB), counter GB/s")
    pats = {"softmax": CLASS_PATTERNS["softmax"], "layernorm": CLASS_PATTERNS["layernorm"]}
    for k in ("softmax", "layernorm"):
        alg = rb[k]["algorithmic_bytes_per_launch"]
        print(f"{k}: {rb[k]['form']}; algorithmic {alg / 1e6:.1f} MB per launch")
        for mode in ("warm", "cold"):
            tot = 0.0
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                _, kib = counter_kib(os.path.join(a.dir, f"pmc_rb_{a.workload}_{mode}_{c}", "p_counter_collection.csv"),
                                     pats[k])
                tot += kib * 1024.0 * cal[c] / a.launches
            ms = rb[k][mode]["ms_median"]
            print(f"  {k:9s} {mode}: {ms * 1e3:8.1f} us  {alg / ms / 1e6:7.1f} GB/s algorithmic  "
                  f"{tot / 1e6:8.1f} MB  {tot / ms / 1e6:7.1f} GB/s by counters")


def counter_kib(path, pattern):
    """(dispatches, summed counter value) of the kernels whose name matches."""
    disp = set()
    total = 0.0
    for r in csv.DictReader(open(path)):
        if re.search(pattern, r["Kernel_Name"]):
            disp.add(r["Dispatch_Id"])
            total += float(r["Counter_Value"])
    return len(disp), total


def traffic(a):
    cls = a.kernel_class
    if cls in CLASS_PATTERNS:
        pattern = CLASS_PATTERNS[cls]
    else:  # a GEMM class: every epilogue id mapping to it
        ids = [str(e) for e, c in EPI_CLASS.items() if c == cls]
        pattern = r"gemm_\w+_kernel<[^<>]*<[^<>]*>,\s*(" + "|".join(ids) + r")\b"
    src = CLASS_SOURCE.get(cls, "gemm.hip")
    nf, fetch = counter_kib(a.fetch, pattern)
    nw, write = counter_kib(a.write, pattern)
    if nf == 0 or nf != nw:
        sys.exit(f"dispatch counts differ or are zero: FETCH {nf}, WRITE {nw}")
    pf_n, pf = counter_kib(a.probe_fetch, r"copyBuffer")
    pw_n, pw = counter_kib(a.probe_write, r"copyBuffer")
    moved_kib = a.probe_mib * 1024.0
    fs = moved_kib / (pf / pf_n)
    ws = moved_kib / (pw / pw_n)
    per = (fetch / nf * fs + write / nw * ws) * 1024.0 * a.dispatches_per_launch
    sha = hashlib.sha256(open(os.path.join(CSRC, src), "rb").read()).hexdigest()
    print(f"# HBM traffic of the {cls} kernels on {a.workload}, from rocprofv3 --pmc (one counter per run)")
    print("# commands (after `cd /tmp && export TMPDIR=/tmp`, from the repository root):")
    for c in a.command:
        print(f"#   {c}")
    print(f"# kernels matching /{pattern}/; calibration: a {a.probe_mib} MiB device copy reads "
          f"FETCH_SIZE {pf / pf_n:.0f} KiB and WRITE_SIZE {pw / pw_n:.0f} KiB per dispatch, so")
    print(f"#   bytes = FETCH_SIZE * 1024 * {fs:.4f} + WRITE_SIZE * 1024 * {ws:.4f}")
    print(f"dispatches: {nf}")
    print(f"fetch_kib_per_dispatch: {fetch / nf:.1f}")
    print(f"write_kib_per_dispatch: {write / nw:.1f}")
    print(f"fetch_scale: {fs:.4f}")
    print(f"write_scale: {ws:.4f}")
    if a.dispatches_per_launch != 1:
        print(f"# one launch of the class is {a.dispatches_per_launch} kernel dispatches "
              f"(bytes per launch = per-dispatch average x {a.dispatches_per_launch})")
    print(f"hbm_bytes_per_launch: {per:.0f}")
    print(f"source_file: {src}")
    print(f"source_sha256: {sha}")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("stats")
    k.add_argument("--command", required=True)
    k.add_argument("--title", default="")
    k.add_argument("--top", type=int, default=24)
    k.add_argument("--bench-log", default=None, help="stdout of the profiled bench.py run")
    c = sub.add_parser("calls")
    c.add_argument("trace")
    c.add_argument("--bench-json", required=True, help="stdout of the plain bench.py run")
    c.add_argument("--command", required=True)
    c.add_argument("--title", default="")
    r = sub.add_parser("rowbench")
    r.add_argument("--json", required=True)
    r.add_argument("--dir", required=True)
    r.add_argument("--workload", required=True)
    r.add_argument("--launches", type=int, required=True, help="launches per kernel in each --pmc run")
    r.add_argument("--probe-mib", type=float, required=True)
    t = sub.add_parser("traffic")
    for f in ("fetch", "write", "probe_fetch", "probe_write"):
        t.add_argument("--" + f.replace("_", "-"), dest=f, required=True)
    t.add_argument("--probe-mib", type=float, required=True)
    t.add_argument("--kernel-class", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command", action="append", required=True)
    t.add_argument("--dispatches-per-launch", type=int, default=1,
                   help="kernel dispatches that make one launch of the class (the softmax "
                        "runs rows of more than one chunk per lane -- bidirectional rows over "
                        "512 scores, causal rows over 1024 -- as a second dispatch)")
    a = ap.parse_args()
    {"kernels": kernels, "traffic": traffic, "calls": calls, "rowbench": rowbench}[a.mode](a)


if __name__ == "__main__":
    main()
