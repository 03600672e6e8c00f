#!/usr/bin/env python3
"""Throughput of variable-length transformer scoring on one MI355X.

One step = one pass of the whole hot path over the workload's request
stream: DP batch planning, packing, embedding, every layer (QKV GEMM, masked
attention -- fused by default, or scores + row softmax + P.V --, output GEMM +
residual, LayerNorm, FFN GEMMs with fused GELU / residual, LayerNorm), the
last-token reward head and the scatter of rewards back to request order -- a
single es_score_requests call on token ids already resident in HBM (with
--best-of-n on the decoder workload: one es_score_best_of_n call, each
prompt run once for its candidates, plus the per-prompt selection).

The headline is the decoder reward model's best-of-16 stream scored as
1024 plain prompt + summary sequences (the largest workload).  Each step is
bracketed by HIP events on the stream, so the line carries the median and a
95 % t-interval of the step time next to the mean over the timed region.
The other attention form is timed on the same stream ("variants"; for the
decoder also the stream without the last-token refinement), and with
the default workload the shared-prompt form of the same stream and the two
BERT-base streams follow as "extra_workloads", each with its own step
statistics and dominant-kernel roofline.

Prints ONE JSON line (sequences/s for the whole job).  Kernel classes are
timed live with HIP events on the stream they run on (the library's
profiling hook) and reported against the MI355X peaks; the CPU oracle is
timed on a bounded sample of the headline stream on the host cores.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload decoder_rm]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# launch settings of the timed configuration, per workload (the full-size
# parity tests run the same ones): planned batches packed into one pass
# (es_set_batch_grouping) and passes overlapped on internal streams
# (es_set_concurrency).  The encoders gain from two passes in flight
# (bert_base_short 71.7 k -> 77.9 k sequences/s); the decoder's passes each
# fill the GPU with long GEMMs, and one pass at a time of seven planned
# batches runs fastest (same box: 741 sequences/s at 5 / 2, 755 at 5 / 1,
# 762 at 7 / 1).
DEFAULT_GROUP = 5
DEFAULT_IN_FLIGHT = 2
LAUNCH = {"decoder_rm": (7, 1)}
HEADLINE = "decoder_rm"


def launch_config(workload):
    """(planned batches per pass, passes in flight) timed for a workload."""
    return LAUNCH.get(workload, (DEFAULT_GROUP, DEFAULT_IN_FLIGHT))


PEAKS = {  # MI355X published peaks
    "hbm": (8000.0, "GB/s"),
    "mfma_bf16": (2500.0, "TFLOP/s"),
    "alu_fp32": (157.3, "TFLOP/s"),
}
GEMM_CLASSES = ("qkv_gemm", "oproj_gemm", "ffn1_gemm", "ffn2_gemm")
ATTN_CLASSES = ("attn_fused", "scores", "pv")
HBM_CLASSES = ("softmax", "layernorm", "embed", "head", "gather")
WORKLOAD_DESC = {
    "tiny_fp32": "2-layer fp32 encoder (hidden 128, 2 heads, FFN 512, vocab 1000); 8 requests U{2..32}",
    "tinybert": "TinyBERT-shaped bf16 encoder (4x312, 12 heads of 26, FFN 1200, vocab 30522); 64 requests of 128 tokens",
    "bert_base_short": "BERT-base-shaped bf16 encoder (12x768, 12 heads, FFN 3072, vocab 30522); 2000 requests U{2..100}; DP planner T=4096 c=1024",
    "bert_base_longtail": "BERT-base-shaped bf16 encoder; 2000 requests: 1800 U{5..500} + 200 U{400..500}; DP planner T=16384 c=1024",
    "decoder_rm": "decoder reward model bf16 (24x2048, 16 heads, FFN 8192, vocab 50257, causal, pre-LN); best-of-16 for 64 prompts of 512 + summaries U{8..48}, scored as 1024 prompt+summary sequences; DP planner T=16384 c=1024",
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def traffic_from_profiles(workload, kernel_class):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_class}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    src = os.path.join(ROOT, "encoder_scoring_amd", "csrc", kv.get("source_file", ""))
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != kv.get("source_sha256"):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        return max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1]), \
            ",".join(sorted({i.get("internal_api", "?") for i in info if i.get("user_api") == "blas"}))
    except Exception:
        return os.cpu_count() or 1, "unknown"


def cpu_baseline(cfg, weights, ids, lengths, budget_s):
    """The oracle (plain fp32 numpy forward, one sequence at a time) on the host
    cores, over the first requests of the same stream until ~budget_s."""
    import numpy as np
    import oracle
    from synth.generate import split
    seqs = split(ids, lengths)
    m = oracle.OracleModel(cfg, weights, dtype=np.float32, cache=cfg.name != "decoder_rm")
    m.score(seqs[0][:4])  # widen weights outside the timed sample
    t0 = time.perf_counter()
    done = tokens = 0
    while done < len(seqs) and time.perf_counter() - t0 < budget_s:
        m.score(seqs[done])
        tokens += len(seqs[done])
        done += 1
    dt = time.perf_counter() - t0
    threads, api = blas_threads()
    return {"value": round(done / dt, 4), "unit": "sequences/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {done} of {len(seqs)} requests ({tokens} tokens) in request order, "
                      f"numpy float32 forward one sequence at a time, {dt:.1f} s, BLAS={api}, "
                      f"host cpu_count={os.cpu_count()}",
            "tokens_per_s": round(tokens / dt, 1)}


def fixed_length_calls(sc, cfg):
    """Fixed-length batches at batch 1 (latency) and batch 64 (throughput):
    one es_score_batch call each, host-synchronised, wall clock per call,
    median and 99th percentile of 200 after 10 warm-up calls."""
    import numpy as np
    import torch
    from synth import make_fixed_batch
    latency = {}
    for seq_len in (64, 128, 256):
        for batch in (1, 64):
            fid, flen = make_fixed_batch(cfg, seq_len, batch)
            d_f = torch.from_numpy(fid).cuda()
            f_off = np.concatenate([[0], np.cumsum(flen)]).astype(np.int32)
            r_f = torch.empty(batch, dtype=torch.float32, device="cuda")
            walls = []
            for it in range(10 + 200):
                torch.cuda.synchronize()
                ta = time.perf_counter()
                sc.score(d_f, f_off, out=r_f)
                torch.cuda.synchronize()
                if it >= 10:
                    walls.append((time.perf_counter() - ta) * 1e3)
            assert torch.isfinite(r_f).all().item(), "non-finite rewards"
            med = float(np.median(walls))
            latency[f"len{seq_len}_batch{batch}"] = {
                "ms_median": round(med, 4), "ms_p99": round(float(np.percentile(walls, 99)), 4),
                "sequences_per_s": round(batch / (med / 1e3), 1)}
    return latency


def step_stats(step_ms):
    """Median, mean and a 95 % Student-t interval of the mean of per-step times."""
    import numpy as np
    a = np.asarray(step_ms, dtype=np.float64)
    k = a.size
    mean = float(a.mean())
    if k > 1:
        from scipy.stats import t as student_t
        half = float(student_t.ppf(0.975, k - 1) * a.std(ddof=1) / math.sqrt(k))
    else:
        half = float("nan")
    return {"n": k, "median": round(float(np.median(a)), 4), "mean": round(mean, 4),
            "ci95": [round(mean - half, 4), round(mean + half, 4)],
            "min": round(float(a.min()), 4), "max": round(float(a.max()), 4)}


def timed_steps(step, steps):
    """Run `steps` steps, each bracketed by HIP events on the current stream.
    Returns (wall ms of the whole region, per-step ms from the events)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return wall, [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def class_table(pc, prof_steps, bf16):
    table = {}
    for k, v in pc.items():
        if v["launches"] == 0:
            continue
        sec = v["total_ms"] / 1e3
        if k in HBM_CLASSES:
            kpeak, kunit = PEAKS["hbm"]
            ach = v["bytes"] / sec / 1e9
        else:   # GEMMs and attention contractions: flops against the MFMA peak
            kpeak, kunit = PEAKS["mfma_bf16" if bf16 else "alu_fp32"]
            ach = v["flops"] / sec / 1e12
        table[k] = {"ms_per_step": round(v["total_ms"] / prof_steps, 3),
                    "achieved": round(ach, 2), "unit": kunit, "frac": round(ach / kpeak, 4),
                    "launches_per_step": v["launches"] // prof_steps,
                    "avg_launch_us": round(v["total_ms"] * 1e3 / v["launches"], 3)}
    return table


class Workload:
    """One loaded model + request stream, and its step function."""

    def __init__(self, name, args, best_of_n=False, weights=None):
        import numpy as np
        import torch
        from encoder_scoring_amd import Scorer, blob
        from synth import get_config, make_fixed_batch, make_reference_set, make_requests, make_weights
        cfg = get_config(name)
        self.cfg, self.best_of_n = cfg, best_of_n
        self.c = cfg.batch_overhead if args.batch_overhead is None else args.batch_overhead
        t = time.perf_counter()
        self.weights = make_weights(cfg) if weights is None else weights
        group = None
        if cfg.name == "tinybert":
            ids, lengths = make_fixed_batch(cfg, 128, 64)
        else:
            ids, lengths, group = make_requests(cfg)
        self.ids, self.lengths = ids, lengths
        self.n, self.n_tokens = int(lengths.size), int(lengths.sum())
        log(f"{cfg.name}{' (shared prompts)' if best_of_n else ''}: {self.n} requests, "
            f"{self.n_tokens} tokens; weights drawn in {time.perf_counter() - t:.1f} s")
        sc = Scorer(blob.to_bytes(cfg, self.weights, 0.0), cfg.max_tokens,
                    max(1, min(cfg.max_tokens, 65536)))
        self.sc = sc
        if not args.single_step:
            rid, rlen = make_reference_set(cfg)
            d_ref = torch.from_numpy(rid).cuda()
            roff = np.concatenate([[0], np.cumsum(rlen)]).astype(np.int32)
            sc.reward_offset = sc.calibrate_offset(d_ref, roff)   # reference set averages zero
        sc.set_memory_mode(args.memory)
        per_pass, in_flight = launch_config(name)
        self.group = args.group if args.group is not None else per_pass
        self.in_flight = args.in_flight if args.in_flight is not None else in_flight
        sc.set_grouping(self.group)
        sc.set_concurrency(self.in_flight)
        self.attention = ("fused" if best_of_n else args.attention) if cfg.bf16 else "unfused"
        if cfg.bf16:
            sc.set_attention(self.attention)
        self.out = torch.empty(self.n, dtype=torch.float32, device="cuda")
        self.stats = None
        if best_of_n:
            # same requests in prompt / candidate form: prompts once, then candidates
            from synth.generate import best_of_n_form
            p_ids, pl, c_ids, cl, cn = best_of_n_form(ids, lengths, group, 512)
            self.d_ids = torch.from_numpy(np.concatenate([p_ids, c_ids])).cuda()
            self.best = torch.empty(pl.size, dtype=torch.int32, device="cuda")
            self._bon = (pl, cl, cn)
        else:
            self.d_ids = torch.from_numpy(ids).cuda()

    def step(self):
        if self.best_of_n:
            pl, cl, cn = self._bon
            _, _, self.stats = self.sc.score_best_of_n(self.d_ids, pl, cl, cn, self.c, self.out,
                                                       self.best)
        else:
            _, self.stats = self.sc.score_requests(self.d_ids, self.lengths, self.c, self.out)

    def finite(self):
        return bool(self.out.isfinite().all().item())

    def measure(self, steps, warmup):
        """Warm-up, then exactly `steps` timed steps (no profiling events)."""
        import torch
        for _ in range(max(1, warmup)):
            self.step()
        torch.cuda.synchronize()
        self.sc.memory_stats(reset=True)
        wall, per_step = timed_steps(self.step, steps)
        assert self.finite(), "non-finite rewards"
        ms = wall / steps
        return {"value": round(self.n / (ms / 1e3), 2), "ms_per_step": round(ms, 3),
                "tokens_per_s": round(self.n_tokens / (ms / 1e3), 1),
                "step_ms": step_stats(per_step)}

    def profile_name(self):
        """Name of the committed counter profiles of this stream: the shared-
        prompt form runs other passes than the plain stream, so it has its own
        (traffic_<class>_decoder_rm_best_of_n.txt)."""
        return self.cfg.name + ("_best_of_n" if self.best_of_n else "")

    def profile(self, steps):
        """Per-class kernel times: one pass in flight so each kernel runs alone,
        every launch bracketed by HIP events on the stream it runs on."""
        sc = self.sc
        sc.set_concurrency(1)
        self.step()
        sc.profile_enable(None)
        wall, _ = timed_steps(self.step, steps)
        pc = sc.profile_collect()
        sc.profile_enable([])
        sc.set_concurrency(self.in_flight)
        return pc, wall / steps

    def roofline(self, pc, prof_steps, ms_isolated):
        bf16 = self.cfg.bf16
        dominant = max((k for k in pc if pc[k]["launches"]), key=lambda k: pc[k]["total_ms"])
        dom = pc[dominant]
        launches = dom["launches"] / prof_steps
        avg_ms = dom["total_ms"] / max(1, dom["launches"])
        if dominant in HBM_CLASSES:
            key, bound = "hbm", "hbm"
            achieved = dom["bytes"] / (dom["total_ms"] / 1e3) / 1e9
        else:
            key = "mfma_bf16" if bf16 else "alu_fp32"
            bound = "mfma" if bf16 else "alu"
            achieved = dom["flops"] / (dom["total_ms"] / 1e3) / 1e12
        peak, unit = PEAKS[key]
        return {"bound": bound, "kernel": dominant, "achieved": round(achieved, 2),
                "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": traffic_from_profiles(self.profile_name(), dominant),
                "avg_launch_ms": round(avg_ms, 5), "launches_per_step": launches,
                "measured": f"HIP events around every launch over {prof_steps} steps with one "
                            f"pass in flight ({ms_isolated:.2f} ms/step)"}

    def other_attention(self, steps, warmup, prof_steps):
        """The other attention form on the same stream: its own timed steps and
        kernel table (the row-softmax kernel runs only in the unfused form)."""
        other = "unfused" if self.attention == "fused" else "fused"
        self.sc.set_attention(other)
        res = self.measure(steps, warmup)
        pc, _ = self.profile(prof_steps)
        res["kernels"] = class_table(pc, prof_steps, self.cfg.bf16)
        self.sc.set_attention(self.attention)
        return "attention_" + other, res

    def without_refinement(self, steps, warmup):
        """The same stream with the last-token refinement off (es_set_refinement):
        timed steps only, to show what the reward rows' fp32 pass costs."""
        self.sc.set_refinement(False)
        try:
            return self.measure(steps, warmup)
        finally:
            self.sc.set_refinement(True)

    def config(self, args):
        cfg, st = self.cfg, self.stats
        return {"workload": cfg.name, "description": WORKLOAD_DESC[cfg.name],
                "requests": self.n, "tokens": self.n_tokens, "batches": st["n_batches"],
                "padded_tokens": st["padded_tokens"], "max_tokens": cfg.max_tokens,
                "batch_overhead": self.c, "batches_per_pass": self.group,
                "passes_in_flight": self.in_flight, "attention": self.attention,
                "shared_prompts": self.best_of_n, "computed_tokens": st["packed_tokens"]}

    def close(self):
        self.sc.close()


def row_reductions(workload, tables):
    """The Softmax and LayerNorm row reductions' bandwidth: algorithmic bytes
    over HIP-event time, and HBM bytes from the committed rocprofv3 counter
    summary (when it describes the current source) over the same time."""
    out = {}
    for cls in ("softmax", "layernorm"):
        t = next((tb[cls] for tb in tables if cls in tb), None)
        if t is None:
            continue
        e = {"avg_launch_us": t["avg_launch_us"], "algorithmic_GBps": t["achieved"],
             "frac_algorithmic": t["frac"]}
        b = traffic_from_profiles(workload, cls)
        if b is not None:
            gbps = b / (t["avg_launch_us"] * 1e-6) / 1e9
            e.update({"counter_bytes_per_launch": b, "counter_GBps": round(gbps, 1),
                      "frac_counter": round(gbps / PEAKS["hbm"][0], 4)})
        out[cls] = e
    return out


def run_entry(w, args, steps, warmup, prof_steps, variants=True, refinement_variant=False):
    """Timed steps, kernel table, roofline and (optionally) the other attention
    form, and the stream without the last-token refinement, for one workload."""
    res = w.measure(steps, warmup)
    log(f"{w.cfg.name}{' shared prompts' if w.best_of_n else ''}: {res['value']} seq/s, "
        f"step ms {res['step_ms']}")
    pc, ms_iso = w.profile(prof_steps)
    res["kernels"] = class_table(pc, prof_steps, w.cfg.bf16)
    res["roofline"] = w.roofline(pc, prof_steps, ms_iso)
    log("isolated per-class ms/step:", {k: v["ms_per_step"] for k, v in res["kernels"].items()})
    res["variants"] = {}
    if variants and w.cfg.bf16 and not w.best_of_n:  # shared prompts always use the fused form
        k, v = w.other_attention(steps, warmup, prof_steps)
        res["variants"][k] = v
        log(f"  {k}: {v['value']} seq/s")
    if refinement_variant and w.sc.refinement():
        v = w.without_refinement(steps, warmup)
        res["variants"]["no_refinement"] = v
        log(f"  no_refinement: {v['value']} seq/s")
    res["row_reductions"] = row_reductions(
        w.profile_name(), [res["kernels"]] + [v["kernels"] for v in res["variants"].values() if "kernels" in v])
    res["config"] = w.config(args)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOAD_DESC))
    ap.add_argument("--batch-overhead", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the chosen workload only (no shared-prompt / BERT-base entries)")
    ap.add_argument("--no-variants", action="store_true",
                    help="do not time the other attention form")
    ap.add_argument("--single-step", action="store_true",
                    help="one warm-up call and one step, then exit (for counter collection)")
    ap.add_argument("--attention", default="fused", choices=["unfused", "fused"],
                    help="attention as scores + softmax row reduction + P.V, or one fused kernel")
    ap.add_argument("--in-flight", type=int, default=None,
                    help="passes overlapped on internal streams (es_set_concurrency); "
                         "default: the workload's timed configuration (launch_config)")
    ap.add_argument("--best-of-n", action="store_true",
                    help="decoder_rm only: score through es_score_best_of_n (each prompt run once "
                         "for its candidates) instead of prompt + candidate sequences")
    ap.add_argument("--group", type=int, default=None,
                    help="planned batches packed into one pass through the layers "
                         "(es_set_batch_grouping); default: the workload's timed configuration")
    ap.add_argument("--cost-model", default="linear", choices=["linear", "measured"],
                    help="planner cost of a batch: overhead + |B| * max_len, or a table measured "
                         "on this GPU before the run (es_set_cost_table)")
    ap.add_argument("--fixed-length-only", action="store_true",
                    help="tinybert only: time the fixed-length calls (lengths 64/128/256 at batch "
                         "1 and 64) and print them alone, without the stream")
    ap.add_argument("--memory", default="length_aware", choices=["length_aware", "fixed", "exact"],
                    help="workspace memory mode (es_set_memory_mode)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the scoring path is "
              "data-parallel over batches and runs one process per GPU -- run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.best_of_n and args.workload != "decoder_rm":
        sys.exit("--best-of-n applies to the decoder_rm workload (prompts shared by 16 candidates)")

    import numpy as np
    import torch

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    torch.cuda.set_device(0)
    w = Workload(args.workload, args, best_of_n=args.best_of_n)
    cfg = w.cfg
    cost_note = None
    if args.cost_model == "measured":
        if args.best_of_n:
            sys.exit("--cost-model measured applies to es_score_requests, not --best-of-n")
        from encoder_scoring_amd.costmodel import dense_cost_table, measure_cost_grid
        t = time.perf_counter()
        cap = min(cfg.max_tokens, 65536)
        bg = [b for b in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048) if b * 8 <= cap]
        lg = sorted({l for l in (8, 16, 32, 64, 128, 256, 512, 1024) if l < cfg.max_pos} | {cfg.max_pos})
        meas = measure_cost_grid(w.sc, bg, lg)
        w.sc.set_cost_table(dense_cost_table(bg, lg, meas, cfg.max_pos))
        cost_note = (f"{int(np.sum(~np.isnan(meas)))} points, batch sizes {bg[0]}..{bg[-1]} x "
                     f"lengths {lg[0]}..{lg[-1]}, measured in {time.perf_counter() - t:.1f} s "
                     "before the run")
        log("cost table: " + cost_note)
    if args.fixed_length_only:
        if cfg.name != "tinybert":
            sys.exit("--fixed-length-only applies to the tinybert workload")
        print(json.dumps({"workload": cfg.name, "fixed_length_calls": fixed_length_calls(w.sc, cfg)}),
              flush=True)
        return
    if args.single_step:
        for _ in range(2):
            w.step()
        torch.cuda.synchronize()
        print(json.dumps({"single_step": cfg.name, "finite": w.finite()}), flush=True)
        return

    prof_steps = max(2, min(args.steps, 3 if cfg.name == "decoder_rm" else 5))
    head = run_entry(w, args, args.steps, args.warmup, prof_steps, variants=not args.no_variants,
                     refinement_variant=not (args.no_variants or args.no_extras))
    mem = w.sc.memory_stats()
    w.sc.set_memory_mode("fixed")   # the workspace the fixed mode would hold for the same settings
    fixed_bytes = w.sc.memory_stats()["work_bytes"]
    w.sc.set_memory_mode(args.memory)
    latency = fixed_length_calls(w.sc, cfg) if cfg.name == "tinybert" else None
    config = head.pop("config")
    if cost_note is not None:
        config["batch_overhead"] = None
        config["cost_model"] = {"kind": "measured", "grid": cost_note}
    else:
        config["cost_model"] = args.cost_model
    line = {
        "metric": "sequences scored/sec on var-len batches",
        "value": head["value"],
        "unit": "sequences/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.bf16 else "f32",
        "data": "synthetic (seeded ids and N(0,0.02) weights of the stated shapes)",
        "config": config,
        "tokens_per_s": head["tokens_per_s"],
        "step_ms": head["step_ms"],
        "roofline": head["roofline"],
        "memory": {"mode": args.memory, "work_bytes": mem["work_bytes"],
                   "peak_work_bytes": mem["peak_work_bytes"], "fixed_mode_work_bytes": fixed_bytes,
                   "allocs_in_timed_steps": mem["allocs"],
                   "alloc_ms_in_timed_steps": round(mem["alloc_ms"], 3)},
        "kernels": head["kernels"],
        "row_reductions": head["row_reductions"],
        "variants": head["variants"],
        "fixed_length_calls": latency,
        "device": torch.cuda.get_device_name(0),
    }
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, w.weights, w.ids, w.lengths, args.cpu_seconds)
    extras = {}
    if not args.no_extras and args.workload == HEADLINE and not args.best_of_n:
        weights = w.weights
        w.close()
        del w
        torch.cuda.empty_cache()
        for name, bon in (("decoder_rm", True), ("bert_base_short", False),
                          ("bert_base_longtail", False)):
            e = Workload(name, args, best_of_n=bon, weights=weights if name == HEADLINE else None)
            key = name + ("_shared_prompts" if bon else "")
            extras[key] = run_entry(e, args, args.steps, args.warmup,
                                    max(2, min(args.steps, 5)), variants=not args.no_variants)
            e.close()
            del e
            torch.cuda.empty_cache()
        line["extra_workloads"] = extras
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
