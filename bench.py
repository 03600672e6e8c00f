#!/usr/bin/env python3
"""Throughput of variable-length transformer scoring on one MI355X.

One step = one pass of the whole hot path over the workload's request
stream: DP batch planning, packing, embedding, every layer (QKV GEMM, masked
attention -- fused by default, or scores + row softmax + P.V --, output GEMM +
residual, LayerNorm, FFN GEMMs with fused GELU / residual, LayerNorm), the
last-token reward head and the scatter of rewards back to request order -- a
single es_score_requests call on token ids already resident in HBM (with
--best-of-n on the decoder workload: one es_score_best_of_n call, each
prompt run once for its candidates, plus the per-prompt selection).  The
other attention form is timed on the same stream and reported under
"variants".

Prints ONE JSON line (sequences/s for the whole job).  The dominant kernel
class is timed live with HIP events on the stream it runs on (the library's
profiling hook) and reported against the MI355X peak; the CPU oracle is timed
on a bounded sample of the same stream on the host cores.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload bert_base_short]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAKS = {  # MI355X published peaks
    "hbm": (8000.0, "GB/s"),
    "mfma_bf16": (2500.0, "TFLOP/s"),
    "alu_fp32": (157.3, "TFLOP/s"),
}
GEMM_CLASSES = ("qkv_gemm", "oproj_gemm", "ffn1_gemm", "ffn2_gemm", "attn_fused")
HBM_CLASSES = ("softmax", "layernorm", "embed", "head", "gather")
WORKLOAD_DESC = {
    "tiny_fp32": "2-layer fp32 encoder (hidden 128, 2 heads, FFN 512, vocab 1000); 8 requests U{2..32}",
    "tinybert": "TinyBERT-shaped bf16 encoder (4x312, 12 heads of 26, FFN 1200, vocab 30522); 64 requests of 128 tokens",
    "bert_base_short": "BERT-base-shaped bf16 encoder (12x768, 12 heads, FFN 3072, vocab 30522); 2000 requests U{2..100}; DP planner T=4096 c=1024",
    "bert_base_longtail": "BERT-base-shaped bf16 encoder; 2000 requests: 1800 U{5..500} + 200 U{400..500}; DP planner T=16384 c=1024",
    "decoder_rm": "decoder reward model bf16 (24x2048, 16 heads, FFN 8192, vocab 50257, causal, pre-LN); best-of-16 for 64 prompts of 512 + summaries U{8..48}; DP planner T=16384 c=1024",
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def traffic_from_profiles(workload, kernel_class, launches_per_step):
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="bert_base_short", choices=sorted(WORKLOAD_DESC))
    ap.add_argument("--batch-overhead", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--single-step", action="store_true",
                    help="one warm-up call and one step, then exit (for counter collection)")
    ap.add_argument("--attention", default="fused", choices=["unfused", "fused"],
                    help="attention as scores + softmax row reduction + P.V, or one fused kernel")
    ap.add_argument("--in-flight", type=int, default=2,
                    help="passes overlapped on internal streams (es_set_concurrency)")
    ap.add_argument("--best-of-n", action="store_true",
                    help="decoder_rm only: score through es_score_best_of_n (each prompt run once "
                         "for its candidates) instead of prompt + candidate sequences")
    ap.add_argument("--group", type=int, default=5,
                    help="planned batches packed into one pass through the layers "
                         "(es_set_batch_grouping)")
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

    import numpy as np
    import torch
    from encoder_scoring_amd import Scorer, blob
    from synth import get_config, make_reference_set, make_requests, make_weights, make_fixed_batch

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    torch.cuda.set_device(0)
    cfg = get_config(args.workload)
    c = cfg.batch_overhead if args.batch_overhead is None else args.batch_overhead
    t = time.perf_counter()
    weights = make_weights(cfg)
    group = None
    if cfg.name == "tinybert":
        ids, lengths = make_fixed_batch(cfg, 128, 64)
    else:
        ids, lengths, group = make_requests(cfg)
    if args.best_of_n and cfg.name != "decoder_rm":
        sys.exit("--best-of-n applies to the decoder_rm workload (prompts shared by 16 candidates)")
    n, n_tokens = int(lengths.size), int(lengths.sum())
    log(f"{cfg.name}: {n} requests, {n_tokens} tokens; weights drawn in {time.perf_counter() - t:.1f} s")
    sc = Scorer(blob.to_bytes(cfg, weights, 0.0), cfg.max_tokens, max(1, min(cfg.max_tokens, 65536)))
    rid, rlen = make_reference_set(cfg)
    d_ref = torch.from_numpy(rid).cuda()
    roff = np.concatenate([[0], np.cumsum(rlen)]).astype(np.int32)
    if not args.single_step:
        sc.reward_offset = sc.calibrate_offset(d_ref, roff)   # reference set averages zero
    sc.set_memory_mode(args.memory)
    sc.set_grouping(args.group)
    sc.set_concurrency(args.in_flight)
    if cfg.bf16:
        sc.set_attention(args.attention)
    cost_note = None
    if args.cost_model == "measured":
        if args.best_of_n:
            sys.exit("--cost-model measured applies to es_score_requests, not --best-of-n")
        from encoder_scoring_amd.costmodel import dense_cost_table, measure_cost_grid
        t = time.perf_counter()
        cap = min(cfg.max_tokens, 65536)
        bg = [b for b in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048) if b * 8 <= cap]
        lg = sorted({l for l in (8, 16, 32, 64, 128, 256, 512, 1024) if l < cfg.max_pos} | {cfg.max_pos})
        meas = measure_cost_grid(sc, bg, lg)
        sc.set_cost_table(dense_cost_table(bg, lg, meas, cfg.max_pos))
        cost_note = (f"{int(np.sum(~np.isnan(meas)))} points, batch sizes {bg[0]}..{bg[-1]} x "
                     f"lengths {lg[0]}..{lg[-1]}, measured in {time.perf_counter() - t:.1f} s "
                     "before the run")
        log("cost table: " + cost_note)
    if args.fixed_length_only:
        if cfg.name != "tinybert":
            sys.exit("--fixed-length-only applies to the tinybert workload")
        print(json.dumps({"workload": cfg.name, "fixed_length_calls": fixed_length_calls(sc, cfg)}),
              flush=True)
        return
    d_ids = torch.from_numpy(ids).cuda()
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    stats = None
    if args.best_of_n:
        # same requests in prompt / candidate form: prompts once, then candidates
        from synth.generate import best_of_n_form
        p_ids, pl, c_ids, cl, cn = best_of_n_form(ids, lengths, group, 512)
        d_bon = torch.from_numpy(np.concatenate([p_ids, c_ids])).cuda()
        best = torch.empty(pl.size, dtype=torch.int32, device="cuda")

        def step():
            nonlocal stats
            _, _, stats = sc.score_best_of_n(d_bon, pl, cl, cn, c, out, best)
    else:
        def step():
            nonlocal stats
            _, stats = sc.score_requests(d_ids, lengths, c, out)

    if args.single_step:
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"single_step": cfg.name, "finite": bool(torch.isfinite(out).all().item())}))
        return
    # warm-up (also sizes the metadata buffers), then the timed region: K steps
    # of the production configuration with no profiling events
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    sc.memory_stats(reset=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    mem = sc.memory_stats()
    ms = (t1 - t0) * 1e3 / args.steps
    value = n / (ms / 1e3)
    assert torch.isfinite(out).all().item(), "non-finite rewards"

    def timed(steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    # roofline pass: one pass in flight so each kernel runs alone, every
    # kernel class bracketed by HIP events on the stream it is launched on
    prof_steps = max(2, min(args.steps, 5))

    def profile_pass():
        sc.set_concurrency(1)
        step()
        sc.profile_enable(None)
        ms_iso = timed(prof_steps)
        pc = sc.profile_collect()
        sc.profile_enable([])
        sc.set_concurrency(args.in_flight)
        return pc, ms_iso

    def class_table(pc):
        table = {}
        for k, v in pc.items():
            if v["launches"] == 0:
                continue
            sec = v["total_ms"] / 1e3
            if k in GEMM_CLASSES:
                kpeak, kunit = PEAKS["mfma_bf16" if cfg.bf16 else "alu_fp32"]
                ach = v["flops"] / sec / 1e12
            elif k in HBM_CLASSES:
                kpeak, kunit = PEAKS["hbm"]
                ach = v["bytes"] / sec / 1e9
            else:   # attention contractions: report flops against the MFMA peak
                kpeak, kunit = PEAKS["mfma_bf16" if cfg.bf16 else "alu_fp32"]
                ach = v["flops"] / sec / 1e12
            table[k] = {"ms_per_step": round(v["total_ms"] / prof_steps, 3),
                        "achieved": round(ach, 2), "unit": kunit, "frac": round(ach / kpeak, 4),
                        "launches_per_step": v["launches"] // prof_steps}
        return table

    per_class, ms_isolated = profile_pass()
    dominant = max(per_class, key=lambda k: per_class[k]["total_ms"])
    dom = per_class[dominant]
    log("isolated per-class ms/step:", {k: round(v["total_ms"] / prof_steps, 3)
                                        for k, v in per_class.items()})

    launches = dom["launches"] / prof_steps
    avg_ms = dom["total_ms"] / max(1, dom["launches"])
    if dominant in GEMM_CLASSES:
        key = "mfma_bf16" if cfg.bf16 else "alu_fp32"
        bound = "mfma" if cfg.bf16 else "alu"
        achieved = dom["flops"] / (dom["total_ms"] / 1e3) / 1e12
    else:
        key, bound = "hbm", "hbm"
        achieved = dom["bytes"] / (dom["total_ms"] / 1e3) / 1e9
    peak, unit = PEAKS[key]
    traffic = traffic_from_profiles(cfg.name, dominant, launches)
    kernels = class_table(per_class)

    # the other attention form, same stream and settings: its own timed steps
    # and kernel table (the row-softmax kernel runs only in the unfused form)
    variants = {}
    if cfg.bf16 and not args.best_of_n:  # shared prompts always use the fused attention
        other = "unfused" if args.attention == "fused" else "fused"
        sc.set_attention(other)
        step()
        ms_other = timed(args.steps)
        assert torch.isfinite(out).all().item(), "non-finite rewards"
        pc_other, _ = profile_pass()
        variants["attention_" + other] = {"value": round(n / (ms_other / 1e3), 2),
                                          "ms_per_step": round(ms_other, 3),
                                          "kernels": class_table(pc_other)}
        sc.set_attention(args.attention)

    latency = fixed_length_calls(sc, cfg) if cfg.name == "tinybert" else None

    # the workspace the fixed mode would hold for the same settings
    sc.set_memory_mode("fixed")
    fixed_bytes = sc.memory_stats()["work_bytes"]
    line_mem = {"mode": args.memory, "work_bytes": mem["work_bytes"],
                "peak_work_bytes": mem["peak_work_bytes"], "fixed_mode_work_bytes": fixed_bytes,
                "allocs_in_timed_steps": mem["allocs"], "alloc_ms_in_timed_steps": round(mem["alloc_ms"], 3)}
    line = {
        "metric": "sequences scored/sec on var-len batches",
        "value": round(value, 2),
        "unit": "sequences/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.bf16 else "f32",
        "data": "synthetic (seeded ids and N(0,0.02) weights of the stated shapes)",
        "config": {"workload": cfg.name, "description": WORKLOAD_DESC[cfg.name],
                   "requests": n, "tokens": n_tokens, "batches": stats["n_batches"],
                   "padded_tokens": stats["padded_tokens"], "max_tokens": cfg.max_tokens,
                   "batch_overhead": c if cost_note is None else None,
                   "cost_model": args.cost_model if cost_note is None else
                   {"kind": "measured", "grid": cost_note},
                   "batches_per_pass": args.group,
                   "passes_in_flight": args.in_flight,
                   "attention": ("fused" if args.best_of_n else args.attention) if cfg.bf16 else "unfused",
                   "shared_prompts": bool(args.best_of_n),
                   "computed_tokens": stats["packed_tokens"]},
        "tokens_per_s": round(n_tokens / (ms / 1e3), 1),
        "roofline": {"bound": bound, "kernel": dominant, "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic, "avg_launch_ms": round(avg_ms, 5),
                     "launches_per_step": launches,
                     "measured": f"HIP events around every launch over {prof_steps} steps with one "
                                 f"pass in flight ({ms_isolated:.2f} ms/step)"},
        "memory": line_mem,
        "kernels": kernels,
        "variants": variants,
        "fixed_length_calls": latency,
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, weights, ids, lengths, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
