#!/usr/bin/env python3
"""Warm and cold-cache timing of the two row reductions (Softmax, LayerNorm)
on one pass of a workload's planned stream.

    python rowbench.py [--workload decoder_rm] [--reps 20] [--mode both|warm|cold]

The pass: the DP plan of the workload's request stream split, as the
library splits it, into ceil(nb / G) passes of as equal a planned-batch count
as possible (G from bench.py's timed configuration of the workload), and of
those the one with the most
visible score pairs (the plan is sorted by length, so that is the pass of
the longest sequences: the one that dominates the Softmax's time).
Softmax runs es_op_softmax over that pass's ragged score layout (causal or
bidirectional as the model), fp32 scores in, bf16 probabilities out; LayerNorm runs the form the model uses after its
attention-out GEMM (pre-LN: x -> bf16 GEMM input; post-LN: x + residual ->
fp32 and bf16 outputs) on the pass's tokens.

"warm" launches run back to back, so a launch finds much of its input in the
256 MB Infinity Cache (MALL) that the previous one left there; "cold" puts a
1 GiB device copy between launches (4x the MALL), so each launch reads its
input from HBM.  Each launch is bracketed by HIP events on its stream.  One
JSON line: per kernel the algorithmic bytes per launch (the library's own
accounting: (4 + 2) bytes per visible score; T x H x (4 + 2) or
(4 + 4 + 4 + 2) for LayerNorm) and the median launch time and bandwidth in
each mode.  Under rocprofv3 --pmc, --mode warm / --mode cold give the
counter bytes of each mode on their own.
"""
import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FLUSH_MIB = 1024   # bytes copied between cold launches (4x the 256 MB MALL)


def pass_lengths(cfg):
    import numpy as np
    from encoder_scoring_amd import plan_batches
    from synth import make_requests
    _, lengths, _ = make_requests(cfg)
    order, starts, _ = plan_batches(lengths, cfg.max_tokens, cfg.batch_overhead)
    nb = len(starts) - 1
    from bench import launch_config
    group = launch_config(cfg.name)[0]
    groups = np.array_split(np.arange(nb), -(-nb // group))
    srt = np.asarray(lengths)[order]

    def pairs(ls):
        return sum(n * (n + 1) // 2 if cfg.causal else n * n for n in ls.tolist())
    best = max(groups, key=lambda g: pairs(srt[starts[g[0]]:starts[g[-1] + 1]]))
    return srt[starts[best[0]]:starts[best[-1] + 1]], len(best)


def timed(torch, launch, reps, flush):
    """Median launch time (ms) over reps launches, each bracketed by events."""
    import numpy as np
    times = []
    for i in range(reps + 2):
        if flush is not None:
            flush[1].copy_(flush[0])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        launch()
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            times.append(e0.elapsed_time(e1))
    return float(np.median(times))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="decoder_rm")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--mode", choices=("both", "warm", "cold"), default="both")
    a = ap.parse_args()
    import numpy as np
    import torch
    from encoder_scoring_amd import RaggedScores, layernorm, softmax_ragged
    from synth import get_config
    cfg = get_config(a.workload)
    lens, n_batches = pass_lengths(cfg)
    T, H = int(lens.sum()), cfg.hidden
    g = torch.Generator(device="cuda").manual_seed(7)
    flush = None
    if a.mode != "warm":
        n = FLUSH_MIB * (1 << 20) // 4
        flush = (torch.ones(n, dtype=torch.float32, device="cuda"), torch.empty(n, dtype=torch.float32, device="cuda"))
    modes = ("warm", "cold") if a.mode == "both" else (a.mode,)

    rag = RaggedScores(lens, cfg.n_heads, cfg.causal)
    s = torch.randn(rag.n_elems, device="cuda", dtype=torch.float32, generator=g)
    p = torch.empty(rag.n_elems, device="cuda", dtype=torch.int16)
    pairs = int(sum(cfg.n_heads * (n * (n + 1) // 2 if cfg.causal else n * n) for n in lens.tolist()))
    sm_bytes = 6.0 * pairs

    Hp = (H + 63) // 64 * 64
    x = torch.randn((T, H), device="cuda", dtype=torch.float32, generator=g)
    gam = 1.0 + 0.02 * torch.randn(H, device="cuda", dtype=torch.float32, generator=g)
    bet = 0.02 * torch.randn(H, device="cuda", dtype=torch.float32, generator=g)
    xb = torch.zeros((T, Hp), device="cuda", dtype=torch.int16)
    if cfg.pre_ln:
        ln = lambda: layernorm(x, gam, bet, cfg.eps, ybf16=xb)
        ln_bytes = T * H * (4.0 + 2.0)
        ln_form = "pre-LN: x -> bf16 GEMM input"
    else:
        sub = torch.randn((T, H), device="cuda", dtype=torch.float32, generator=g)
        y = torch.empty((T, H), device="cuda", dtype=torch.float32)
        ln = lambda: layernorm(x, gam, bet, cfg.eps, y=y, ybf16=xb, sub=sub)
        ln_bytes = T * H * (4.0 + 4.0 + 4.0 + 2.0)
        ln_form = "post-LN: x + residual -> fp32 and bf16"

    out = {"workload": a.workload, "pass": {"sequences": int(lens.size), "tokens": T,
                                            "planned_batches": n_batches, "heads": cfg.n_heads,
                                            "causal": bool(cfg.causal)},
           "flush_mib_between_cold_launches": FLUSH_MIB if flush is not None else 0}
    for name, launch, nbytes, form in (
            ("softmax", lambda: softmax_ragged(rag, s, p), sm_bytes, "fp32 scores -> bf16 probabilities"),
            ("layernorm", ln, ln_bytes, ln_form)):
        r = {"form": form, "algorithmic_bytes_per_launch": nbytes}
        for m in modes:
            ms = timed(torch, launch, a.reps, flush if m == "cold" else None)
            r[m] = {"ms_median": round(ms, 4), "GB_per_s": round(nbytes / ms / 1e6, 1)}
        out[name] = r
    rag.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
