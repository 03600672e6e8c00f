#!/usr/bin/env python3
"""Write the oracle's reward for every request of every workload stream.

Imports only ``oracle`` (the plain float64 forward, one sequence at a time)
and ``synth`` (the seeded inputs); nothing from the GPU library.  The files
are the expected values of the full-size parity tests, which compare every
reward the GPU returns for a stream against them.

Output, one file per stream under tests/golden/:
  stream_rewards_<name>.npy   float64[n], request (arrival) order, offset 0
  stream_rewards_<name>.json  provenance: command, precision, seeds, count

Streams:
  tiny_fp32           the 8-request stream
  tinybert_b64_n{64,128,256}  the fixed-length batches of 64
  bert_base_short     2000 requests U{2..100}
  bert_base_longtail  1800 x U{5..500} + 200 x U{400..500}
  decoder_rm          64 prompts x 16 candidates (1024 sequences of 520-560)

Long runs checkpoint every few sequences to ``<file>.partial.npy`` and resume
from it, so an interrupted decoder run (about an hour or more of CPU in
float64) loses little.

    python tests/golden/make_stream_rewards.py [--dtype float64] [name ...]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synth import get_config, make_fixed_batch, make_requests, make_weights  # noqa: E402
from synth.generate import split  # noqa: E402

STREAMS = ["tiny_fp32", "tinybert_b64_n64", "tinybert_b64_n128", "tinybert_b64_n256",
           "bert_base_short", "bert_base_longtail", "decoder_rm"]


def stream_inputs(name):
    """(config, ids, lengths, how) for a named stream."""
    if name.startswith("tinybert_b64_n"):
        cfg = get_config("tinybert")
        n = int(name.rsplit("n", 1)[1])
        ids, lengths = make_fixed_batch(cfg, n, 64)
        return cfg, ids, lengths, f"make_fixed_batch(tinybert, {n}, 64)"
    cfg = get_config(name)
    ids, lengths, _ = make_requests(cfg)
    return cfg, ids, lengths, f"make_requests({name})"


def run(name, dtype, checkpoint_every=16):
    cfg, ids, lengths, how = stream_inputs(name)
    out = os.path.join(HERE, f"stream_rewards_{name}.npy")
    part = out[:-4] + ".partial.npy"
    seqs = split(ids, lengths)
    done = np.load(part) if os.path.exists(part) else np.zeros(0)
    rew = np.full(len(seqs), np.nan)
    rew[:done.size] = done
    print(f"[golden] {name}: {len(seqs)} sequences, {int(lengths.sum())} tokens, "
          f"resuming at {done.size}", flush=True)
    m = oracle.OracleModel(cfg, make_weights(cfg), dtype=dtype)
    t0 = time.time()
    for i in range(done.size, len(seqs)):
        rew[i] = m.score(seqs[i], 0.0)
        if (i + 1) % checkpoint_every == 0 or i + 1 == len(seqs):
            np.save(part, rew[:i + 1])
            el = time.time() - t0
            print(f"[golden] {name}: {i + 1}/{len(seqs)} done, {el:.0f} s", flush=True)
    np.save(out, rew)
    os.remove(part)
    meta = {
        "stream": name,
        "inputs": how,
        "seeds": cfg.seeds,
        "requests": int(lengths.size),
        "tokens": int(lengths.sum()),
        "precision": np.dtype(dtype).name,
        "reward_offset": 0.0,
        "order": "request (arrival) order",
        "command": "python tests/golden/make_stream_rewards.py " + name,
        "computed_by": "oracle.OracleModel.score, one sequence at a time",
    }
    with open(out[:-4] + ".json", "w") as f:
        json.dump(meta, f, indent=1)
        f.write("\n")
    print(f"[golden] {name}: wrote {out}", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("names", nargs="*", default=STREAMS)
    ap.add_argument("--dtype", default="float64", choices=["float64", "float32"])
    a = ap.parse_args()
    for n in a.names:
        if n not in STREAMS:
            raise SystemExit(f"unknown stream {n!r}; known: {STREAMS}")
        run(n, np.dtype(a.dtype))


if __name__ == "__main__":
    main()
