"""Exercise the host-only library under AddressSanitizer / UBSan.

Run by tests/test_host_sanitizers.py in a child process with the sanitizer
runtime preloaded (python itself is not instrumented):
    python tests/host_sanitized_driver.py LIBPATH
Drives the planner (every workload's stream, random streams, the measured
cost table), offset packing, the arena planner, the pass metadata builder and
its checker (every workload, grouping, shared prompts) and the blob parser
(valid and corrupted blobs); exits 0 when every call behaved.
"""
import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from encoder_scoring_amd import _lib, blob  # noqa: E402
from encoder_scoring_amd.api import check_plan, pack_offsets, plan_arena, plan_batches, plan_batches_measured  # noqa: E402
from encoder_scoring_amd._lib import EncScoreError  # noqa: E402
from synth import get_config, make_requests, make_weights  # noqa: E402
from synth.configs import ORDERED  # noqa: E402
from synth.generate import best_of_n_form  # noqa: E402


def main(path):
    lib = _lib.load_host(path)
    rng = np.random.default_rng(5)
    calls = 0
    for name in ORDERED:
        cfg = get_config(name)
        _, lengths, group = make_requests(cfg)
        order, starts, _ = plan_batches(lengths, cfg.max_tokens, cfg.batch_overhead, lib=lib)
        for b in range(len(starts) - 1):
            pack_offsets(lengths, order, starts[b], starts[b + 1], lib=lib)
        for g in (1, 5):
            check_plan(lengths, cfg.n_heads, cfg.causal, cfg.max_pos, cfg.max_tokens,
                       min(cfg.max_tokens, 65536), cfg.batch_overhead, g, lib=lib)
            calls += 1
        if name == "decoder_rm":
            _, pl, _, cl, cn = best_of_n_form(np.zeros(int(lengths.sum()), np.int32), lengths, group, 512)
            check_plan(cl, cfg.n_heads, True, cfg.max_pos, cfg.max_tokens, min(cfg.max_tokens, 65536),
                       cfg.batch_overhead, 5, prompt_lengths=pl, cand_counts=cn, lib=lib)
    for _ in range(200):
        n = int(rng.integers(1, 40))
        lengths = rng.integers(1, 70, size=n)
        T = int(rng.integers(70, 400))
        plan_batches(lengths, T, int(rng.integers(0, 50)), lib=lib)
        table = np.cumsum(rng.integers(0, 5, size=(8, 80)), axis=1)
        try:
            plan_batches_measured(lengths, T, table, lib=lib)
        except EncScoreError:
            pass
        A = int(rng.integers(1, 5))
        check_plan(lengths, A, bool(rng.integers(0, 2)), 80, T, 64, 16, int(rng.integers(1, 4)), lib=lib)
        k = int(rng.integers(0, 12))
        first = rng.integers(0, 6, size=k)
        plan_arena(rng.integers(0, 5000, size=k), first, first + rng.integers(0, 4, size=k), 64, lib=lib)
        calls += 3
    for bad in ([0, 3], [5000], [-1]):  # error paths
        try:
            check_plan(np.array(bad), 2, 1, 64, 128, 8, 4, 1, lib=lib)
        except EncScoreError:
            pass
    cfg = get_config("tiny_fp32")
    data = bytearray(blob.to_bytes(cfg, make_weights(cfg), 0.5))
    info = _lib.ModelInfo()
    buf = ctypes.create_string_buffer(bytes(data), len(data))
    assert lib.es_blob_info(ctypes.cast(buf, ctypes.c_void_p), len(data), ctypes.byref(info)) == 0
    assert info.hidden == cfg.hidden and info.n_layers == cfg.n_layers
    for cut in (0, 10, 64, 65, len(data) // 2, len(data) - 4):
        short = ctypes.create_string_buffer(bytes(data[:cut]), max(cut, 1))
        assert lib.es_blob_info(ctypes.cast(short, ctypes.c_void_p), cut, ctypes.byref(info)) != 0
    long_ = ctypes.create_string_buffer(bytes(data) + b"\0" * 8, len(data) + 8)
    assert lib.es_blob_info(ctypes.cast(long_, ctypes.c_void_p), len(data) + 8, ctypes.byref(info)) != 0
    for field in range(4, 64, 4):  # every header word set to garbage
        d = bytearray(data)
        d[field:field + 4] = b"\xff\xff\xff\x7f"
        b = ctypes.create_string_buffer(bytes(d), len(d))
        lib.es_blob_info(ctypes.cast(b, ctypes.c_void_p), len(d), ctypes.byref(info))
    print(f"sanitized host driver: {calls} planner / metadata calls ok", flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
