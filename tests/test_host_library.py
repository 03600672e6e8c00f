"""CPU tests of libencscore: exported symbols, the host planner (bit-exact vs
the oracle), offset packing, error codes and blob validation.  Nothing here
calls a compute entry point, so no GPU is needed.
"""
import ctypes
import os
import re
import struct

import numpy as np
import pytest

import oracle
from oracle import memplan
from encoder_scoring_amd import _lib, blob, pack_offsets, plan_arena, plan_batches, plan_batches_measured
from encoder_scoring_amd.costmodel import dense_cost_table
from encoder_scoring_amd._lib import EncScoreError
from synth import CONFIGS, get_config, make_requests, make_weights
from synth.configs import ORDERED

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "encscore.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(es_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = _lib.load()
    decl = declared_functions()
    assert len(decl) >= 20
    assert sorted(_lib.EXPORTS) == decl
    for name in decl:
        assert hasattr(lib, name), name


def test_version_string():
    assert b"gfx950" in _lib.load().es_version()


@pytest.mark.parametrize("name", ORDERED)
def test_planner_matches_oracle_on_every_workload(name):
    cfg = get_config(name)
    _, lengths, _ = make_requests(cfg)
    T = cfg.max_tokens
    c = cfg.batch_overhead
    o_order, o_starts, o_cost = oracle.plan_batches(lengths, T, c)
    order, starts, cost = plan_batches(lengths, T, c)
    assert np.array_equal(order, o_order)
    assert np.array_equal(starts, o_starts)
    assert cost == o_cost
    for b in range(len(starts) - 1):
        off = pack_offsets(lengths, order, starts[b], starts[b + 1])
        assert np.array_equal(off, oracle.pack_offsets(lengths, order, starts[b], starts[b + 1]))


def test_planner_matches_oracle_random():
    rng = np.random.default_rng(99)
    for _ in range(300):
        n = int(rng.integers(0, 60))
        T = int(rng.choice([8, 16, 64, 300]))
        c = int(rng.choice([0, 1, 5, 64, 1024]))
        lengths = rng.integers(1, min(T, int(rng.choice([4, 20, T]))) + 1, size=n)
        got = plan_batches(lengths, T, c)
        want = oracle.plan_batches(lengths, T, c)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
        assert got[2] == want[2]


def test_planner_matches_exhaustive_small():
    rng = np.random.default_rng(5)
    for _ in range(150):
        n = int(rng.integers(1, 8))
        T, c = int(rng.choice([8, 12, 20])), int(rng.choice([0, 2, 9]))
        lengths = rng.integers(1, 7, size=n)
        _, starts, cost = plan_batches(lengths, T, c)
        assert cost == oracle.exhaustive_set_partition_cost(lengths, T, c)
        assert list(starts) == oracle.best_contiguous_plan(lengths, T, c)[0]


@pytest.mark.parametrize("lengths,T,c,code", [
    ([0, 3], 10, 1, _lib.ES_ERR_RANGE),
    ([11], 10, 1, _lib.ES_ERR_RANGE),
    ([1], 10, -1, _lib.ES_ERR_ARG),
    ([1], 0, 1, _lib.ES_ERR_ARG),
])
def test_planner_errors(lengths, T, c, code):
    with pytest.raises(EncScoreError) as e:
        plan_batches(lengths, T, c)
    assert e.value.status == code


def test_planner_empty_and_null():
    order, starts, cost = plan_batches([], 10, 3)
    assert order.size == 0 and starts.tolist() == [0] and cost == 0
    lib = _lib.load()
    nb, cost = ctypes.c_int32(), ctypes.c_int64()
    st = lib.es_plan_batches(None, 3, 10, 0, None, None, ctypes.byref(nb), ctypes.byref(cost))
    assert st == _lib.ES_ERR_ARG
    assert b"NULL" in lib.es_last_error()


def test_pack_offsets_errors():
    with pytest.raises(EncScoreError):
        pack_offsets([1, 2], [0, 1], 2, 1)


# ------------------------------------------------------------------ measured-cost planner

def _monotone_table(rng, max_batch, max_len, step=4):
    steps = rng.integers(0, step, size=(max_batch, max_len)) * (rng.random((max_batch, max_len)) < 0.7)
    return np.cumsum(steps, axis=1) + rng.integers(0, 5, size=(max_batch, 1))


def test_measured_planner_matches_oracle_random():
    rng = np.random.default_rng(31)
    for _ in range(300):
        n = int(rng.integers(0, 60))
        max_len = int(rng.choice([4, 20, 64]))
        max_batch = int(rng.integers(1, 40))
        T = int(rng.choice([max_len, 3 * max_len, 300]))
        table = _monotone_table(rng, max_batch, max_len)
        lengths = rng.integers(1, max_len + 1, size=n)
        got = plan_batches_measured(lengths, T, table)
        want = oracle.plan_batches_table(lengths, T, table)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
        assert got[2] == want[2]


def test_measured_planner_matches_exhaustive_small():
    rng = np.random.default_rng(6)
    for _ in range(150):
        n = int(rng.integers(1, 8))
        max_len, max_batch = 6, int(rng.integers(1, 5))
        T = int(rng.choice([6, 12, 20]))
        table = _monotone_table(rng, max_batch, max_len)
        lengths = rng.integers(1, 7, size=n)
        _, starts, cost = plan_batches_measured(lengths, T, table)
        assert cost == oracle.exhaustive_set_partition_cost_table(lengths, T, table)
        assert list(starts) == oracle.best_contiguous_plan_table(lengths, T, table)[0]


@pytest.mark.parametrize("name", ["bert_base_short", "bert_base_longtail"])
def test_linear_table_reproduces_the_linear_planner(name):
    """C[b, l] = c + b * l is the linear cost: the same plan, bit for bit."""
    cfg = get_config(name)
    _, lengths, _ = make_requests(cfg)
    T, c = cfg.max_tokens, cfg.batch_overhead
    P = int(lengths.max())
    b = np.arange(1, T + 1, dtype=np.int64)[:, None]
    table = c + b * np.arange(1, P + 1, dtype=np.int64)[None, :]
    got = plan_batches_measured(lengths, T, table)
    want = plan_batches(lengths, T, c)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


@pytest.mark.parametrize("table,lengths,T,code", [
    ([[1, 0, 2]], [1], 10, _lib.ES_ERR_ARG),           # falls along the length
    ([[-1, 0]], [1], 10, _lib.ES_ERR_ARG),             # negative entry
    ([[2 ** 62, 2 ** 62]], [1], 10, _lib.ES_ERR_ARG),  # too large for int64 sums
    ([[1, 2]], [3], 10, _lib.ES_ERR_RANGE),            # longer than the table
    ([[1, 2, 3]], [3], 2, _lib.ES_ERR_RANGE),          # longer than the budget
    ([[1, 2]], [1], 0, _lib.ES_ERR_ARG),               # max_tokens < 1
])
def test_measured_planner_errors(table, lengths, T, code):
    with pytest.raises(EncScoreError) as e:
        plan_batches_measured(lengths, T, np.array(table, dtype=np.int64))
    assert e.value.status == code


def test_measured_planner_empty_and_null():
    order, starts, cost = plan_batches_measured([], 10, np.ones((2, 3), dtype=np.int64))
    assert order.size == 0 and starts.tolist() == [0] and cost == 0
    lib = _lib.load()
    nb, cost = ctypes.c_int32(), ctypes.c_int64()
    st = lib.es_plan_batches_measured(None, 0, 10, None, 1, 1, None, None, ctypes.byref(nb),
                                      ctypes.byref(cost))
    assert st == _lib.ES_ERR_ARG


def test_dense_cost_table_is_exact_on_bilinear_costs():
    """Piecewise-linear in the batch size, then in the length, reproduces a
    function linear in each (also past the last measured size, and where
    corners beyond the token budget were not measured)."""
    f = lambda b, l: 0.02 + 0.001 * b + 0.0004 * l + 0.00003 * b * l   # ms
    bg, lg = [1, 2, 4, 8, 16], [1, 16, 64, 128]
    meas = np.array([[f(b, l) if b * l <= 512 else np.nan for l in lg] for b in bg])
    table = dense_cost_table(bg, lg, meas, 160)
    assert table.shape == (16, 160)
    b = np.arange(1, 17)[:, None]
    l = np.arange(1, 161)[None, :]
    assert np.abs(table - f(b, l) * 1e6).max() <= 1.0                    # ns rounding (+ fp)
    assert np.all(np.diff(table, axis=1) >= 0)


def test_dense_cost_table_clamps_and_is_monotone():
    bg, lg = [1, 4], [8, 32]
    meas = np.array([[1.0, 0.5], [2.0, 3.0]])                     # falls along the length at b = 1
    table = dense_cost_table(bg, lg, meas, 40)
    assert np.all(np.diff(table, axis=1) >= 0) and np.all(table >= 0)
    assert np.all(table[0, :8] == 1_000_000)                       # below the grid: the first point
    assert np.all(table[0, 8:] == 1_000_000)                       # running maximum keeps 1 ms
    assert table[3, 7] == 2_000_000 and table[3, 31] == 3_000_000
    with pytest.raises(ValueError):
        dense_cost_table([2, 1], lg, meas, 40)


# ------------------------------------------------------------------ arena planner

def test_plan_arena_matches_oracle_random():
    """es_plan_arena places exactly as the oracle's largest-first lowest-fit
    rule, validly, and never below the brute-force optimum (n <= 6)."""
    rng = np.random.default_rng(17)
    for trial in range(400):
        n = int(rng.integers(0, 12))
        nb = [int(x) for x in rng.integers(0, 50, size=n) * int(rng.choice([1, 3, 1000]))]
        f = [int(x) for x in rng.integers(0, 10, size=n)]
        l = [a + int(rng.integers(0, 5)) for a in f]
        align = int(rng.choice([1, 64, 4096]))
        off, total = plan_arena(nb, f, l, align)
        o_off, o_total = memplan.greedy_by_size(nb, f, l, align)
        assert list(off) == o_off and total == o_total, (nb, f, l, align)
        assert memplan.valid(nb, f, l, list(off), align)
        assert total >= memplan.lower_bound(nb, f, l, align)
        if n <= 6:
            assert total >= memplan.optimum(nb, f, l, align)


def test_plan_arena_on_a_pass_of_the_encoder():
    """The workspace records of a BERT-base pass (16384 rows, fused attention):
    x, xb, qkv, ctx, y, hmid; the plan reaches the bytes alive at the
    attention-out GEMM (x + xb + qkv + ctx + y), the lower bound."""
    rows, H, act = 16384, 768, 2
    nb = [rows * H * 4, rows * H * act, rows * 3 * H * act, rows * H * act, rows * H * 4,
          rows * 4 * H * act, 0, 0]
    f = [0, 0, 2, 3, 4, 7, 3, 3]
    l = [10, 10, 5, 5, 9, 8, 3, 3]
    off, total = plan_arena(nb, f, l, 4096)
    assert memplan.valid(nb, f, l, list(off), 4096)
    assert total == memplan.lower_bound(nb, f, l, 4096) == rows * H * (4 + 2 + 6 + 2 + 4)
    assert total < sum(nb)


def test_plan_arena_errors():
    with pytest.raises(EncScoreError):
        plan_arena([10], [3], [2])            # first step after last
    with pytest.raises(EncScoreError):
        plan_arena([-1], [0], [0])            # negative size
    with pytest.raises(EncScoreError):
        plan_arena([10], [0], [0], align=48)  # not a power of two
    off, total = plan_arena([], [], [])
    assert off.size == 0 and total == 0


def test_host_only_build_exports_the_arena_planner(tmp_path):
    from encoder_scoring_amd import build
    lib = _lib.load_host(build.build_host())
    off, total = plan_arena([5, 7], [0, 1], [1, 2], 4, lib=lib)
    assert total == 16 and memplan.valid([5, 7], [0, 1], [1, 2], list(off), 4)


# ------------------------------------------------------------------ blob

def _tiny_blob(offset=0.0):
    cfg = get_config("tiny_fp32")
    return cfg, blob.to_bytes(cfg, make_weights(cfg), offset)


def _load_mem(data):
    lib = _lib.load()
    h = ctypes.c_void_p()
    buf = ctypes.create_string_buffer(bytes(data), len(data))
    st = lib.es_load_weights_mem(ctypes.cast(buf, ctypes.c_void_p), len(data), 64, 8, ctypes.byref(h))
    return st, lib.es_last_error().decode()


def test_blob_size_matches_layout():
    cfg, data = _tiny_blob()
    H, F, V, P, L = cfg.hidden, cfg.ffn, cfg.vocab, cfg.max_pos, cfg.n_layers
    per_layer = 4 * (3 * H * H + 3 * H + H * H + H + 2 * H + F * H + F + H * F + H + 2 * H)
    assert len(data) == 64 + 4 * (V * H + P * H + 2 * H) + L * per_layer + 4 * (H + 1)
    magic, version, nl, hid = struct.unpack_from("<4s3I", data)
    assert (magic, version, nl, hid) == (b"ESW1", 1, L, H)


def test_bf16_blob_is_smaller():
    cfg = get_config("tinybert")
    w = make_weights(cfg)
    assert w["tok_emb"].dtype == np.uint16 and w["l0.b_qkv"].dtype == np.float32
    data = blob.to_bytes(cfg, w)
    H = cfg.hidden
    assert len(data) < 4 * cfg.vocab * H


@pytest.mark.parametrize("mutate,msg", [
    (lambda d: b"XXXX" + d[4:], "magic"),
    (lambda d: d[:4] + struct.pack("<I", 7) + d[8:], "version"),
    (lambda d: d[:-4], "truncated"),
    (lambda d: d + b"\0\0\0\0", "trailing"),
    (lambda d: d[:12] + struct.pack("<I", 130) + d[16:], "hidden"),      # not a multiple of 4... 130
    (lambda d: d[:16] + struct.pack("<I", 3) + d[20:], "n_heads"),      # 3 does not divide 128
    (lambda d: d[:20], "header"),
])
def test_corrupt_blob_rejected_before_any_device_call(mutate, msg):
    _, data = _tiny_blob()
    st, err = _load_mem(mutate(data))
    assert st == _lib.ES_ERR_FORMAT, err
    assert msg in err


def test_missing_blob_file():
    lib = _lib.load()
    h = ctypes.c_void_p()
    st = lib.es_load_weights(b"/nonexistent/weights.bin", 64, 8, ctypes.byref(h))
    assert st == _lib.ES_ERR_IO


def test_bad_capacity_arguments():
    _, data = _tiny_blob()
    lib = _lib.load()
    h = ctypes.c_void_p()
    buf = ctypes.create_string_buffer(data, len(data))
    assert lib.es_load_weights_mem(ctypes.cast(buf, ctypes.c_void_p), len(data), 0, 8,
                                   ctypes.byref(h)) == _lib.ES_ERR_ARG
    assert lib.es_load_weights_mem(ctypes.cast(buf, ctypes.c_void_p), len(data), 64, 0,
                                   ctypes.byref(h)) == _lib.ES_ERR_ARG


def test_null_handle_calls_fail_cleanly():
    lib = _lib.load()
    off = np.array([0, 3], dtype=np.int32)
    assert lib.es_score_batch(None, None, _lib.i32p(off), 1, None, None) == _lib.ES_ERR_ARG
    assert lib.es_set_reward_offset(None, 0.0) == _lib.ES_ERR_ARG
    lib.es_free(None)


def test_blob_writer_rejects_wrong_dtype():
    cfg = get_config("tinybert")
    w = make_weights(cfg)
    w["l0.w_qkv"] = w["l0.w_qkv"].astype(np.float32)
    with pytest.raises(ValueError):
        blob.to_bytes(cfg, w)
