"""User-facing wrappers over the C ABI (marshalling only, no compute).

Device tensors are torch tensors on the current ROCm device; the HIP stream is
torch's current stream.  Host arrays are numpy.
"""
import ctypes
import os

import numpy as np

from . import _lib
from ._lib import as_i32, check, i32p


def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _dptr(t, dtype, name):
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def version():
    return _lib.load().es_version().decode()


# ------------------------------------------------------------------ planner

def plan_batches(lengths, max_tokens, batch_overhead, lib=None):
    """Host DP planner -> (order int32[n], batch_starts int32[B+1], total_cost)."""
    lib = lib or _lib.load()
    lengths = as_i32(lengths)
    n = lengths.size
    order = np.zeros(n, dtype=np.int32)
    starts = np.zeros(n + 1, dtype=np.int32)
    nb = ctypes.c_int32()
    cost = ctypes.c_int64()
    check(lib, lib.es_plan_batches(i32p(lengths), n, int(max_tokens), int(batch_overhead),
                                   i32p(order), i32p(starts), ctypes.byref(nb), ctypes.byref(cost)))
    return order, starts[: nb.value + 1].copy(), cost.value


def plan_batches_measured(lengths, max_tokens, cost_table, lib=None):
    """Host DP planner under a measured cost table (es_plan_batches_measured):
    cost_table[b-1, l-1] is the cost of b sequences whose longest has l
    tokens -> (order int32[n], batch_starts int32[B+1], total_cost)."""
    lib = lib or _lib.load()
    lengths = as_i32(lengths)
    table = np.ascontiguousarray(cost_table, dtype=np.int64)
    if table.ndim != 2:
        raise ValueError("cost_table must be 2-D [max_batch, max_len]")
    n = lengths.size
    order = np.zeros(n, dtype=np.int32)
    starts = np.zeros(n + 1, dtype=np.int32)
    nb = ctypes.c_int32()
    cost = ctypes.c_int64()
    check(lib, lib.es_plan_batches_measured(
        i32p(lengths), n, int(max_tokens), table.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        table.shape[0], table.shape[1], i32p(order), i32p(starts), ctypes.byref(nb), ctypes.byref(cost)))
    return order, starts[: nb.value + 1].copy(), cost.value


def plan_arena(nbytes, first_step, last_step, align=1, lib=None):
    """Offsets of tensors with step lifetimes in one arena (es_plan_arena)
    -> (offsets int64[n], total bytes)."""
    lib = lib or _lib.load()
    nbytes = np.ascontiguousarray(nbytes, dtype=np.int64)
    first, last = as_i32(first_step), as_i32(last_step)
    n = nbytes.size
    if first.size != n or last.size != n:
        raise ValueError("nbytes, first_step and last_step differ in length")
    off = np.zeros(n, dtype=np.int64)
    total = ctypes.c_int64()
    p64 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    check(lib, lib.es_plan_arena(p64(nbytes), i32p(first), i32p(last), n, int(align), p64(off),
                                 ctypes.byref(total)))
    return off, total.value


def check_plan(lengths, n_heads, causal, max_pos, max_tokens, max_seqs, batch_overhead,
               batches_per_pass, prompt_lengths=None, cand_counts=None, lib=None):
    """es_check_plan: build a call's per-pass metadata on the host and check
    every index in it -> (passes, checks, violations); raises on a failure."""
    lib = lib or _lib.load()
    lengths = as_i32(lengths)
    n_prompts = 0
    pl = cc = None
    if prompt_lengths is not None:
        pl, cc = as_i32(prompt_lengths), as_i32(cand_counts)
        n_prompts = pl.size
    passes, checked, bad = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    check(lib, lib.es_check_plan(i32p(lengths), lengths.size, i32p(pl) if pl is not None else None,
                                 i32p(cc) if cc is not None else None, n_prompts, int(n_heads),
                                 int(bool(causal)), int(max_pos), int(max_tokens), int(max_seqs),
                                 int(batch_overhead), int(batches_per_pass), ctypes.byref(passes),
                                 ctypes.byref(checked), ctypes.byref(bad)))
    return passes.value, checked.value, bad.value


def pack_offsets(lengths, order, begin, end, lib=None):
    lib = lib or _lib.load()
    lengths, order = as_i32(lengths), as_i32(order)
    out = np.zeros(max(end - begin, 0) + 1, dtype=np.int32)
    check(lib, lib.es_pack_offsets(i32p(lengths), i32p(order), int(begin), int(end), i32p(out)))
    return out


# ------------------------------------------------------------------ model

class _MemoryStats(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("device_bytes", ctypes.c_int64),
                ("work_bytes", ctypes.c_int64), ("peak_work_bytes", ctypes.c_int64),
                ("allocs", ctypes.c_int64), ("alloc_ms", ctypes.c_double)]


class Scorer:
    """A loaded scoring model on the current device.

    ``blob`` is the weight blob as bytes or a file path.  ``max_tokens`` and
    ``max_seqs`` size the workspace (tokens / sequences per packed batch).
    """

    def __init__(self, blob, max_tokens, max_seqs):
        self.lib = _lib.load()
        h = ctypes.c_void_p()
        if isinstance(blob, (bytes, bytearray, memoryview, np.ndarray)):
            arr = np.frombuffer(blob, dtype=np.uint8)     # no copy
            st = self.lib.es_load_weights_mem(ctypes.c_void_p(arr.ctypes.data), arr.size,
                                              int(max_tokens), int(max_seqs), ctypes.byref(h))
        else:
            st = self.lib.es_load_weights(os.fsencode(blob), int(max_tokens), int(max_seqs),
                                          ctypes.byref(h))
        check(self.lib, st)
        self.handle = h
        self.info = _lib.ModelInfo()
        check(self.lib, self.lib.es_model_info(self.handle, ctypes.byref(self.info)))

    def close(self):
        if getattr(self, "handle", None):
            self.lib.es_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def reward_offset(self):
        v = ctypes.c_float()
        check(self.lib, self.lib.es_get_reward_offset(self.handle, ctypes.byref(v)))
        return v.value

    @reward_offset.setter
    def reward_offset(self, value):
        check(self.lib, self.lib.es_set_reward_offset(self.handle, float(value)))

    def score(self, d_ids, offsets, out=None):
        """Rewards float32[n] (device) of one packed batch; offsets on the host."""
        torch = _torch()
        offsets = as_i32(offsets)
        n = offsets.size - 1
        if out is None:
            out = torch.empty(max(n, 0), dtype=torch.float32, device=d_ids.device)
        check(self.lib, self.lib.es_score_batch(self.handle, _dptr(d_ids, torch.int32, "ids"),
                                                i32p(offsets), n,
                                                _dptr(out, torch.float32, "out"), _stream()))
        return out

    def score_static(self, d_ids, offsets, out):
        """es_score_batch_static: like score(), with every intermediate in the
        library's fixed per-GPU scratch array (no device allocation; the
        caller provides ``out``)."""
        torch = _torch()
        offsets = as_i32(offsets)
        check(self.lib, self.lib.es_score_batch_static(
            self.handle, _dptr(d_ids, torch.int32, "ids"), i32p(offsets), offsets.size - 1,
            _dptr(out, torch.float32, "out"), _stream()))
        return out

    def score_requests(self, d_ids, lengths, batch_overhead=1024, out=None):
        """Plan, pack, score and scatter a request stream; returns (rewards, stats)."""
        torch = _torch()
        lengths = as_i32(lengths)
        n = lengths.size
        if out is None:
            out = torch.empty(n, dtype=torch.float32, device=d_ids.device)
        stats = _lib.StreamStats()
        check(self.lib, self.lib.es_score_requests(
            self.handle, _dptr(d_ids, torch.int32, "ids"), i32p(lengths), n, int(batch_overhead),
            _dptr(out, torch.float32, "out"), _stream(), ctypes.byref(stats)))
        return out, {"n_batches": stats.n_batches, "total_cost": stats.total_cost,
                     "padded_tokens": stats.padded_tokens, "packed_tokens": stats.packed_tokens}

    def score_best_of_n(self, d_ids, prompt_lengths, cand_lengths, cand_counts,
                        batch_overhead=1024, rewards=None, best=None):
        """Best-of-N with shared prompts: d_ids holds the prompts back to back,
        then the candidates; returns (rewards per candidate, best index per
        prompt, stats)."""
        torch = _torch()
        pl, cl, cc = as_i32(prompt_lengths), as_i32(cand_lengths), as_i32(cand_counts)
        if rewards is None:
            rewards = torch.empty(cl.size, dtype=torch.float32, device=d_ids.device)
        if best is None:
            best = torch.empty(pl.size, dtype=torch.int32, device=d_ids.device)
        stats = _lib.StreamStats()
        check(self.lib, self.lib.es_score_best_of_n(
            self.handle, _dptr(d_ids, torch.int32, "ids"), i32p(pl), pl.size, i32p(cl), i32p(cc),
            int(batch_overhead), _dptr(rewards, torch.float32, "rewards"),
            _dptr(best, torch.int32, "best"), _stream(), ctypes.byref(stats)))
        return rewards, best, {"n_batches": stats.n_batches, "total_cost": stats.total_cost,
                               "padded_tokens": stats.padded_tokens,
                               "packed_tokens": stats.packed_tokens}

    def hidden(self, d_ids, offsets, n_layers=None):
        """fp32 residual stream [tokens, hidden] after ``n_layers`` layers (diagnostic)."""
        torch = _torch()
        offsets = as_i32(offsets)
        L = self.info.n_layers if n_layers is None else n_layers
        out = torch.empty((int(offsets[-1]), self.info.hidden), dtype=torch.float32,
                          device=d_ids.device)
        check(self.lib, self.lib.es_forward_hidden(self.handle, _dptr(d_ids, torch.int32, "ids"),
                                                   i32p(offsets), offsets.size - 1, int(L),
                                                   _dptr(out, torch.float32, "out"), _stream()))
        return out

    def calibrate_offset(self, d_ids, offsets):
        """offset = -mean raw reward of the reference set (does not set it)."""
        torch = _torch()
        offsets = as_i32(offsets)
        v = ctypes.c_float()
        check(self.lib, self.lib.es_calibrate_offset(self.handle, _dptr(d_ids, torch.int32, "ids"),
                                                     i32p(offsets), offsets.size - 1, _stream(),
                                                     ctypes.byref(v)))
        return v.value

    def set_concurrency(self, batches_in_flight):
        """Planned batches es_score_requests overlaps on internal streams (1..4)."""
        check(self.lib, self.lib.es_set_concurrency(self.handle, int(batches_in_flight)))

    def set_grouping(self, batches_per_pass):
        """Planned batches score_requests packs into one pass (es_set_batch_grouping)."""
        check(self.lib, self.lib.es_set_batch_grouping(self.handle, int(batches_per_pass)))

    def set_cost_table(self, cost_table):
        """Plan score_requests with measured batch costs (es_set_cost_table):
        cost_table[b-1, l-1] = cost of b sequences whose longest has l tokens;
        None goes back to the linear cost."""
        if cost_table is None:
            check(self.lib, self.lib.es_set_cost_table(self.handle, None, 0, 0))
            return
        table = np.ascontiguousarray(cost_table, dtype=np.int64)
        if table.ndim != 2:
            raise ValueError("cost_table must be 2-D [max_batch, max_len]")
        check(self.lib, self.lib.es_set_cost_table(
            self.handle, table.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            table.shape[0], table.shape[1]))

    def set_pruning(self, enabled):
        """Last layer on the last tokens only (default on; es_set_pruning)."""
        check(self.lib, self.lib.es_set_pruning(self.handle, 1 if enabled else 0))

    def set_refinement(self, enabled):
        """Last-token refinement of the reward rows (es_set_refinement; default on
        where the model supports it)."""
        check(self.lib, self.lib.es_set_refinement(self.handle, 1 if enabled else 0))

    def refinement(self):
        """Whether the last-token refinement runs (es_get_refinement)."""
        v = ctypes.c_int32()
        check(self.lib, self.lib.es_get_refinement(self.handle, ctypes.byref(v)))
        return bool(v.value)

    MEMORY_MODES = {"fixed": 0, "length_aware": 1, "exact": 2}

    def set_memory_mode(self, mode):
        """"length_aware" (default), "fixed" or "exact" (es_set_memory_mode)."""
        check(self.lib, self.lib.es_set_memory_mode(self.handle, self.MEMORY_MODES[mode]))

    def memory_stats(self, reset=False):
        """es_memory_stats as a dict (bytes, allocation count, ms)."""
        st = _MemoryStats()
        check(self.lib, self.lib.es_memory_stats(self.handle, ctypes.byref(st), 1 if reset else 0))
        names = {v: k for k, v in self.MEMORY_MODES.items()}
        return {"mode": names.get(st.mode, st.mode), "device_bytes": st.device_bytes,
                "work_bytes": st.work_bytes, "peak_work_bytes": st.peak_work_bytes,
                "allocs": st.allocs, "alloc_ms": st.alloc_ms}

    def set_attention(self, mode):
        """"unfused" (scores, softmax row reduction, P.V) or "fused" (one kernel)."""
        code = {"unfused": 0, "fused": 1}[mode]
        check(self.lib, self.lib.es_set_attention(self.handle, code))

    def profile_enable(self, classes=None):
        """Record HIP events around the given kernel classes (names; None = all)."""
        names = _lib.KERNEL_CLASSES
        mask = (1 << len(names)) - 1 if classes is None else \
            sum(1 << names.index(c) for c in classes)
        check(self.lib, self.lib.es_profile_enable(self.handle, mask))

    def profile_collect(self):
        """Per-class {launches, total_ms, flops, bytes} since profile_enable."""
        arr = (_lib.KernelStat * len(_lib.KERNEL_CLASSES))()
        check(self.lib, self.lib.es_profile_collect(self.handle, arr))
        return {_lib.KERNEL_CLASSES[k.kernel_class]: {"launches": k.launches, "total_ms": k.total_ms,
                                                      "flops": k.flops, "bytes": k.bytes}
                for k in arr}

    def check_device_errors(self):
        check(self.lib, self.lib.es_check_device_errors(self.handle, _stream()))


# ------------------------------------------------------------------ single ops

def layernorm(x, gamma, beta, eps, y=None, ybf16=None, sub=None):
    """Row LayerNorm of fp32 x [rows, cols] (of x + sub with `sub`, through
    es_op_add_layernorm) into y (fp32) and/or ybf16 (int16 bits)."""
    torch = _torch()
    lib = _lib.load()
    rows, cols = x.shape
    ld = ybf16.shape[1] if ybf16 is not None else 0
    outs = (_dptr(y, torch.float32, "y") if y is not None else None,
            _dptr(ybf16, torch.int16, "ybf16") if ybf16 is not None else None, ld, _stream())
    g, b = _dptr(gamma, torch.float32, "gamma"), _dptr(beta, torch.float32, "beta")
    if sub is None:
        check(lib, lib.es_op_layernorm(_dptr(x, torch.float32, "x"), g, b, rows, cols, float(eps), *outs))
    else:
        if tuple(sub.shape) != (rows, cols):
            raise ValueError(f"sub shape {tuple(sub.shape)} != x shape {(rows, cols)}")
        check(lib, lib.es_op_add_layernorm(_dptr(x, torch.float32, "x"), _dptr(sub, torch.float32, "sub"),
                                           g, b, rows, cols, float(eps), *outs))


class RaggedScores:
    """Ragged score layout of one batch (see es_ragged_create)."""

    def __init__(self, lengths, n_heads, causal):
        self.lib = _lib.load()
        self.lengths = as_i32(lengths)
        self.n_heads, self.causal = int(n_heads), int(bool(causal))
        h = ctypes.c_void_p()
        n_el = ctypes.c_int64()
        check(self.lib, self.lib.es_ragged_create(i32p(self.lengths), self.lengths.size,
                                                  self.n_heads, self.causal, ctypes.byref(h),
                                                  ctypes.byref(n_el)))
        self.handle, self.n_elems = h, n_el.value

    def close(self):
        if getattr(self, "handle", None):
            self.lib.es_ragged_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def softmax_ragged(rag, scores, probs):
    """Row softmax over the ragged layout; probs fp32 or int16 (bf16 bits)."""
    torch = _torch()
    lib = _lib.load()
    p_bf16 = probs.dtype == torch.int16
    check(lib, lib.es_op_softmax(rag.handle, _dptr(scores, torch.float32, "scores"),
                                 _dptr(probs, probs.dtype, "probs"), int(p_bf16), _stream()))


def attention_fused(rag, qkv, ctx, head_dim, scale=None):
    """Fused masked attention over the ragged layout (es_op_attention): qkv and
    ctx int16 tensors of bf16 bits, [T, ld] row-major."""
    torch = _torch()
    lib = _lib.load()
    if qkv.dim() != 2 or ctx.dim() != 2 or qkv.shape[0] != ctx.shape[0]:
        raise ValueError("qkv and ctx must be [T, ld] with the same T")
    if scale is None:
        scale = 1.0 / float(head_dim) ** 0.5
    check(lib, lib.es_op_attention(rag.handle, _dptr(qkv, torch.int16, "qkv"), int(qkv.stride(0)),
                                   int(head_dim), float(scale), _dptr(ctx, torch.int16, "ctx"),
                                   int(ctx.stride(0)), _stream()))


def gemm_bf16(a, w, bias, out, M, N, K, epilogue, res=None, tile=None):
    """out = epilogue(A W^T + bias) on the bf16 MFMA kernel (a, w as int16 bits);
    tile forces a block-tile configuration (0..6), None chooses from the shape."""
    torch = _torch()
    lib = _lib.load()
    args = (_dptr(a, torch.int16, "a"), a.shape[1], _dptr(w, torch.int16, "w"),
            _dptr(bias, torch.float32, "bias"),
            _dptr(res, torch.float32, "res") if res is not None else None,
            ctypes.c_void_p(out.data_ptr()), out.shape[1], int(M), int(N), int(K), int(epilogue))
    if tile is None:
        check(lib, lib.es_op_gemm_bf16(*args, _stream()))
    else:
        check(lib, lib.es_op_gemm_bf16_tile(*args, int(tile), _stream()))


# ------------------------------------------- last-token refinement kernels

def split_rows(a, out):
    """fp32 rows a [M, K] into the split-operand layout (es_op_split); out an
    int16 tensor of at least 2 * 32 ceil(M / 32) * K elements."""
    torch = _torch()
    lib = _lib.load()
    M, K = a.shape
    check(lib, lib.es_op_split(_dptr(a, torch.float32, "a"), int(a.stride(0)), int(M), int(K),
                               _dptr(out, torch.int16, "out"), _stream()))


def layernorm_split(x, gamma, beta, eps, out):
    """Row LayerNorm of fp32 x [rows, cols] into the split-operand layout."""
    torch = _torch()
    lib = _lib.load()
    rows, cols = x.shape
    check(lib, lib.es_op_layernorm_split(_dptr(x, torch.float32, "x"), _dptr(gamma, torch.float32, "gamma"),
                                         _dptr(beta, torch.float32, "beta"), int(rows), int(cols),
                                         float(eps), _dptr(out, torch.int16, "out"), _stream()))


def gemm_split(a_split, w, bias, M, N, K, epilogue, out=None, out_split=None, res=None):
    """epilogue(A W^T + bias) with A in the split-operand layout (es_op_gemm_split):
    epilogue 3 / 2 into fp32 out [M, ldc] (2 adds res), 1 (GELU) into out_split."""
    torch = _torch()
    lib = _lib.load()
    check(lib, lib.es_op_gemm_split(_dptr(a_split, torch.int16, "a_split"), _dptr(w, torch.int16, "w"),
                                    _dptr(bias, torch.float32, "bias"),
                                    _dptr(res, torch.float32, "res") if res is not None else None,
                                    _dptr(out, torch.float32, "out") if out is not None else None,
                                    _dptr(out_split, torch.int16, "out_split") if out_split is not None else None,
                                    int(out.stride(0)) if out is not None else 0, int(M), int(N), int(K),
                                    int(epilogue), _stream()))


def attention_last(rag, qkv, ql, ctx_split, head_dim, kc, scale=None):
    """fp32 attention of each sequence's last query (es_op_attention_last)."""
    torch = _torch()
    lib = _lib.load()
    if scale is None:
        scale = 1.0 / float(head_dim) ** 0.5
    check(lib, lib.es_op_attention_last(rag.handle, _dptr(qkv, torch.int16, "qkv"), int(qkv.stride(0)),
                                        _dptr(ql, torch.float32, "ql"), int(ql.stride(0)), int(head_dim),
                                        float(scale), _dptr(ctx_split, torch.int16, "ctx_split"), int(kc),
                                        _stream()))
