"""ctypes binding of libencscore.so (argument marshalling only).

Every step of scoring runs inside the library's HIP kernels; this module only
converts arguments.  PyTorch supplies device memory and the current HIP
stream.  If the shared library has not been built the import fails loudly:
there is no fallback path.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libencscore.so")

ES_OK, ES_ERR_ARG, ES_ERR_RANGE, ES_ERR_CAPACITY = 0, -1, -2, -3
STATIC_SCRATCH_BYTES = 64 * 1024 * 1024  # ES_STATIC_SCRATCH_BYTES (es_score_batch_static)
ES_ERR_FORMAT, ES_ERR_IO, ES_ERR_HIP, ES_ERR_DEVICE_FLAG = -4, -5, -6, -7
STATUS_NAMES = {0: "ES_OK", -1: "ES_ERR_ARG", -2: "ES_ERR_RANGE", -3: "ES_ERR_CAPACITY",
                -4: "ES_ERR_FORMAT", -5: "ES_ERR_IO", -6: "ES_ERR_HIP", -7: "ES_ERR_DEVICE_FLAG"}

# every symbol declared in include/encscore.h
EXPORTS = [
    "es_load_weights", "es_load_weights_mem", "es_free", "es_model_info", "es_score_batch",
    "es_score_batch_static", "es_check_plan", "es_blob_info",
    "es_score_requests",
    "es_forward_hidden", "es_set_reward_offset", "es_get_reward_offset", "es_calibrate_offset",
    "es_check_device_errors", "es_plan_batches", "es_plan_batches_measured", "es_set_cost_table", "es_pack_offsets", "es_op_layernorm", "es_op_add_layernorm",
    "es_ragged_create", "es_ragged_free", "es_op_softmax", "es_op_attention", "es_op_gemm_bf16", "es_op_gemm_bf16_tile", "es_op_split", "es_op_layernorm_split", "es_op_gemm_split", "es_op_attention_last", "es_last_error",
    "es_version", "es_set_concurrency", "es_set_batch_grouping", "es_score_best_of_n", "es_set_pruning", "es_set_refinement", "es_get_refinement", "es_set_memory_mode", "es_memory_stats", "es_plan_arena", "es_set_attention", "es_profile_enable", "es_profile_collect", "es_kernel_class_name",
]

KERNEL_CLASSES = ["embed", "qkv_gemm", "scores", "softmax", "pv", "oproj_gemm", "layernorm",
                  "ffn1_gemm", "ffn2_gemm", "head", "attn_fused", "gather", "refine"]


class EncScoreError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class ModelInfo(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32), ("max_pos", ctypes.c_int32),
                ("pre_ln", ctypes.c_int32), ("causal", ctypes.c_int32), ("bf16", ctypes.c_int32),
                ("eps", ctypes.c_float), ("reward_offset", ctypes.c_float),
                ("max_tokens", ctypes.c_int64), ("max_seqs", ctypes.c_int32),
                ("device_bytes", ctypes.c_int64)]


class StreamStats(ctypes.Structure):
    _fields_ = [("n_batches", ctypes.c_int32), ("total_cost", ctypes.c_int64),
                ("padded_tokens", ctypes.c_int64), ("packed_tokens", ctypes.c_int64)]


class KernelStat(ctypes.Structure):
    _fields_ = [("kernel_class", ctypes.c_int32), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double)]


_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)
_SIGS = {
    "es_load_weights": (ctypes.c_int32, [ctypes.c_char_p, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(_P)]),
    "es_load_weights_mem": (ctypes.c_int32, [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(_P)]),
    "es_free": (None, [_P]),
    "es_model_info": (ctypes.c_int32, [_P, ctypes.POINTER(ModelInfo)]),
    "es_score_batch": (ctypes.c_int32, [_P, _P, _I32P, ctypes.c_int32, _P, _P]),
    "es_score_batch_static": (ctypes.c_int32, [_P, _P, _I32P, ctypes.c_int32, _P, _P]),
    "es_blob_info": (ctypes.c_int32, [_P, ctypes.c_int64, ctypes.POINTER(ModelInfo)]),
    "es_check_plan": (ctypes.c_int32, [_I32P, ctypes.c_int32, _I32P, _I32P, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_int64)]),
    "es_score_requests": (ctypes.c_int32, [_P, _P, _I32P, ctypes.c_int32, ctypes.c_int64, _P, _P, ctypes.POINTER(StreamStats)]),
    "es_forward_hidden": (ctypes.c_int32, [_P, _P, _I32P, ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "es_score_best_of_n": (ctypes.c_int32, [_P, _P, _I32P, ctypes.c_int32, _I32P, _I32P, ctypes.c_int64, _P, _P, _P, ctypes.POINTER(StreamStats)]),
    "es_set_reward_offset": (ctypes.c_int32, [_P, ctypes.c_float]),
    "es_set_concurrency": (ctypes.c_int32, [_P, ctypes.c_int32]),
    "es_set_batch_grouping": (ctypes.c_int32, [_P, ctypes.c_int32]),
    "es_set_pruning": (ctypes.c_int32, [_P, ctypes.c_int32]),
    "es_set_refinement": (ctypes.c_int32, [_P, ctypes.c_int32]),
    "es_get_refinement": (ctypes.c_int32, [_P, ctypes.POINTER(ctypes.c_int32)]),
    "es_set_attention": (ctypes.c_int32, [_P, ctypes.c_int32]),
    "es_get_reward_offset": (ctypes.c_int32, [_P, ctypes.POINTER(ctypes.c_float)]),
    "es_calibrate_offset": (ctypes.c_int32, [_P, _P, _I32P, ctypes.c_int32, _P, ctypes.POINTER(ctypes.c_float)]),
    "es_check_device_errors": (ctypes.c_int32, [_P, _P]),
    "es_plan_arena": (ctypes.c_int32, [_I64P, _I32P, _I32P, ctypes.c_int32, ctypes.c_int64, _I64P, _I64P]),
    "es_set_memory_mode": (ctypes.c_int32, [_P, ctypes.c_int32]),
    "es_memory_stats": (ctypes.c_int32, [_P, _P, ctypes.c_int32]),
    "es_plan_batches": (ctypes.c_int32, [_I32P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, _I32P, _I32P, _I32P, _I64P]),
    "es_plan_batches_measured": (ctypes.c_int32, [_I32P, ctypes.c_int32, ctypes.c_int64, _I64P, ctypes.c_int32, ctypes.c_int32, _I32P, _I32P, _I32P, _I64P]),
    "es_set_cost_table": (ctypes.c_int32, [_P, _I64P, ctypes.c_int32, ctypes.c_int32]),
    "es_pack_offsets": (ctypes.c_int32, [_I32P, _I32P, ctypes.c_int32, ctypes.c_int32, _I32P]),
    "es_op_layernorm": (ctypes.c_int32, [_P, _P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, _P, _P, ctypes.c_int32, _P]),
    "es_op_add_layernorm": (ctypes.c_int32, [_P, _P, _P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, _P, _P, ctypes.c_int32, _P]),
    "es_ragged_create": (ctypes.c_int32, [_I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_P), _I64P]),
    "es_ragged_free": (None, [_P]),
    "es_op_softmax": (ctypes.c_int32, [_P, _P, _P, ctypes.c_int32, _P]),
    "es_op_attention": (ctypes.c_int32, [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, ctypes.c_int32, _P]),
    "es_op_gemm_bf16": (ctypes.c_int32, [_P, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P]),
    "es_op_gemm_bf16_tile": (ctypes.c_int32, [_P, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P]),
    "es_op_split": (ctypes.c_int32, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "es_op_layernorm_split": (ctypes.c_int32, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, _P]),
    "es_op_gemm_split": (ctypes.c_int32, [_P, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P]),
    "es_op_attention_last": (ctypes.c_int32, [_P, _P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, ctypes.c_int32, _P]),
    "es_profile_enable": (ctypes.c_int32, [_P, ctypes.c_uint32]),
    "es_profile_collect": (ctypes.c_int32, [_P, ctypes.POINTER(KernelStat)]),
    "es_kernel_class_name": (ctypes.c_char_p, [ctypes.c_int32]),
    "es_last_error": (ctypes.c_char_p, []),
    "es_version": (ctypes.c_char_p, []),
}

_lib = None


def load(path=None):
    """Load (once) and return the ctypes handle of libencscore.so."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is not built; run `python -m encoder_scoring_amd.build` "
                          "(the HIP library is required, there is no fallback)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def load_host(path):
    """Load a host-only build (planner + blob parser) with the planner signatures."""
    lib = ctypes.CDLL(path)
    for name in ("es_plan_batches", "es_plan_batches_measured", "es_pack_offsets", "es_plan_arena",
                 "es_check_plan", "es_blob_info", "es_last_error", "es_version"):
        res, args = _SIGS[name]
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


def check(lib, status):
    if status != ES_OK:
        raise EncScoreError(status, lib.es_last_error().decode(errors="replace"))


def i32p(a):
    return a.ctypes.data_as(_I32P)


def as_i32(a):
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)
