"""MI355X-native variable-length transformer scoring (gfx950 HIP behind a C ABI).

Public API (all compute runs in libencscore's HIP kernels; PyTorch only
provides device memory and the current stream):

    Scorer(blob, max_tokens, max_seqs)       load a weight blob (bytes or path)
    Scorer.score(d_ids, offsets)             one packed batch -> rewards (device)
    Scorer.score_requests(d_ids, lengths)    plan + pack + score + scatter a stream
    plan_batches(lengths, max_tokens, c)     host DP batch planner
    plan_batches_measured(lengths, T, C)     the same DP under a measured cost table C[b-1, l-1]
    pack_offsets(lengths, order, b, e)       packed offsets of one planned batch
    plan_arena(bytes, first, last, align)    offsets of tensors with lifetimes (workspace planner)
    check_plan(lengths, heads, causal, ...)  build a call's per-pass metadata and check every index
    layernorm, softmax_ragged, attention_fused, gemm_bf16
                                             single kernels of the bf16 pass on caller buffers
    split_rows, layernorm_split, gemm_split, attention_last
                                             the last-token refinement's kernels (split-operand layout)
"""
from .api import (  # noqa: F401
    Scorer,
    plan_batches,
    plan_batches_measured,
    pack_offsets,
    plan_arena,
    check_plan,
    layernorm,
    RaggedScores,
    softmax_ragged,
    attention_fused,
    gemm_bf16,
    split_rows,
    layernorm_split,
    gemm_split,
    attention_last,
    version,
)
from ._lib import EncScoreError, EXPORTS  # noqa: F401
from . import blob  # noqa: F401
