"""CPU oracle for variable-length transformer scoring -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct definition of what the GPU
library computes.  It shares no code with the HIP path: it never imports
``encoder_scoring_amd`` and the library never imports it.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.

Sources (the pages, by title and section):
  * "TurboTransformers: An Efficient GPU Serving System For Transformer
    Models" (review): Abstract and Proposed method -- Softmax and LayerNorm
    as row ("batch") reductions next to the BLAS GEMMs; requests sorted by
    length and grouped by a dynamic-programming batch scheduler with minimal
    padding.
  * "Learning to summarize from human feedback" (summary), Method adaptation: the reward
    model is a transformer with a scalar head, the reward is read at the end
    of the complete sequence, and rewards are normalised so that reference
    summaries average zero; best-of-N scores N candidates per prompt.
  * SambaNova, "Breakthrough efficiency in NLP model deployment": compact
    BERT (TinyBERT) for online inference.
  * "Learning to summarize from human feedback" (summary), Method adaptation:
    best-of-N selection over the reward model's scores (selection.py).

Precision: float64 by default (``dtype`` argument; float32 is the plain fp32
forward used as the CPU baseline).  GELU's erf is evaluated in float64 by
scipy in both modes.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
closed forms, textbook values (tests/golden), brute force on tiny inputs and
an independent third-party layer implementation (torch.nn.TransformerEncoderLayer
on the CPU).
"""
from .model import (  # noqa: F401
    OracleModel,
    layer_norm,
    softmax_rows,
    gelu,
    linear,
    attention,
    masked_attention,
)
from .selection import best_of_n  # noqa: F401
from .scheduler import (  # noqa: F401
    plan_batches,
    pack_offsets,
    plan_cost,
    exhaustive_set_partition_cost,
    best_contiguous_plan,
    plan_batches_table,
    plan_cost_table,
    exhaustive_set_partition_cost_table,
    best_contiguous_plan_table,
)
