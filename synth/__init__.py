"""Seeded synthetic inputs shared by the oracle and the GPU library.

This package holds data only: model shapes, seeded weight draws and seeded
request streams.  It performs none of the scoring arithmetic, so both the
CPU oracle (``oracle/``) and the HIP path (``encoder_scoring_amd``) may use it
without sharing any computation.
"""
from .configs import ModelConfig, CONFIGS, get_config  # noqa: F401
from .generate import (  # noqa: F401
    make_weights,
    make_requests,
    make_reference_set,
    make_fixed_batch,
    round_to_bf16,
    WEIGHT_ORDER,
)
