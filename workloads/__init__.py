"""Seeded synthetic workloads for RLT exact replay.

This package holds only the five model/batch shapes and the seeded input
generators (weights, token ids, bf16 rounding of inputs).  It contains none of
the method's arithmetic, so both the fp64 oracle (``oracle/``) and the HIP path
(``cross_token_recurrent_amd``) may import it without sharing any compute code.
"""
from .configs import CONFIGS, ModelConfig, Workload, get_workload  # noqa: F401
from .synth import (  # noqa: F401
    PARAM_ORDER,
    bf16_round,
    make_tokens,
    make_weights,
    param_shapes,
    perturb_untied,
)
