"""fp64 CPU oracle for RLT exact replay (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.
"""
from .rlt_oracle import (  # noqa: F401
    OracleModel,
    OracleState,
    attend,
    causal_attention,
    decode,
    decoder_step,
    encode,
    gelu,
    init_state,
    logits,
    replay,
    replay_batch,
    score_actions,
    rms_norm,
    sample_tokens,
    sigmoid,
    silu,
    step,
)
from .rlt_backward import (  # noqa: F401
    DETACH_PATHS,
    bptt,
    bptt_batch,
    next_token_loss,
)
