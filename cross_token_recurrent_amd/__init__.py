"""RLT exact replay on MI355X (gfx950): HIP kernels behind the C ABI of librlt.so.

``rlt`` is the thin ctypes binding; ``build`` compiles the library in-tree.
"""
from .rlt import (  # noqa: F401
    LIB_PATH,
    Model,
    RltError,
    State,
    load_library,
    make_config,
    replay,
    rlt_bptt,
    rlt_bptt_workspace_bytes,
    rlt_decoder_replay,
    rlt_decoder_replay_noalloc,
    rlt_decoder_step,
    rlt_decoder_step_sample,
    rlt_encoder_forward,
    rlt_logits,
    rlt_model_workspace_bytes,
    rlt_param_table,
    rlt_sample_tokens,
    rlt_score_actions,
    rlt_state_load_encoder_outputs,
    rlt_state_read_encoder_outputs,
    rlt_state_restore,
    rlt_state_save,
    rlt_state_snapshot_bytes,
)
