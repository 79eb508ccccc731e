"""MI355X-native Kimi Delta Attention (KDA): a C-ABI library of HIP kernels
for gfx950 (libkda.so, declared in include/kda.h) and its Python binding.

    from gated_delta_rule_101_amd import kda_chunk_fwd, kda_decode_step
    from gated_delta_rule_101_amd import kda_verify_step, kda_commit_step        # speculative decoding
    from gated_delta_rule_101_amd import kda_chunk_fwd_gate, kda_decode_step_gate  # g from gate logits
    from gated_delta_rule_101_amd import kda_output_gate, kda_decode_step_gated    # output epilogue
    from gated_delta_rule_101_amd import kda_chunk_bwd                             # gradients
    from gated_delta_rule_101_amd import kda_chunk_fwd_seqpar                      # sequence-parallel forward
    from gated_delta_rule_101_amd import kda_chunk_fwd_gate_seqpar                 # the same from gate logits
"""

from .kda import (  # noqa: F401
    EXPORTS, KDA_BF16, KDA_ERR_INVALID_ARG, KDA_ERR_LAUNCH, KDA_ERR_SCRATCH, KDA_ERR_UNSUPPORTED, KDA_F32,
    KDA_OK, KdaError, debug_set_spin_limit, kda_chunk_bwd, kda_chunk_bwd_workspace_bytes, kda_chunk_fwd,
    kda_chunk_fwd_gate, kda_chunk_fwd_gate_seqpar, kda_chunk_fwd_noalloc, kda_chunk_fwd_seqpar,
    kda_chunk_fwd_seqpar_segments,
    kda_chunk_fwd_seqpar_workspace_bytes,
    kda_chunk_fwd_workspace_bytes, kda_commit_step, kda_decode_step,
    kda_decode_step_gate, kda_decode_step_gated, kda_output_gate, kda_verify_step, load_library,
    status_string,
)
