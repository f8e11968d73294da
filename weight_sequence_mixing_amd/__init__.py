"""weight_sequence_mixing_amd -- causal kernelized linear attention in
fast-weight form for AMD Instinct MI355X (gfx950).

The computation lives in liblinattn.so (hand-written HIP kernels behind the C
ABI declared in include/la.h).  This package is its thin Python binding: the
functions below carry the C names and only marshal torch tensors, shapes and
the current HIP stream.
"""
from .binding import (  # noqa: F401
    EXPORTS, KERNEL_IDS, LA_BF16, LA_F32, LA_MAX_HEADS, LA_PHI_ELU1, LA_PHI_RELU, LA_PHI_TRIG_RF,
    LA_PHI_TRIG_RF_PLAIN, LA_PHI_TRIG_RF_SOFTMAX, LaError, Phi,
    la_decode_step, la_forward_causal, la_forward_causal_noalloc, la_forward_causal_masked, la_forward_causal_varlen, la_forward_cross,
    la_forward_noncausal, la_init_state, la_init_state_identity, la_kernel_name, la_workspace_size_cross,
    la_workspace_size_varlen, la_backward_causal, la_workspace_size_backward, la_backward_cross,
    la_workspace_size_backward_cross,
    la_last_error, la_profile_begin, la_profile_end, la_status_string, la_workspace_size,
    load_library, rf_scale,
)
