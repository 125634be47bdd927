"""Block-wise dynamic token dropping (UniPrefill-style) on MI355X.

Thin Python binding over the C ABI of ``libuniprefill.so`` (declared in
``include/uniprefill.h``).  This module only marshals arguments: torch tensors
provide device memory and the current HIP stream; every step of the path runs in
the library's HIP kernels.  There is no fallback: if the library is missing the
import of the binding raises.
"""
from ._binding import (  # noqa: F401
    UniPrefillError,
    LayerDecision,
    block_scores,
    block_scores_chunks,
    block_scores_lse,
    block_scores_lse_paged,
    block_scores_paged,
    block_scores_lse_workspace_bytes,
    block_scores_workspace_bytes,
    compose_drops,
    device_error,
    expand_compact,
    expand_compact_noalloc,
    expand_compact_workspace_bytes,
    lib,
    profile_enable,
    profile_read,
    profile_reset,
    topk_select,
    topp_select,
    rope_attention,
    rope_attention_scores,
    rope_attention_scores_workspace_bytes,
    rope_attention_workspace_bytes,
    linear,
    swiglu,
    swiglu_ffn,
    swiglu_ffn_workspace_bytes,
    KERNEL_IDS,
)
