"""BDLM masked attention for AMD MI355X (gfx950): hand-written HIP kernels behind
a C ABI (include/bdlm_attn.h), with a thin torch binding.

Block diffusion LM attention over [clean x0 ; corrupted xt] in blocks of B
tokens ("Block Parallelism For Efficient Distributed Long-Context Diffusion
Language Model Training", arXiv 2609.19242), forward and backward, plus the
per-block (BP / CSBP) share mode with (O, LSE) partial merging.
"""
from .api import (  # noqa: F401
    KernelTimer,
    attention_bwd,
    attention_fwd,
    bdlm_attn_bwd,
    bdlm_attn_bwd_noalloc,
    bdlm_attn_fwd,
    bdlm_attn_merge_partials,
    bdlm_attention,
    bdlm_attn_workspace_bytes,
    bdlm_calib_mfma,
    desc_for,
    merge_partials,
    schedule_walk,
    share_bwd,
    share_fwd,
    workspace,
)
from ._lib import LIB_PATH, load  # noqa: F401
