"""SimSD verification hot path on MI355X (gfx950).

The target model's single verification pass of SimSD-style speculative
decoding for block diffusion LMs (page "SimSD - Simple Speculative Decoding
in Diffusion Language Models"): grouped-query attention of the paired data /
mask block rows over the prompt KV cache under the tau-driven temporal mask
with RoPE copy, and the tau-ordered rejection-sampling acceptance.  The
kernels are HIP for gfx950 behind the C ABI of include/simsd.h
(libsimsd.so); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    BF16, F32, IMPL_AUTO, IMPL_MFMA, IMPL_VALU, MASK_FULL, MASK_TEMPORAL, ROPE_COPY, ROPE_SEQUENTIAL, SimsdError,
    ST_POS_NEG, ST_PROMPT_LEN, ST_TAU_NOT_PERM, ST_TAU_RANGE, ST_TOKEN_RANGE,
)
from .api import (  # noqa: F401
    accept_coupled, accept_coupled_workspace_bytes, accept_prefix, accept_prefix_noalloc, accept_workspace_bytes, append_kv, bind_accept,
    bind_append_kv, bind_commit, bind_next_round, next_round,
    bind_accept_coupled, bind_linear, bind_qkv_proj, bind_verify, commit, debug_mask, debug_rope, linear, make_desc,
    mfma_probe, qkv_proj, read_probe, stream_probe, verify_attn,
    verify_plan,
    verify_workspace_bytes,
)
