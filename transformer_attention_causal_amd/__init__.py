"""MI355X-native reshaped-softmax causal attention (tempered and dilution).

The computation lives in ``libattn.so`` (hand-written HIP kernels for gfx950
behind a C ABI, declared in ``include/attn.h``); ``binding`` marshals torch
tensors to it.  ``workloads`` draws the seeded synthetic inputs.
"""
from .binding import (ATTN_BF16, ATTN_DILUTION, ATTN_F32, ATTN_TEMPERED, AttnError,  # noqa: F401
                      attn_bwd, attn_bwd_workspace_bytes, attn_decode, attn_decode_ex,
                      attn_decode_workspace_bytes, attn_fwd, attn_fwd_ex,
                      attn_fwd_workspace_bytes, attn_prefill, attn_prefill_workspace_bytes,
                      attn_strerror, attn_yarn_tau, bwd, decode, fwd, prefill)
