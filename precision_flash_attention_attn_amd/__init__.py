"""Precision flash attention for MI355X (gfx950).

Tiled flash attention with the online safe softmax, forward and backward, BF16
with FP32 accumulation, in three modes: plain BF16 output ("bf16_out"), FP32
output ("fp32_out") and the repeated-maximum-aware safe softmax
("tie_aware_softmax").  The kernels are hand-written HIP behind the C ABI in
include/pfa_attn.h; this package is the thin Python binding.
"""
from ._binding import (DELTA_SRC, LIB_PATH, MODES, AttnError, attn_bwd,  # noqa: F401
                       attn_bwd_noalloc, attn_bwd_noalloc_max_bytes,
                       attn_bwd_delta, attn_bwd_dkdv, attn_bwd_dq, attn_bwd_dq_delta, attn_bwd_prep,
                       attn_bwd_workspace_bytes, attn_delta_error, attn_fwd, attn_fwd_diag, attn_fwd_heads,
                       attn_strerror, backward, forward, forward_heads, lib)

__version__ = "0.1.0"
