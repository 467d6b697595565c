"""MI355X (gfx950) RoPE + GQA / causal / sliding-window / MLA attention, and RMSNorm.

The compute runs in the HIP kernels of ``libapex_attn.so``; this package only
marshals torch tensors (device memory and the current stream) into its C ABI
(``include/apex_attn.h``). There is no CPU fallback: without the built library
every call raises.
"""
from ._binding import (APEX_BF16, APEX_F32, ApexError, apex_attn_decode,  # noqa: F401
                       apex_attn_decode_mla, apex_attn_decode_noalloc,
                       apex_attn_decode_workspace_bytes,
                       apex_attn_prefill, apex_attn_prefill_mla, apex_rmsnorm, apex_rope_qk,
                       apex_strerror, lib, lib_path)
