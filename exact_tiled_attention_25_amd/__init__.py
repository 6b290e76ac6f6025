"""Exact tiled attention for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library libattn.so (hand-written HIP kernels, see
include/attn.h); ``binding`` is its thin ctypes wrapper over torch tensors.
"""
from .binding import (attn_fwd, attn_bwd, attn_bwd_workspace_bytes, attn_fp8_quantize,  # noqa: F401
                      attn_fwd_fp8, AttnError, load)
