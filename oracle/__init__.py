"""Plain, slow, CPU fp64 oracle for exact attention, its LSE-recompute gradients and the
FP8 (e4m3) block-quantised, Hadamard-rotated forward.

This package is TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The GPU library never calls it, and it
shares no code, constant or helper with the HIP sources: it is written from the pages'
definitions so that it can judge the kernels.

Sources (the three pages about FlashAttention-3):
  * "FlashAttention-3: Hopper Asynchrony and FP8 Attention" (explainer of arXiv 2407.08608):
    Symbol Map; Deep Dive "FP8 accuracy controls" and "Backward warp specialization";
    "Putting It Together" (the epilogue row).
  * "FlashAttention 3 Hardware Acceleration: Hopper GPU Strategies ..." (enterprise post):
    sections "Online Softmax", "FP8 Accumulation", "FP8 Assumptions".
  * Rotary position embedding, which the pages only name as fusable with the Hadamard
    transform, follows Su et al., "RoFormer" (2021); see rope.py.

Pin status of every function is stated in its module docstring; every function here is
pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_*.py``.
"""
from .attention import (forward, forward_rows, backward, head_forward, head_backward,  # noqa: F401
                        head_probs, flops_forward, kv_head, forward_varlen,
                        backward_varlen)
from .fp8 import (e4m3_decode, e4m3_encode, e4m3_finite_values, splitmix64, hadamard_signs,  # noqa: F401
                  sylvester_hadamard, rotation_matrix, quantize_blocks, quantize_per_tensor,
                  dequantize_blocks,
                  fp8_emulated_forward, FP8_BLOCK_ROWS, E4M3_MAX)
from .rope import (apply_rope, rope_frequencies, rope_angles, quantize_rope_blocks,  # noqa: F401
                   ROPE_BASE)
