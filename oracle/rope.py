"""Rotary position embedding (RoPE) for the fused RoPE + Hadamard + quantise prologue.

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU baseline use it.

The explainer page ("FlashAttention-3: Hopper Asynchrony and FP8 Attention", Deep Dive "FP8
accuracy controls") says that the random-sign Hadamard transform of Q and K can be fused with
rotary embedding, and the enterprise post (torch.compile integration) names the same fusion.
Neither page defines the embedding. Reading taken: the rotary position embedding of Su et al.,
"RoFormer: Enhanced Transformer with Rotary Position Embedding" (2021):

  * the head dimension is split into d/2 adjacent pairs (x_{2i}, x_{2i+1});
  * pair i has frequency theta_i = base^(-2i/d) (base 10000 unless given);
  * the row at position m (its 0-based index within its sequence) has each pair rotated by
    the angle m * theta_i:  (a, b) -> (a cos - b sin, a sin + b cos).

Applied to Q and K (not V) before the Hadamard rotation: both are orthogonal, so the scores
are those of RoPE attention, q_m^T R(n - m) k_n.

Pinned (tests/test_oracle_rope.py) by the complex-number form of the same rotation, the
relative-position property, norm preservation, position 0, the frequency table's closed
values, and brute force on a tiny case.
"""
import numpy as np

ROPE_BASE = 10000.0


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def rope_frequencies(d, base=ROPE_BASE):
    """theta_i = base^(-2i/d) for the d/2 pairs, fp64."""
    if d % 2:
        raise ValueError("RoPE needs an even head dimension")
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def rope_angles(positions, d, base=ROPE_BASE):
    """Angle of pair i at each position: [len(positions), d/2] fp64."""
    return np.asarray(positions, dtype=np.float64)[:, None] * rope_frequencies(d, base)[None, :]


def apply_rope(x, base=ROPE_BASE):
    """x [B, N, H, d] (row n of each batch at position n) -> RoPE(x), fp64."""
    x = _f64(x)
    B, N, H, d = x.shape
    ang = rope_angles(np.arange(N), d, base)          # [N, d/2]
    c = np.cos(ang)[None, :, None, :]
    s = np.sin(ang)[None, :, None, :]
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def quantize_rope_blocks(x, rotate, seed=0, base=ROPE_BASE):
    """The fused prologue's result: RoPE, then (if rotate) the random-sign Hadamard rotation,
    then 64-row block e4m3 quantisation, each step as the oracle defines it on its own.
    Returns (codes, descale, y) as quantize_blocks does, y being the rotated RoPE(x)."""
    from .fp8 import quantize_blocks
    return quantize_blocks(apply_rope(x, base), rotate, seed)
