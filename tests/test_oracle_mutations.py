"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case swaps one oracle function for a plausibly wrong variant and checks that at least
one of the pin tests then fails. This guards the pins themselves: a pin that passes for a
broken oracle would not protect the GPU parity tests.
"""
import numpy as np
import pytest

import oracle
from oracle import attention as A
from oracle import fp8 as F
import test_oracle_attention as TA
import test_oracle_fp8 as TF


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _scores_flipped_mask(qh, kh, rows, causal, scale):
    s = scale * (qh[rows] @ kh.T)
    if causal:
        keys = np.arange(kh.shape[0])[None, :]
        s = np.where(keys < rows[:, None], -np.inf, s)
    return s


def _scores_no_scale(qh, kh, rows, causal, scale):
    return _ORIG_SCORES(qh, kh, rows, causal, 1.0)


_ORIG_SCORES = A._scores
_ORIG_HEAD_FWD = A.head_forward
_ORIG_HEAD_BWD = A.head_backward


def _fwd_log2(*a, **k):
    o, lse = _ORIG_HEAD_FWD(*a, **k)
    return o, lse / np.log(2.0)


def _bwd_dv_transposed(qh, kh, vh, doh, causal=False, scale=None):
    dq, dk, dv = _ORIG_HEAD_BWD(qh, kh, vh, doh, causal, scale)
    p = A.head_probs(qh, kh, causal, scale)
    return dq, dk, p @ A._f64(doh)


def _bwd_dk_unscaled(qh, kh, vh, doh, causal=False, scale=None):
    dq, dk, dv = _ORIG_HEAD_BWD(qh, kh, vh, doh, causal, scale)
    sc = A._default_scale(A._f64(qh).shape[1], scale)
    return dq, dk / sc, dv


def _bwd_d_sign(qh, kh, vh, doh, causal=False, scale=None):
    qh, kh, vh, doh = (A._f64(x) for x in (qh, kh, vh, doh))
    sc = A._default_scale(qh.shape[1], scale)
    p = A.head_probs(qh, kh, causal, sc)
    dp = doh @ vh.T
    ds = p * (dp + (p * dp).sum(1, keepdims=True))
    return sc * ds @ kh, sc * ds.T @ qh, p.T @ doh


def _kv_head_interleaved(h, H, Hkv):
    return h % Hkv


def _varlen_as_one_sequence(q, k, v, cu_seqlens, causal=False, scale=None):
    o, lse = A.forward(A._f64(q)[None], A._f64(k)[None], A._f64(v)[None], causal, scale)
    return o[0], lse[0]


ATTN_CASES = {
    "grouped heads interleaved": ("kv_head", _kv_head_interleaved),
    "packed sequences attend across": ("forward_varlen", _varlen_as_one_sequence),
    "flipped causal mask": ("_scores", _scores_flipped_mask),
    "dropped scale": ("_scores", _scores_no_scale),
    "log2 lse": ("head_forward", _fwd_log2),
    "dV not transposed": ("head_backward", _bwd_dv_transposed),
    "dK missing scale": ("head_backward", _bwd_dk_unscaled),
    "D with wrong sign": ("head_backward", _bwd_d_sign),
}


def _attention_pins():
    return [
        (TA.test_forward_matches_torch_math_attention, (2, 5, 2, 8), True, 0.37),
        (TA.test_forward_matches_torch_math_attention, (1, 33, 3, 16), False, 0.37),
        (TA.test_lse_and_probs_match_scipy, True),
        (TA.test_backward_matches_torch_autograd, (1, 33, 3, 16), True),
        (TA.test_backward_matches_torch_autograd, (2, 5, 2, 8), False),
        (TA.test_backward_finite_differences, 8, 8, True),
        (TA.test_grouped_kv_heads_match_torch, 2, True),
        (TA.test_varlen_sequences_are_isolated, True),
        (TA.test_varlen_closed_forms,),
    ]


@pytest.mark.parametrize("name", list(ATTN_CASES))
def test_attention_mutation_is_caught(monkeypatch, name):
    attr, bad = ATTN_CASES[name]
    monkeypatch.setattr(A, attr, bad)
    monkeypatch.setattr(oracle, attr, bad, raising=False)
    assert any(_fails(fn, *args) for fn, *args in _attention_pins()), name



_ORIG_DECODE = F.e4m3_decode
_ORIG_ENCODE = F.e4m3_encode


def _decode_wrong_bias(codes):
    return _ORIG_DECODE(codes) * 0.5


def _encode_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    vals = F.e4m3_finite_values()
    a = np.abs(x)
    lo = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    code = np.where(vals[hi] - a <= a - vals[lo], hi, lo)
    code = np.where(a >= 448.0, 0x7E, code) | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def _rotation_unnormalised(d, seed):
    return F.hadamard_signs(seed, d)[:, None] * F.sylvester_hadamard(d)


def _per_tensor_scale_per_head(x, rotate, seed=0, block=F.FP8_BLOCK_ROWS):
    """One scale per (batch, head) slice instead of one for the whole tensor."""
    x = F._f64(x)
    codes = np.empty(x.shape, dtype=np.uint8)
    B, N, H, d = x.shape
    descale = np.empty((B, H, (N + block - 1) // block), dtype=np.float32)
    y = np.empty_like(x)
    for b in range(B):
        for h in range(H):
            c, ds, yy = _ORIG_PER_TENSOR(x[b:b + 1, :, h:h + 1], rotate, seed, block)
            codes[b, :, h], descale[b, h], y[b, :, h] = c[0, :, 0], ds[0, 0], yy[0, :, 0]
    return codes, descale, y


def _per_tensor_amax_before_rotation(x, rotate, seed=0, block=F.FP8_BLOCK_ROWS):
    """The scale taken from the input before the rotation."""
    codes, descale, y = _ORIG_PER_TENSOR(x, rotate, seed, block)
    ds = np.float32(np.float32(np.abs(F._f64(x)).max()) / np.float32(F.E4M3_MAX))
    return F.e4m3_encode((y.astype(np.float32) / ds).astype(np.float64)), np.full_like(descale, ds), y


_ORIG_PER_TENSOR = F.quantize_per_tensor

FP8_CASES = {
    "e4m3 bias 8": ("e4m3_decode", _decode_wrong_bias),
    "round half up": ("e4m3_encode", _encode_half_up),
    "Hadamard without 1/sqrt(d)": ("rotation_matrix", _rotation_unnormalised),
    "per-tensor scale per head": ("quantize_per_tensor", _per_tensor_scale_per_head),
    "per-tensor amax before rotation": ("quantize_per_tensor", _per_tensor_amax_before_rotation),
}


def _fp8_pins():
    return [
        (TF.test_e4m3_ocp_fixed_points,),
        (TF.test_e4m3_midpoints_round_to_even_and_neighbours_to_nearest,),
        (TF.test_rotation_is_orthogonal_and_preserves_scores, 128),
        (TF.test_per_tensor_quantizer, False),
        (TF.test_per_tensor_quantizer, True),
    ]


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_fp8_mutation_is_caught(monkeypatch, name):
    attr, bad = FP8_CASES[name]
    monkeypatch.setattr(F, attr, bad)
    monkeypatch.setattr(oracle, attr, bad)
    assert any(_fails(fn, *args) for fn, *args in _fp8_pins()), name


from oracle import rope as RP  # noqa: E402
import test_oracle_rope as TR  # noqa: E402

_ORIG_FREQ = RP.rope_frequencies


def _rope_half_split(x, base=RP.ROPE_BASE):
    """Pairs (x_i, x_{i+d/2}) instead of adjacent pairs."""
    x = RP._f64(x)
    d = x.shape[-1]
    perm = np.stack([np.arange(d // 2), np.arange(d // 2) + d // 2], axis=1).reshape(-1)
    y = np.empty_like(x)
    y[..., perm] = _ORIG_ROPE(x[..., perm], base)
    return y


def _rope_negative_angle(x, base=RP.ROPE_BASE):
    x = RP._f64(x)
    flip = x.copy()
    flip[..., 1::2] *= -1
    y = _ORIG_ROPE(flip, base)
    y[..., 1::2] *= -1
    return y


def _rope_from_position_one(x, base=RP.ROPE_BASE):
    x = RP._f64(x)
    pad = np.concatenate([np.zeros_like(x[:, :1]), x], axis=1)
    return _ORIG_ROPE(pad, base)[:, 1:]


def _freq_exponent_i_over_d(d, base=RP.ROPE_BASE):
    return np.power(float(base), -np.arange(d // 2, dtype=np.float64) / d)


_ORIG_ROPE = RP.apply_rope

ROPE_CASES = {
    "half-split pairs": ("apply_rope", _rope_half_split),
    "rotation by minus the angle": ("apply_rope", _rope_negative_angle),
    "positions start at 1": ("apply_rope", _rope_from_position_one),
    "frequency exponent i/d": ("rope_frequencies", _freq_exponent_i_over_d),
}


def _rope_pins():
    return [
        (TR.test_frequency_table_closed_values,),
        (TR.test_rope_is_complex_multiplication, 64),
        (TR.test_rope_is_the_exponential_of_its_generator,),
        (TR.test_position_zero_is_identity_and_norms_are_kept,),
        (TR.test_scores_depend_only_on_relative_position,),
    ]


@pytest.mark.parametrize("name", list(ROPE_CASES))
def test_rope_mutation_is_caught(monkeypatch, name):
    attr, bad = ROPE_CASES[name]
    monkeypatch.setattr(RP, attr, bad)
    assert any(_fails(fn, *args) for fn, *args in _rope_pins()), name
