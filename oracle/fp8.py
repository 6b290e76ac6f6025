"""FP8 (e4m3) forward attention oracle: codec, rotation, block and per-tensor quantisers,
emulated forward.

What is computed (page "FlashAttention-3: Hopper Asynchrony and FP8 Attention", Deep Dive
"FP8 accuracy controls"):
  * Block quantisation: one fp32 scale per Q, K or V block.
  * Incoherent processing: Q and K are both multiplied by the same orthogonal M before
    quantisation, so (QM)(KM)^T = QK^T; M is a product of a random-sign diagonal and a
    Hadamard matrix.
The enterprise post ("FlashAttention 3 Hardware Acceleration", section "FP8 Accumulation")
adds that scale factors are computed in FP32 and that blocks are 64-row tiles; section
"FP8 Assumptions" says Q, K and V are quantised explicitly, with scales, before the call.

Readings where the pages are silent or disagree:
  * e4m3 is OCP E4M3FN: sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinity,
    NaN = S.1111.111, subnormals down to 2^-9, largest finite 448. Encoding is
    round-to-nearest-even with saturation to +-448.
  * A block is 64 consecutive rows of one (batch, head) and the full head dimension d
    (the "natural attention tiles" of the explainer; a split of d would break the single
    contraction over d).
  * descale = fp32(fp32(amax) / 448), and descale = 1 when amax = 0; the stored code is
    RNE of the fp32 quotient fp32(fp32(y) / descale) (the scale arithmetic is fp32, so the
    code is decided on that fp32 value); the dequantised value is decode(code) * descale.
  * M = diag(s) H_d / sqrt(d), H_d the Sylvester Hadamard matrix, one sign vector s per
    call shared by every (batch, head) and by Q and K; s_t = +1 unless the top bit of the
    t-th SplitMix64 output for `seed` is set (then -1). V is never rotated.

Pins (tests/test_oracle_fp8.py): OCP e4m3 facts (max 448, min normal 2^-6, min subnormal
2^-9, 1.0 = 0x38), exhaustive encode/decode round trip over all 256 codes with RNE at every
midpoint and saturation; scipy.linalg.hadamard; M M^T = I; (QM)(KM)^T = QK^T; SplitMix64
against the published reference outputs for seed 0; per-element error bound of the block
quantiser and exact mapping of each block's amax to the +-448 code; the per-tensor
quantiser: same error bound, only the tensor's amax reaches +-448, its descale is the
largest block descale, power-of-two scaling of the input moves only the descale, and on a
single 64-row block it equals the block quantiser.
"""
import numpy as np

from .attention import forward as _forward, _f64

E4M3_MAX = 448.0
FP8_BLOCK_ROWS = 64
_MASK64 = (1 << 64) - 1


def e4m3_decode(codes):
    """Decode e4m3 (OCP E4M3FN) byte codes to fp64 values."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_finite_values():
    """Non-negative finite e4m3 values indexed by code 0x00..0x7E (increasing)."""
    return e4m3_decode(np.arange(0x7F))


def e4m3_encode(x):
    """Saturating round-to-nearest-even encode of real values to e4m3 codes (uint8).

    Ties between two neighbouring codes go to the code with an even mantissa (LSB 0).
    |x| >= 448 saturates to 448; the sign bit follows the sign of x (also for zeros).
    """
    x = np.asarray(x, dtype=np.float64)
    vals = e4m3_finite_values()
    a = np.abs(x)
    lo = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    dlo = a - vals[lo]
    dhi = vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & ((lo & 1) == 1))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.where(np.isnan(x), 0x7F, code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def splitmix64(seed, count):
    """First `count` outputs of the SplitMix64 generator (Steele, Lea and Flood, 2014) seeded
    with `seed`: state += 0x9E3779B97F4A7C15, then the variant-13 finaliser of MurmurHash3."""
    out = []
    state = seed & _MASK64
    for _ in range(count):
        state = (state + 0x9E3779B97F4A7C15) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def hadamard_signs(seed, d):
    """Random sign vector s in {+1,-1}^d: s_t = -1 iff the top bit of output t is set."""
    return np.array([-1.0 if (z >> 63) else 1.0 for z in splitmix64(seed, d)])


def sylvester_hadamard(d):
    """H_1 = [1]; H_2n = [[H_n, H_n], [H_n, -H_n]] (entries +-1, d a power of two)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation_matrix(d, seed):
    """The orthogonal M = diag(s) H_d / sqrt(d) applied to rows of Q and K (x -> x M)."""
    return hadamard_signs(seed, d)[:, None] * sylvester_hadamard(d) / np.sqrt(d)


def quantize_blocks(x, rotate, seed=0, block=FP8_BLOCK_ROWS):
    """Quantise x [B, N, H, d] to e4m3 codes with one fp32 descale per 64-row block per head.

    Returns (codes uint8 [B, N, H, d], descale float32 [B, H, ceil(N/64)], y fp64) where y
    is the rotated (or unrotated) input in fp64, i.e. the value each code approximates
    as decode(code) * descale.
    """
    x = _f64(x)
    B, N, H, d = x.shape
    y = x @ rotation_matrix(d, seed) if rotate else x.copy()
    nblk = (N + block - 1) // block
    codes = np.empty(x.shape, dtype=np.uint8)
    descale = np.empty((B, H, nblk), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for j in range(nblk):
                tile = y[b, j * block:(j + 1) * block, h]
                amax = np.float32(np.abs(tile).max())
                ds = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
                descale[b, h, j] = ds
                scaled = tile.astype(np.float32) / ds          # fp32 / fp32, correctly rounded
                codes[b, j * block:(j + 1) * block, h] = e4m3_encode(scaled.astype(np.float64))
    return codes, descale, y


def quantize_per_tensor(x, rotate, seed=0, block=FP8_BLOCK_ROWS):
    """Quantise x [B, N, H, d] to e4m3 codes with ONE fp32 descale for the whole tensor.

    The per-tensor baseline that block quantisation is compared with (explainer, "FP8
    accuracy controls"; enterprise post, "FP8 Accumulation" and "FP8 Validation": block
    scales instead of a single scale for the entire tensor). amax runs over every element
    of the (rotated) tensor, all batches and heads; descale and codes follow the same fp32
    arithmetic as quantize_blocks. The descale is returned in the block layout
    [B, H, ceil(N/64)] with every entry equal, so dequantize_blocks and
    fp8_emulated_forward take it unchanged. Returns (codes, descale, y) like quantize_blocks.
    """
    x = _f64(x)
    B, N, H, d = x.shape
    y = x @ rotation_matrix(d, seed) if rotate else x.copy()
    amax = np.float32(np.abs(y).max()) if y.size else np.float32(0.0)
    ds = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    codes = e4m3_encode((y.astype(np.float32) / ds).astype(np.float64))
    descale = np.full((B, H, (N + block - 1) // block), ds, dtype=np.float32)
    return codes, descale, y


def dequantize_blocks(codes, descale, block=FP8_BLOCK_ROWS):
    """decode(code) * descale of the code's block, fp64 [B, N, H, d]."""
    codes = np.asarray(codes)
    B, N, H, d = codes.shape
    rows = np.arange(N) // block
    ds = np.asarray(descale, dtype=np.float64)[:, :, rows]          # [B, H, N]
    return e4m3_decode(codes) * np.transpose(ds, (0, 2, 1))[..., None]


def fp8_emulated_forward(q8, k8, v8, dq, dk, dv, causal=False, scale=None):
    """Exact fp64 attention on the dequantised e4m3 inputs (Q and K in the rotated basis).

    This isolates kernel error from input-quantisation error: it is what the FP8 kernel
    would return if its only rounding were the input quantisation.
    """
    return _forward(dequantize_blocks(q8, dq), dequantize_blocks(k8, dk), dequantize_blocks(v8, dv),
                    causal, scale)
