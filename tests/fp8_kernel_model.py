"""CPU model of the FP8 attention kernel's own arithmetic (test code, not the oracle).

The oracle's FP8 emulation is exact attention on the dequantised inputs: it leaves out the
one rounding the kernel adds, the e4m3 rounding of the probabilities before the second
product (page "FlashAttention-3: Hopper Asynchrony and FP8 Attention", Deep Dive "FP8
accuracy controls": P is quantised for the P V product; how is left open). That rounding
costs about 2^-4/sqrt(3) = 3.6% rms of O, so the emulation alone can only gate the kernel
loosely. This model adds exactly that step, in the kernel's order, so that the kernel can
be gated at output-dtype rounding:

  * rows are worked in groups of 32 (one wave), keys in tiles of 64 (one K and one V
    descale block each), tiles in increasing order;
  * the exp2-domain reference m of each row moves only when some row of its group sees a
    tile maximum more than tau = 2.5 above its reference (lazy rescale decided per group);
    O and l are then multiplied by 2^(m_old - m_new);
  * the weight of tile t, 64 * dv_t / dv_max (dv_t the V descale of the key's tile, dv_max
    the head's largest V descale, taken as 1 for an all-zero head), is split as 2^e_t w_t
    with w_t in [32, 64) (w_t = 64, e_t = -127 for a zero descale); the PV operand of key j
    is the e4m3 rounding of P~_j * w_t, with P~_j = 2^(s_j - m), and the product applies
    2^e_t exactly (the matrix core's block scale);
  * two row sums: l of the unrounded P~, and lr of the rounded operands divided by w_t;
  * O = dv_max / 64 * (sum_t 2^e_t sum_j e4m3(P~_j w_t) V8_j) / lr, with V8_j the decoded
    e4m3 codes of V (no descale), so that O's weights are exactly the operands the product
    used, and L = (m + log2 l) ln 2.

Everything else is fp64. The kernel differs from the model by fp32 rounding, by rare e4m3
rounding flips where a product sits within fp32 error of a midpoint, and by the e4m3
matrix core's own addition, which aligns its 64 products to about 12-13 bits below the
largest (measured on the hardware; the accumulator input is added at about 22 bits).
`l_rounded=False` normalises O by l and `pow2=False` puts the whole weight on P~ (the two
choices the kernel did not take; kept to measure them). `p_round`
selects the rounding of the PV operand: "rne" is the kernel's convert; "rtz" is a planted
mistake that the tests use to show that the bias gate catches a systematic error; "exact"
leaves the operand unrounded, which must reproduce the oracle's emulation (a check of the
model's own bookkeeping: lazy reference, weights, tiles).
"""
import numpy as np
import torch

import oracle

TILE = 64
WAVE_ROWS = 32
TAU = 2.5
PSCALE = 64.0
LOG2E = 1.4426950408889634074


def kernel_coefficient(scale):
    """The exp2 coefficient the C ABI forms: fp32(scale * log2 e), from an fp32 scale."""
    return np.float32(np.float64(np.float32(scale)) * LOG2E)


def round_e4m3(x, mode="rne"):
    """Round non-negative values to e4m3 values (fp64): nearest-even or toward zero."""
    x = np.asarray(x, np.float64)
    if mode == "exact":   # no rounding: the model then reduces to exact attention
        return x
    if mode == "rne":
        return oracle.e4m3_decode(oracle.e4m3_encode(x))
    if mode == "rtz":
        vals = oracle.e4m3_finite_values()
        return vals[np.clip(np.searchsorted(vals, x, side="right") - 1, 0, len(vals) - 1)]
    raise ValueError(mode)


def split_weight(w):
    """w = 64 dv/dv_max as (w2, e) with w = w2 * 2^e and w2 in [32, 64) (frexp), the factor
    2^e applied by the matrix core's E8M0 scale; a weight below 64 * 2^-126 is (64, -127)."""
    r = w / PSCALE
    if r < 2.0 ** -126:
        return PSCALE, -127.0
    f, k = np.frexp(r)
    return PSCALE * f, float(k)


def head_model(q8, k8, v8, dq, dk, dv, b, h, rows, causal, scale, p_round="rne", l_rounded=True, pow2=True,
               e_shift=0):
    """Model output for (batch b, head h) at the given rows, which must be whole 32-row
    groups (the lazy rescale couples the rows of a group). The defaults are the kernel's
    choices (see the module docstring). Returns (O fp64 [len, d] before output rounding,
    L fp64 [len]). e_shift != 0 plants a mistake (the scale applied off by that power)."""
    rows = np.asarray(rows)
    assert len(rows) % WAVE_ROWS == 0 and np.all(rows.reshape(-1, WAVE_ROWS)[:, 0] % WAVE_ROWS == 0)
    assert np.all(np.diff(rows.reshape(-1, WAVE_ROWS), axis=1) == 1)
    N = q8.shape[1]
    qd = oracle.e4m3_decode(np.asarray(q8)[b, :, h])
    kd = oracle.e4m3_decode(np.asarray(k8)[b, :, h])
    vd = oracle.e4m3_decode(np.asarray(v8)[b, :, h])
    dqh = np.asarray(dq, np.float32)[b, h]
    dkh = np.asarray(dk, np.float32)[b, h]
    dvh = np.asarray(dv, np.float32)[b, h]
    c = kernel_coefficient(scale)
    valid = rows < N
    rr = np.minimum(rows, N - 1)
    cq = (c * dqh[rr // TILE]).astype(np.float32)                 # per row, fp32
    dvm = np.float64(dvh.max()) if dvh.size else 0.0
    if not dvm > 0:
        dvm = 1.0
    nr, d = len(rows), vd.shape[1]
    m = np.full(nr, -np.inf)
    l = np.zeros(nr)    # row sum of the unrounded P~ (gives L)
    lr = np.zeros(nr)   # row sum of the rounded operands over their weights (normalises O)
    o = np.zeros((nr, d))
    groups = nr // WAVE_ROWS
    for t in range((N + TILE - 1) // TILE):
        k0, k1 = t * TILE, min(N, (t + 1) * TILE)
        coef = (cq * dkh[t]).astype(np.float32).astype(np.float64)  # per row, fp32 product
        x = qd[rr] @ kd[k0:k1].T                                     # exact products of e4m3 values
        s = x * coef[:, None]
        keys = np.arange(k0, k1)[None, :]
        mask = ~valid[:, None] | (causal & (keys > rows[:, None]))
        s = np.where(mask, -np.inf, s)
        mx = s.max(axis=1)
        m_cand = np.maximum(m, mx)
        trig = (m_cand > m + TAU).reshape(groups, WAVE_ROWS).any(axis=1)
        trig = np.repeat(trig, WAVE_ROWS)
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isneginf(m), 0.0, np.exp2(np.where(np.isneginf(m), 0.0, m - m_cand)))
        alpha = np.where(trig, alpha, 1.0)
        m = np.where(trig, m_cand, m)
        o *= alpha[:, None]
        l *= alpha
        lr *= alpha
        w = PSCALE * np.float64(dvh[t]) / dvm
        if pow2:
            w2, e2 = split_weight(w)
        else:   # the whole weight on P~ (floored: a zero block keeps a finite log)
            w2, e2 = max(w, 2.0 ** -100), 0.0
        mu = np.where(np.isneginf(m), 0.0, m)
        p = np.where(mask, 0.0, np.exp2(s - mu[:, None]))
        pr = round_e4m3(p * w2, p_round)
        l += p.sum(axis=1)
        lr += pr.sum(axis=1) / w2
        o += (pr * 2.0 ** (e2 + e_shift)) @ vd[k0:k1]
    with np.errstate(divide="ignore", invalid="ignore"):
        out = o * (dvm / PSCALE) / (lr if l_rounded else l)[:, None]
        lse = (np.where(np.isneginf(m), 0.0, m) + np.log2(l)) * np.log(2.0)
    return out, lse


def round_to(x, dtype):
    """Round fp64 values to a 16-bit dtype ("bf16" or "fp16") and back (RNE)."""
    t = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(x)).to(t).to(torch.float64).numpy()


def whole_groups(rows, N):
    """The 32-row groups that contain the given rows, as one sorted array (rows of the last
    group may lie past N; the model leaves them out of every tile)."""
    starts = np.unique(np.asarray(rows) // WAVE_ROWS) * WAVE_ROWS
    return np.concatenate([np.arange(s0, s0 + WAVE_ROWS) for s0 in starts])


def bias_slope(got, ref):
    """Least-squares factor a minimising |got - a ref|^2: 1 when got is unbiased around ref."""
    got, ref = np.asarray(got, np.float64).ravel(), np.asarray(ref, np.float64).ravel()
    return float(got @ ref / (ref @ ref))
