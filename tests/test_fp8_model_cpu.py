"""CPU checks of the FP8 kernel model (tests/fp8_kernel_model.py) before it judges the GPU.

* With the PV operand left unrounded, the model is exact attention on the dequantised
  inputs: it must equal the oracle's emulation to fp64 rounding. This pins the model's own
  bookkeeping (lazy reference per 32-row group, 64-key tiles, V-block weights, the final
  scale dv_max / 64 / l) against the oracle, on inputs whose V blocks have very different
  descales.
* scale = 0 with one V descale: every P~ w is exactly 64, so the rounded model is the
  closed form (prefix) mean of the dequantised V, with L = ln(number of visible keys).
* The model gate the GPU tests use (relative RMSE 3e-3) separates the kernel's arithmetic
  from planted mistakes of the PV stage, and the kernel's choices leave O unbiased on rows
  of many keys (least-squares factor against the emulation).
* Normalising O by the row sum of the rounded operands roughly halves the P-rounding
  error against the emulation compared with the unrounded row sum.
"""
import numpy as np
import pytest

import oracle
import workloads
from fp8_kernel_model import bias_slope, head_model, whole_groups

# gates used by the GPU tests as well: |slope - 1| of O against the emulation, and the
# relative RMSE of the kernel against the model
SLOPE_GATE = 5e-3
MODEL_RMSE = 3e-3


def _codes(B, N, H, d, seed, v_scale_blocks=None, outlier_frac=0.0):
    x = workloads.make_inputs(B, N, H, d, "bf16", seed, outlier_frac=outlier_frac)
    if v_scale_blocks:
        v = x["v"].float()
        for blk, f in v_scale_blocks.items():
            v[:, blk * 64:(blk + 1) * 64] *= f
        x["v"] = v.to(x["v"].dtype)
    cq, dq, _ = oracle.quantize_blocks(x["q"], True, 3)
    ck, dk, _ = oracle.quantize_blocks(x["k"], True, 3)
    cv, dv, _ = oracle.quantize_blocks(x["v"], False, 3)
    return cq, ck, cv, dq, dk, dv


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_unrounded_model_is_the_emulation(causal):
    B, N, H, d = 1, 300, 2, 64
    cq, ck, cv, dq, dk, dv = _codes(B, N, H, d, 21, v_scale_blocks={1: 100.0, 3: 0.01})
    scale = 1 / np.sqrt(d)
    o_ref, l_ref = oracle.fp8_emulated_forward(cq, ck, cv, dq, dk, dv, causal, scale)
    rows = whole_groups(np.arange(N), N)
    for h in range(H):
        o, l = head_model(cq, ck, cv, dq, dk, dv, 0, h, rows, causal, scale, p_round="exact")
        ok = rows < N
        # the coefficient scale*log2e is rounded to fp32 like the kernel's: scores agree to
        # about 1e-7 relative, far below any gate here
        np.testing.assert_allclose(o[ok], o_ref[0, :, h], rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(l[ok], l_ref[0, h], rtol=0, atol=1e-6)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_model_scale_zero_is_the_closed_form(causal):
    B, N, H, d = 1, 200, 1, 128
    x = workloads.make_inputs(B, N, H, d, "bf16", 22)
    cq, dq, _ = oracle.quantize_blocks(x["q"], True, 1)
    ck, dk, _ = oracle.quantize_blocks(x["k"], True, 1)
    cv, dv, _ = oracle.quantize_per_tensor(x["v"], False)
    vd = oracle.dequantize_blocks(cv, dv)[0, :, 0]
    rows = whole_groups(np.arange(N), N)
    o, l = head_model(cq, ck, cv, dq, dk, dv, 0, 0, rows, causal, 0.0)
    ok = rows < N
    n = np.arange(1, N + 1)
    if causal:
        o_ref, l_ref = np.cumsum(vd, 0) / n[:, None], np.log(n)
    else:
        o_ref, l_ref = np.broadcast_to(vd.mean(0), vd.shape), np.full(N, np.log(N))
    np.testing.assert_allclose(o[ok], o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l[ok], l_ref, rtol=0, atol=1e-12)


def test_model_gate_catches_planted_mistakes():
    """The GPU tests gate the kernel against the model at relative RMSE 3e-3. On a workload
    with V blocks of different scale, each plausible mistake of the PV stage moves O by
    far more than that: a round-toward-zero convert of the operand, the power-of-two tile
    scale applied off by one, the V block descales left out of the weights. The kernel's
    choices also leave O unbiased against the emulation on rows of many keys."""
    B, N, H, d = 1, 2048, 1, 128
    cq, ck, cv, dq, dk, dv = _codes(B, N, H, d, 23, v_scale_blocks={3: 8.0, 9: 0.2})
    scale = 1 / np.sqrt(d)
    rows = whole_groups(np.arange(0, N, 7)[:40], N)
    ok, _ = head_model(cq, ck, cv, dq, dk, dv, 0, 0, rows, False, scale)
    o_emul, _ = oracle.fp8_emulated_forward(cq, ck, cv, dq, dk, dv, False, scale)
    assert abs(bias_slope(ok, o_emul[0, rows, 0]) - 1) <= SLOPE_GATE / 3
    flat_dv = np.full_like(dv, dv.max())
    for dvx, kw in ((dv, dict(p_round="rtz")), (dv, dict(e_shift=1)), (dv, dict(e_shift=-1)), (flat_dv, {})):
        o, _ = head_model(cq, ck, cv, dq, dk, dvx, 0, 0, rows, False, scale, **kw)
        rel = np.sqrt(((o - ok) ** 2).mean() / (ok ** 2).mean())
        assert rel > 3 * MODEL_RMSE, (kw, rel)


def test_consistent_normalisation_halves_the_p_rounding_error():
    """O normalised by the row sum of the rounded operands (the kernel's choice) against the
    unrounded row sum: on the outlier workload the P-rounding error against the emulation
    falls by about half (the common error of a row's rounded weights cancels)."""
    B, N, H, d = 1, 2048, 1, 128
    cq, ck, cv, dq, dk, dv = _codes(B, N, H, d, 24, outlier_frac=1e-3)
    scale = 1 / np.sqrt(d)
    rows = whole_groups(np.arange(N), N)
    o_emul, _ = oracle.fp8_emulated_forward(cq, ck, cv, dq, dk, dv, False, scale)
    ref = o_emul[0, :, 0]
    rel = {}
    for lr in (True, False):
        o, _ = head_model(cq, ck, cv, dq, dk, dv, 0, 0, rows, False, scale, l_rounded=lr)
        rel[lr] = np.sqrt(((o - ref) ** 2).mean() / (ref ** 2).mean())
    assert rel[True] < 0.7 * rel[False], rel
