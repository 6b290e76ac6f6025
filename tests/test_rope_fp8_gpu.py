"""Fused RoPE + Hadamard + block-quantise prologue on the GPU against the oracle.

* attn_fp8_quantize_rope vs oracle.quantize_rope_blocks (fp64 RoPE, fp64 rotation, codes
  decided on the fp32 quotient): descales within 1e-6 relative; a code may differ from the
  oracle's only by one step, and only where the oracle's quotient lies within the kernel's
  fp32 error of the midpoint between the two codes. That error is bounded by a few fp32 ulps
  of the row's norm (RoPE and the Hadamard rotation are orthogonal, so no element can carry
  more), which the test takes as 64 * 2^-24 * |x_row|_2 / descale in code units.
* Positions up to 32767 (long context): the angle n * theta is reduced in fp64, so codes at
  the last rows are as exact as at the first.
* End to end (GPU prologue for Q and K, plain quantiser for V, fp8 attention) vs the fp64
  oracle attention on RoPE(Q), RoPE(K), V: RMSE(O) <= 3e-2 on the 0.1%-outlier inputs, at
  B=1 N=2048 H=4 (every row) and at the full outlier workload B=2 N=8192 H=16 (sampled rows).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import errs, log, to64
from oracle import rope as R

pytestmark = pytest.mark.gpu

EPS32 = 2.0 ** -24


def _binding():
    from exact_tiled_attention_25_amd import binding
    return binding


def _compare_codes_rope(codes_gpu, ds_gpu, x, rotate, seed, base):
    codes_ref, ds_ref, y = R.quantize_rope_blocks(x, rotate, seed, base)
    np.testing.assert_allclose(ds_gpu, ds_ref, rtol=1e-6, atol=0)
    vg, vr = oracle.e4m3_decode(codes_gpu), oracle.e4m3_decode(codes_ref)
    bad = np.argwhere(vg != vr)
    if not len(bad):
        return 0
    ix = tuple(bad.T)
    ds_b = ds_ref[bad[:, 0], bad[:, 2], bad[:, 1] // 64]
    scaled = (y[ix].astype(np.float32) / ds_b).astype(np.float64)
    mid = (vg[ix] + vr[ix]) / 2
    allv = np.sort(oracle.e4m3_finite_values())
    lo = np.minimum(np.abs(vg[ix]), np.abs(vr[ix]))
    hi = np.maximum(np.abs(vg[ix]), np.abs(vr[ix]))
    idx = np.searchsorted(allv, lo)
    assert np.all(np.sign(vg[ix]) * np.sign(vr[ix]) >= 0), "codes of opposite sign"
    assert np.all(allv[np.minimum(idx + 1, len(allv) - 1)] == hi), "non-adjacent codes"
    xf = np.asarray(x.double().numpy())
    rownorm = np.sqrt((xf ** 2).sum(-1))[bad[:, 0], bad[:, 1], bad[:, 2]]
    tol = 64 * EPS32 * rownorm / ds_b + 1e-6 * np.abs(mid)
    assert np.all(np.abs(scaled - mid) <= tol), "mismatch away from a midpoint"
    assert len(bad) <= max(4, 1e-4 * codes_gpu.size), len(bad)
    return len(bad)


@pytest.mark.parametrize("shape", [(1, 200, 3, 64), (2, 129, 2, 128), (1, 77, 2, 256), (1, 64, 1, 128),
                                   (2, 1, 1, 64)], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("rotate", [False, True], ids=["plain", "hadamard"])
def test_rope_quantizer_matches_oracle(lib, shape, dtype, rotate):
    B, N, H, d = shape
    log(f"rope quant B={B} N={N} H={H} d={d} {dtype} rotate={rotate}")
    x = workloads.make_inputs(B, N, H, d, dtype, 43, outlier_frac=1e-2, outlier_sigma=10.0)["q"]
    if N >= 128:
        x[:, 64:128, 0] = 0                       # an all-zero block -> descale 1, zero codes
    seed = 0xBEEF + d
    c8, ds = _binding().attn_fp8_quantize_rope(x.cuda(), rotate, seed, 10000.0)
    torch.cuda.synchronize()
    nbad = _compare_codes_rope(c8.cpu().numpy(), ds.cpu().numpy(), x, rotate, seed, 10000.0)
    log(f"  midpoint flips: {nbad}")


@pytest.mark.parametrize("base", [500000.0, 2.0], ids=["base5e5", "base2"])
def test_rope_quantizer_other_bases(lib, base):
    """A long-context base (5e5) and a tiny one (2: every pair turns fast)."""
    B, N, H, d = 1, 300, 2, 128
    log(f"rope quant base={base}")
    x = workloads.make_inputs(B, N, H, d, "bf16", 44)["q"]
    c8, ds = _binding().attn_fp8_quantize_rope(x.cuda(), True, 7, base)
    torch.cuda.synchronize()
    _compare_codes_rope(c8.cpu().numpy(), ds.cpu().numpy(), x, True, 7, base)


def test_rope_quantizer_long_positions(lib):
    """Positions up to 32767 (the long-context length), one head."""
    B, N, H, d = 1, 32768, 1, 128
    log(f"rope quant long B={B} N={N} H={H} d={d}")
    x = workloads.make_inputs(B, N, H, d, "fp16", 4, input_scale=0.5)["q"]
    c8, ds = _binding().attn_fp8_quantize_rope(x.cuda(), True, 11, 10000.0)
    torch.cuda.synchronize()
    nbad = _compare_codes_rope(c8.cpu().numpy(), ds.cpu().numpy(), x, True, 11, 10000.0)
    log(f"  midpoint flips: {nbad}")


def test_rope_position_zero_is_plain_quantiser(lib):
    """Row 0 of each batch is at position 0, where RoPE is the identity: its codes equal the
    plain quantiser's bit for bit (same block amax only if the block is the same, so one
    row per block: N = 1)."""
    x = workloads.make_inputs(3, 1, 4, 128, "bf16", 45)["q"].cuda()
    b = _binding()
    for rotate in (False, True):
        c_r, d_r = b.attn_fp8_quantize_rope(x, rotate, 3, 10000.0)
        c_p, d_p = b.attn_fp8_quantize(x, rotate, 3)
        torch.cuda.synchronize()
        assert torch.equal(c_r, c_p) and torch.equal(d_r, d_p)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_rope_fp8_end_to_end(lib, causal):
    """GPU prologue (RoPE + Hadamard + quantise) on Q and K, plain quantiser on V, fp8 attention;
    against the fp64 oracle attention on RoPE(Q), RoPE(K), V; all rows of all heads."""
    B, N, H, d = 1, 2048, 4, 128
    log(f"rope fp8 e2e B={B} N={N} H={H} d={d} causal={causal}")
    x = workloads.make_inputs(B, N, H, d, "bf16", 46, with_do=False, outlier_frac=1e-3, outlier_sigma=10.0)
    b = _binding()
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    seed = 0x5EED
    q8, dq = b.attn_fp8_quantize_rope(q, True, seed, 10000.0)
    k8, dk = b.attn_fp8_quantize_rope(k, True, seed, 10000.0)
    v8, dv = b.attn_fp8_quantize(v, False, seed)
    o, lse = b.attn_fwd_fp8(q8, k8, v8, dq, dk, dv, causal, hadamard_seed=seed)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.forward(R.apply_rope(x["q"]), R.apply_rope(x["k"]), x["v"], causal)
    e = errs(to64(o), o_ref)
    el = np.abs(to64(lse) - l_ref).max()
    log(f"  RMSE={e['rmse']:.4e} relRMSE={e['rel_rmse']:.4e} max={e['max_abs']:.3e} maxdL={el:.3e}")
    assert e["rmse"] <= 3e-2, e
    assert e["rel_rmse"] <= 0.1, e
    # Without RoPE the scores (and O) differ: the prologue really applied the embedding.
    o_plain, _ = oracle.forward(x["q"], x["k"], x["v"], causal)
    assert errs(to64(o), o_plain)["rel_rmse"] > 3 * e["rel_rmse"]


def test_rope_fp8_full_size_outlier_workload(lib):
    """The FP8 outlier workload at full size (B=2, N=8192, H=16, d=128) through the fused
    prologue: sampled rows of several heads against the fp64 oracle on RoPE(Q), RoPE(K), V."""
    cfg = workloads.CONFIGS["c5"]
    B, N, H, d = cfg["B"], cfg["N"], cfg["H"], cfg["d"]
    log(f"rope fp8 c5 B={B} N={N} H={H} d={d}")
    x = workloads.config_inputs("c5", with_do=False)
    b = _binding()
    seed = 0x5EED
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    q8, dq = b.attn_fp8_quantize_rope(q, True, seed, 10000.0)
    k8, dk = b.attn_fp8_quantize_rope(k, True, seed, 10000.0)
    v8, dv = b.attn_fp8_quantize(v, False, seed)
    o, _ = b.attn_fwd_fp8(q8, k8, v8, dq, dk, dv, False, hadamard_seed=seed)
    torch.cuda.synchronize()
    o = to64(o)
    rng = np.random.default_rng(55)
    heads = [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(3)]
    rows = np.unique(np.concatenate([[0, 1, N - 1], rng.choice(N, 160, replace=False)]))
    qr, kr = R.apply_rope(x["q"]), R.apply_rope(x["k"])
    ref = np.concatenate([oracle.forward_rows(qr, kr, x["v"], b_, h_, rows, False)[0] for b_, h_ in heads])
    got = np.concatenate([o[b_, rows, h_] for b_, h_ in heads])
    e = errs(got, ref)
    log(f"  RMSE={e['rmse']:.4e} relRMSE={e['rel_rmse']:.4e} max={e['max_abs']:.3e}")
    assert e["rmse"] <= 3e-2, e
    assert e["rel_rmse"] <= 0.1, e
