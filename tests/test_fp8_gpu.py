"""FP8 path on the GPU: block quantiser and e4m3 attention against the oracle.

* attn_fp8_quantize vs oracle.quantize_blocks on the same input: descales and codes are
  bit-exact without rotation; with rotation the kernel's fp32 butterfly differs from the
  oracle's fp64 product by a few ulp, so a code may differ by one step, and only where the
  oracle's fp32 quotient lies within 1e-5 (relative) of the midpoint between the two codes.
* attn_fwd_fp8 on the ORACLE's codes and descales vs oracle.fp8_emulated_forward: LSE within
  1e-3 (scores are exact products of the dequantised inputs up to fp32 rounding); O within a
  relative RMSE of 0.06, the budget of rounding P~ to e4m3 (about 2^-4/sqrt(3) = 3.6% rms).
* End to end (GPU quantiser + GPU attention) vs the fp64 oracle on the original bf16 inputs:
  RMSE(O) <= 3e-2 on the 0.1%-outlier workload, with and without the Hadamard rotation.
* attn_fp8_quantize_per_tensor vs oracle.quantize_per_tensor (same code criteria), and the
  four scaling modes (per tensor / per block, with / without rotation) compared end to end.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import errs, log, to64

pytestmark = pytest.mark.gpu


def _binding():
    from exact_tiled_attention_25_amd import binding
    return binding


def _compare_codes(codes_gpu, ds_gpu, x, rotate, seed, quantize=None):
    codes_ref, ds_ref, y = (quantize or oracle.quantize_blocks)(x, rotate, seed)
    if not rotate:
        np.testing.assert_array_equal(ds_gpu, ds_ref)
        np.testing.assert_array_equal(codes_gpu, codes_ref)
        return 0
    np.testing.assert_allclose(ds_gpu, ds_ref, rtol=1e-6, atol=0)
    vg, vr = oracle.e4m3_decode(codes_gpu), oracle.e4m3_decode(codes_ref)
    bad = np.argwhere(vg != vr)
    if len(bad):
        B, N, H, d = x.shape
        dsr = ds_ref[bad[:, 0], bad[:, 2], bad[:, 1] // 64].astype(np.float64)
        scaled = (y[tuple(bad.T)].astype(np.float32) / ds_ref[bad[:, 0], bad[:, 2], bad[:, 1] // 64]).astype(np.float64)
        mid = (vg[tuple(bad.T)] + vr[tuple(bad.T)]) / 2
        # adjacent codes only, and the exact value sits on (or next to) their midpoint
        allv = np.sort(oracle.e4m3_finite_values())
        lo, hi = np.minimum(np.abs(vg[tuple(bad.T)]), np.abs(vr[tuple(bad.T)])), np.maximum(
            np.abs(vg[tuple(bad.T)]), np.abs(vr[tuple(bad.T)]))
        idx = np.searchsorted(allv, lo)
        assert np.all(allv[np.minimum(idx + 1, len(allv) - 1)] == hi), "non-adjacent codes"
        assert np.all(np.abs(scaled - mid) <= 1e-5 * np.abs(mid) + 1e-12), "mismatch away from a midpoint"
        assert len(bad) <= max(2, 1e-4 * codes_gpu.size), len(bad)
        del dsr
    return len(bad)


@pytest.mark.parametrize("shape", [(1, 200, 3, 64), (2, 129, 2, 128), (1, 77, 2, 256), (1, 64, 1, 128), (2, 1, 1, 64)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("rotate", [False, True], ids=["plain", "hadamard"])
def test_quantizer_matches_oracle(lib, shape, dtype, rotate):
    B, N, H, d = shape
    log(f"quant B={B} N={N} H={H} d={d} {dtype} rotate={rotate}")
    x = workloads.make_inputs(B, N, H, d, dtype, 41, outlier_frac=1e-2, outlier_sigma=10.0)["q"]
    if N >= 128:
        x[:, 64:128, 0] = 0                       # an all-zero block -> descale 1, zero codes
    seed = 0xC0FFEE + d
    b = _binding()
    c8, ds = b.attn_fp8_quantize(x.cuda(), rotate, seed)
    torch.cuda.synchronize()
    nbad = _compare_codes(c8.cpu().numpy(), ds.cpu().numpy(), x, rotate, seed)
    log(f"  midpoint flips: {nbad}")


@pytest.mark.parametrize("shape", [(1, 200, 3, 64), (2, 129, 2, 128), (1, 77, 2, 256), (3, 1, 1, 64)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("rotate", [False, True], ids=["plain", "hadamard"])
def test_quantizer_per_tensor_matches_oracle(lib, shape, rotate):
    B, N, H, d = shape
    log(f"quant per-tensor B={B} N={N} H={H} d={d} rotate={rotate}")
    x = workloads.make_inputs(B, N, H, d, "bf16", 43, outlier_frac=1e-2, outlier_sigma=10.0)["q"]
    if N >= 128:
        x[:, 64:128, 0] = 0                       # an all-zero block: zero codes, shared descale
    seed = 0xBEEF + d
    b = _binding()
    c8, ds = b.attn_fp8_quantize_per_tensor(x.cuda(), rotate, seed)
    torch.cuda.synchronize()
    ds = ds.cpu().numpy()
    assert np.all(ds == ds.flat[0])
    nbad = _compare_codes(c8.cpu().numpy(), ds, x, rotate, seed, oracle.quantize_per_tensor)
    log(f"  midpoint flips: {nbad}")


def test_quantizer_per_tensor_all_zero(lib):
    x = torch.zeros(2, 130, 2, 128, dtype=torch.bfloat16)
    c8, ds = _binding().attn_fp8_quantize_per_tensor(x.cuda(), True, 7)
    torch.cuda.synchronize()
    assert torch.all(ds.cpu() == 1.0) and torch.all(c8.cpu() & 0x7F == 0)


def test_quantizer_signs_follow_seed(lib):
    """Different seeds give different codes; the same seed is reproducible."""
    log("quant seeds")
    x = workloads.make_inputs(1, 64, 1, 128, "bf16", 42)["q"].cuda()
    b = _binding()
    a1, _ = b.attn_fp8_quantize(x, True, 1)
    a2, _ = b.attn_fp8_quantize(x, True, 1)
    a3, _ = b.attn_fp8_quantize(x, True, 2)
    assert torch.equal(a1, a2) and not torch.equal(a1, a3)


def _oracle_codes_to_gpu(x, rotate, seed):
    c, ds, _ = oracle.quantize_blocks(x, rotate, seed)
    return c, ds, torch.from_numpy(c).cuda(), torch.from_numpy(ds).cuda()


@pytest.mark.parametrize("shape", [(1, 128, 2, 64), (2, 200, 2, 128), (1, 333, 1, 128), (1, 150, 2, 256),
                                   (1, 1, 1, 64), (1, 500, 1, 64)], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("out", ["bf16", "fp16"])
def test_fwd_fp8_matches_emulation(lib, shape, causal, out):
    B, N, H, d = shape
    log(f"fp8 fwd B={B} N={N} H={H} d={d} causal={causal} out={out}")
    x = workloads.make_inputs(B, N, H, d, "bf16", 43, outlier_frac=1e-3)
    seed = 77
    cq, dq, q8, dq_g = _oracle_codes_to_gpu(x["q"], True, seed)
    ck, dk, k8, dk_g = _oracle_codes_to_gpu(x["k"], True, seed)
    cv, dv, v8, dv_g = _oracle_codes_to_gpu(x["v"], False, seed)
    b = _binding()
    odt = torch.bfloat16 if out == "bf16" else torch.float16
    o, lse = b.attn_fwd_fp8(q8, k8, v8, dq_g, dk_g, dv_g, causal, hadamard_seed=seed, out_dtype=odt)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fp8_emulated_forward(cq, ck, cv, dq, dk, dv, causal)
    eo, el = errs(to64(o), o_ref), errs(to64(lse), l_ref)
    log(f"  O rel_rmse={eo['rel_rmse']:.3e} max_rel={eo['max_rel']:.3e}  LSE max={el['max_abs']:.3e}")
    assert np.isfinite(to64(o)).all()
    assert el["max_abs"] <= 1e-3, el
    assert eo["rel_rmse"] <= 0.06, eo
    assert eo["max_rel"] <= 0.25, eo


def _end_to_end(x, causal, rotate, seed, per_tensor=False):
    b = _binding()
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    q8, dq = b.attn_fp8_quantize(q, rotate, seed, per_tensor=per_tensor)
    k8, dk = b.attn_fp8_quantize(k, rotate, seed, per_tensor=per_tensor)
    v8, dv = b.attn_fp8_quantize(v, False, seed, per_tensor=per_tensor)
    o, lse = b.attn_fwd_fp8(q8, k8, v8, dq, dk, dv, causal, hadamard_seed=seed)
    torch.cuda.synchronize()
    return to64(o), to64(lse)


def test_fp8_end_to_end_c5_rmse_and_hadamard(lib):
    """The outlier workload at full size: RMSE gate against the fp64 oracle on the original
    inputs, with and without the rotation, on sampled rows of several heads."""
    cfg = workloads.CONFIGS["c5"]
    B, N, H, d = cfg["B"], cfg["N"], cfg["H"], cfg["d"]
    log(f"fp8 c5 B={B} N={N} H={H} d={d}")
    x = workloads.config_inputs("c5", with_do=False)
    rng = np.random.default_rng(5)
    heads = [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(6)]
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 200, replace=False)]))
    refs = {bh: oracle.forward_rows(x["q"], x["k"], x["v"], bh[0], bh[1], rows, False) for bh in heads}
    res = {}
    for rotate in (False, True):
        o, lse = _end_to_end(x, False, rotate, seed=0x5EED)
        got = np.concatenate([o[b_, rows, h_] for b_, h_ in heads])
        ref = np.concatenate([refs[(b_, h_)][0] for b_, h_ in heads])
        e = errs(got, ref)
        res[rotate] = e
        log(f"  rotate={rotate}: RMSE={e['rmse']:.4e} relRMSE={e['rel_rmse']:.4e} max={e['max_abs']:.3e}")
        assert e["rmse"] <= 3e-2, e
    log(f"  RMSE ratio (hadamard / plain) = {res[True]['rmse'] / res[False]['rmse']:.4f}")
    assert res[True]["rmse"] < res[False]["rmse"]


def test_fp8_hadamard_gain_across_seeds(lib):
    """The rotation lowers the end-to-end RMSE for every one of five data seeds (50-54)."""
    cfg = workloads.CONFIGS["c5"]
    B, N, H, d = cfg["B"], cfg["N"], cfg["H"], cfg["d"]
    ratios = []
    for seed in range(50, 55):
        log(f"fp8 c5 seed={seed}")
        x = workloads.config_inputs("c5", with_do=False, seed=seed)
        rng = np.random.default_rng(seed)
        heads = [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(3)]
        rows = rng.choice(N, 128, replace=False)
        ref = np.concatenate([oracle.forward_rows(x["q"], x["k"], x["v"], b_, h_, rows, False)[0] for b_, h_ in heads])
        rm = {}
        for rotate in (False, True):
            o, _ = _end_to_end(x, False, rotate, seed=1000 + seed)
            rm[rotate] = errs(np.concatenate([o[b_, rows, h_] for b_, h_ in heads]), ref)["rmse"]
        ratios.append(rm[True] / rm[False])
        log(f"  plain={rm[False]:.4e} hadamard={rm[True]:.4e} ratio={ratios[-1]:.4f}")
    log(f"  ratio mean={np.mean(ratios):.4f} min={np.min(ratios):.4f} max={np.max(ratios):.4f}")
    assert max(ratios) < 1.0


def test_fp8_scaling_modes_compared(lib):
    """The accuracy comparison of the pages' FP8 controls on the outlier workload: one scale
    per tensor vs one per 64-row block, each with and without the Hadamard rotation, as RMSE
    of O against the fp64 oracle on the original inputs (sampled rows of several heads)."""
    cfg = workloads.CONFIGS["c5"]
    B, N, H, d = cfg["B"], cfg["N"], cfg["H"], cfg["d"]
    log(f"fp8 scaling modes c5 B={B} N={N} H={H} d={d}")
    x = workloads.config_inputs("c5", with_do=False)
    rng = np.random.default_rng(7)
    heads = [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(4)]
    rows = rng.choice(N, 160, replace=False)
    ref = np.concatenate([oracle.forward_rows(x["q"], x["k"], x["v"], b_, h_, rows, False)[0] for b_, h_ in heads])
    rm = {}
    for per_tensor in (True, False):
        for rotate in (False, True):
            o, _ = _end_to_end(x, False, rotate, seed=0x5EED, per_tensor=per_tensor)
            e = errs(np.concatenate([o[b_, rows, h_] for b_, h_ in heads]), ref)
            rm[(per_tensor, rotate)] = e["rmse"]
            log(f"  {'per-tensor' if per_tensor else 'per-block '} rotate={rotate}: RMSE={e['rmse']:.4e} "
                f"relRMSE={e['rel_rmse']:.4e}")
    log(f"  per-tensor / block+Hadamard = {rm[(True, False)] / rm[(False, True)]:.4f}")
    assert rm[(False, True)] <= 3e-2 and rm[(False, False)] <= 3e-2
    # the direction the pages report: both controls beat the per-tensor baseline, and the
    # rotation helps under a single scale (the block-vs-rotation ordering is only reported)
    assert rm[(False, True)] < rm[(True, False)]
    assert rm[(True, True)] < rm[(True, False)]


def test_fwd_fp8_full_size_matches_emulation(lib):
    """The benchmark's FP8 launch (B=2, N=8192, H=16, d=128, non-causal, plain N(0,1) inputs)
    on the oracle's own codes and descales: sampled rows of several heads against exact
    attention on the dequantised inputs (LSE within 1e-3, O within the e4m3 P budget)."""
    cfg = workloads.CONFIGS["c2_8192_d128"]
    B, N, H, d = cfg["B"], cfg["N"], cfg["H"], cfg["d"]
    log(f"fp8 fwd full size B={B} N={N} H={H} d={d}")
    x = workloads.config_inputs("c2_8192_d128", with_do=False)
    seed = 0x5EED
    cq, dq, q8, dq_g = _oracle_codes_to_gpu(x["q"], True, seed)
    ck, dk, k8, dk_g = _oracle_codes_to_gpu(x["k"], True, seed)
    cv, dv, v8, dv_g = _oracle_codes_to_gpu(x["v"], False, seed)
    o, lse = _binding().attn_fwd_fp8(q8, k8, v8, dq_g, dk_g, dv_g, False, hadamard_seed=seed)
    torch.cuda.synchronize()
    o, lse = to64(o), to64(lse)
    qd, kd, vd = oracle.dequantize_blocks(cq, dq), oracle.dequantize_blocks(ck, dk), oracle.dequantize_blocks(cv, dv)
    rng = np.random.default_rng(8)
    heads = [(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))]
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 200, replace=False)]))
    got_o, ref_o, dl = [], [], 0.0
    for b_, h_ in heads:
        ro, rl = oracle.forward_rows(qd, kd, vd, b_, h_, rows, False)
        got_o.append(o[b_, rows, h_])
        ref_o.append(ro)
        dl = max(dl, float(np.abs(lse[b_, h_, rows] - rl).max()))
    e = errs(np.concatenate(got_o), np.concatenate(ref_o))
    log(f"  O rel_rmse={e['rel_rmse']:.3e} max_rel={e['max_rel']:.3e}  LSE max={dl:.3e}")
    assert dl <= 1e-3
    assert e["rel_rmse"] <= 0.06, e
