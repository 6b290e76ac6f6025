"""Backward parity on the GPU: attn_bwd through the C ABI against the oracle's analytic
gradients of sum(dO o O).

Bar (target tolerance): for each of dQ, dK, dV, max |g - g_ref| / max |g_ref| <= 5e-2.
As a guard against a near-zero result passing, every case also gates the relative RMSE of
each gradient at 2e-2. The forward inputs (O, LSE) are the GPU forward's own outputs, as in
training; the oracle computes everything from Q, K, V, dO.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import errs, log, to64

pytestmark = pytest.mark.gpu

SMALL = [(1, 128, 2, 64), (2, 200, 3, 64), (1, 333, 2, 128), (2, 129, 2, 256), (1, 1, 1, 128),
         (1, 65, 1, 64), (3, 256, 2, 128), (1, 77, 2, 256), (1, 520, 1, 128)]


def _gpu_bwd(x, causal, scale=None):
    from exact_tiled_attention_25_amd import binding
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = binding.attn_fwd(q, k, v, causal, scale)
    dq, dk, dv = binding.attn_bwd(q, k, v, o, lse, do, causal, scale)
    torch.cuda.synchronize()
    return to64(dq), to64(dk), to64(dv)


def _check(got, ref, tag):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        e = errs(g, r)
        log(f"  {tag} {name}: max_rel={e['max_rel']:.3e} rel_rmse={e['rel_rmse']:.3e}")
        assert np.isfinite(g).all(), name
        assert e["max_rel"] <= 5e-2, (name, e)
        assert e["rel_rmse"] <= 2e-2, (name, e)


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bwd_small_matches_oracle(lib, shape, dtype, causal):
    B, N, H, d = shape
    log(f"bwd small B={B} N={N} H={H} d={d} {dtype} causal={causal}")
    x = workloads.make_inputs(B, N, H, d, dtype, 31, with_do=True)
    got = _gpu_bwd(x, causal)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["do"], causal)
    _check(got, ref, "small")


def test_bwd_c1_both_masks(lib):
    for causal in (False, True):
        log(f"bwd c1 causal={causal}")
        x = workloads.config_inputs("c1")
        _check(_gpu_bwd(x, causal), oracle.backward(x["q"], x["k"], x["v"], x["do"], causal), "c1")


def test_bwd_gradient_invariants(lib):
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i hold for the kernel's output too."""
    log("bwd invariants")
    x = workloads.make_inputs(1, 300, 2, 128, "bf16", 32, with_do=True)
    dq, dk, dv = _gpu_bwd(x, True)
    do = to64(x["do"])
    scale_k = np.abs(dk).sum(axis=1).max()
    assert np.abs(dk.sum(axis=1)).max() <= 2e-2 * scale_k
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), atol=2e-2 * np.abs(do).sum(axis=1).max())


def test_bwd_deterministic_and_workspace_checked(lib):
    log("bwd determinism + workspace")
    from exact_tiled_attention_25_amd import binding
    x = workloads.make_inputs(2, 250, 2, 64, "bf16", 33, with_do=True)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = binding.attn_fwd(q, k, v, True)
    g1 = binding.attn_bwd(q, k, v, o, lse, do, True)
    g2 = binding.attn_bwd(q, k, v, o, lse, do, True)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(binding.AttnError) as e:
        binding.attn_bwd(q, k, v, o, lse, do, True, workspace=small)
    assert e.value.status == 3


# the causal workloads, and the benchmark's non-causal B=2 N=8192 H=16 d=128 shape
FULL = [("c3_d128", True), ("c3_d256", True), ("c2_8192_d128", False)]


@pytest.mark.parametrize("name,causal", FULL, ids=[f[0] for f in FULL])
def test_bwd_full_size_two_heads(lib, name, causal):
    """Full workload on the GPU; two whole heads compared with the oracle."""
    cfg = workloads.CONFIGS[name]
    B, N, H, d = cfg["B"], cfg["N"], cfg["H"], cfg["d"]
    log(f"bwd full {name} B={B} N={N} H={H} d={d} causal={causal}")
    x = workloads.config_inputs(name, with_do=True)
    dq, dk, dv = _gpu_bwd(x, causal)
    for b, h in ((0, 0), (B - 1, H - 1)):
        ref = oracle.head_backward(x["q"][b, :, h], x["k"][b, :, h], x["v"][b, :, h], x["do"][b, :, h], causal)
        _check((dq[b, :, h], dk[b, :, h], dv[b, :, h]), ref, f"{name} b={b} h={h}")


@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("fp16", False)], ids=["bf16-causal", "fp16-full"])
def test_bwd_ragged_default_form_one_head(lib, dtype, causal):
    """Ragged N = 8000 at the benchmark's head count, in the launch configuration of the
    full-size runs; one whole head against the oracle."""
    B, N, H, d = 2, 8000, 16, 128
    log(f"bwd ragged B={B} N={N} H={H} d={d} {dtype} causal={causal}")
    x = workloads.make_inputs(B, N, H, d, dtype, 34, with_do=True)
    dq, dk, dv = _gpu_bwd(x, causal)
    b, h = 1, 9
    ref = oracle.head_backward(x["q"][b, :, h], x["k"][b, :, h], x["v"][b, :, h], x["do"][b, :, h], causal)
    _check((dq[b, :, h], dk[b, :, h], dv[b, :, h]), ref, f"ragged b={b} h={h}")


@pytest.mark.parametrize("shape", [(1, 150, 2, 128), (2, 333, 2, 64), (1, 77, 2, 256)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bwd_writes_nothing_outside_gradients(lib, shape, causal):
    """Canary bytes around dQ, dK and dV stay untouched: each wave writes whole 32-row tiles
    of them through LDS and relies on the buffer range check to drop the rows past N."""
    from exact_tiled_attention_25_amd import binding
    B, N, H, d = shape
    log(f"bwd canary {shape} causal={causal}")
    x = workloads.make_inputs(B, N, H, d, "bf16", 34, with_do=True)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = binding.attn_fwd(q, k, v, causal)
    pad, n = 4096, B * N * H * d
    bufs = [torch.full((2 * pad + n,), 7.0, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    dq, dk, dv = (b[pad:pad + n].view(B, N, H, d) for b in bufs)
    binding.attn_bwd(q, k, v, o, lse, do, causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for name, b in zip(("dq", "dk", "dv"), bufs):
        assert torch.all(b[:pad] == 7.0) and torch.all(b[-pad:] == 7.0), name
    ref = binding.attn_bwd(q, k, v, o, lse, do, causal)
    for a, r in zip((dq, dk, dv), ref):
        assert torch.equal(a, r)
