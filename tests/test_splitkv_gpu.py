"""Split-KV forward on the GPU (attn_fwd_splitkv) against the fp64 oracle.

Each query tile's key tiles are cut into num_splits parts whose (O/l, L) the merge joins by
log-sum-exp, so the result must meet the forward's bar: max |dO| <= 1e-2, max |dLSE| <= 1e-3
and relative RMSE of O <= 1e-2. The cases include more parts than key tiles (empty parts,
and under the causal mask parts that hold no key of some rows), ragged N, N = 1, every head
dimension, and the short-N long-context shapes the split is meant for.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import errs, log, to64

pytestmark = pytest.mark.gpu

CASES = [  # (B, N, H, d, num_splits)
    (1, 200, 3, 64, 1), (1, 200, 3, 64, 2), (1, 200, 3, 64, 16), (2, 129, 2, 128, 4), (1, 77, 2, 256, 2),
    (1, 1, 1, 64, 5), (1, 1000, 2, 128, 7), (2, 333, 1, 128, 3), (1, 600, 2, 256, 16),
]


def _binding():
    from exact_tiled_attention_25_amd import binding
    return binding


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_splitkv_small_matches_oracle(lib, case, causal):
    B, N, H, d, S = case
    for dtype in ("bf16", "fp16"):
        log(f"splitkv B={B} N={N} H={H} d={d} S={S} {dtype} causal={causal}")
        x = workloads.make_inputs(B, N, H, d, dtype, seed=31)
        q, k, v = (x[n].cuda() for n in "qkv")
        o, lse = _binding().attn_fwd_splitkv(q, k, v, S, causal=causal)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], causal)
        eo, el = errs(to64(o), o_ref), errs(to64(lse), l_ref)
        assert eo["max_abs"] <= 1e-2 and el["max_abs"] <= 1e-3 and eo["rel_rmse"] <= 1e-2, (eo, el)


@pytest.mark.parametrize("N,S", [(1024, 4), (2048, 2), (4096, 2)])
def test_splitkv_short_context_sampled_rows(lib, N, S):
    """The long-context fp16 causal workload (inputs x 0.5) at the short lengths of its sweep,
    where one workgroup per query tile leaves most CUs idle."""
    B, H, d = 1, 16, 128
    log(f"splitkv short-N B={B} N={N} H={H} d={d} S={S}")
    x = workloads.make_inputs(B, N, H, d, "fp16", seed=4, input_scale=0.5)
    q, k, v = (x[n].cuda() for n in "qkv")
    o, lse = _binding().attn_fwd_splitkv(q, k, v, S, causal=True)
    o, lse = to64(o), to64(lse)
    rng = np.random.default_rng(9)
    got, ref, worst_l = [], [], 0.0
    for h in (0, 7, 15):
        rows = np.array(sorted(set(rng.choice(N, 80, replace=False).tolist()) | {0, 1, N - 1}))
        o_ref, l_ref = oracle.forward_rows(x["q"], x["k"], x["v"], 0, h, rows, True)
        got.append(o[0, rows, h]); ref.append(o_ref)
        worst_l = max(worst_l, np.abs(lse[0, h, rows] - l_ref).max())
    e = errs(np.concatenate(got), np.concatenate(ref))
    log(f"  max|dO|={e['max_abs']:.3e} max|dL|={worst_l:.3e} relRMSE={e['rel_rmse']:.3e}")
    assert e["max_abs"] <= 1e-2 and worst_l <= 1e-3 and e["rel_rmse"] <= 1e-2


def test_splitkv_matches_attn_fwd_and_is_deterministic(lib):
    log("splitkv vs attn_fwd")
    x = workloads.make_inputs(2, 700, 2, 128, "bf16", 33)
    q, k, v = (x[n].cuda() for n in "qkv")
    b = _binding()
    o0, l0 = b.attn_fwd(q, k, v, causal=True)
    o1, l1 = b.attn_fwd_splitkv(q, k, v, 3, causal=True)
    o2, l2 = b.attn_fwd_splitkv(q, k, v, 3, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert (o1.float() - o0.float()).abs().max().item() <= 1e-2
    assert (l1 - l0).abs().max().item() <= 1e-4


def test_splitkv_writes_nothing_outside_outputs(lib):
    """Canary bytes around O, LSE and the workspace stay untouched."""
    log("splitkv canary")
    B, N, H, d, S = 1, 150, 2, 128, 3
    x = workloads.make_inputs(B, N, H, d, "bf16", 34)
    b = _binding()
    pad = 4096
    need = b.attn_fwd_splitkv_workspace_bytes(B, H, N, d, S)
    assert need == S * B * H * N * (d + 1) * 4
    o_buf = torch.full((pad * 2 + B * N * H * d,), 7.0, dtype=torch.bfloat16, device="cuda")
    l_buf = torch.full((pad * 2 + B * H * N,), 7.0, dtype=torch.float32, device="cuda")
    w_buf = torch.full((pad * 2 + need,), 0x5A, dtype=torch.uint8, device="cuda")
    o = o_buf[pad:pad + B * N * H * d].view(B, N, H, d)
    lse = l_buf[pad:pad + B * H * N].view(B, H, N)
    b.attn_fwd_splitkv(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), S, causal=True, o=o, lse=lse,
                       workspace=w_buf[pad:pad + need])
    torch.cuda.synchronize()
    assert torch.all(o_buf[:pad] == 7.0) and torch.all(o_buf[-pad:] == 7.0)
    assert torch.all(l_buf[:pad] == 7.0) and torch.all(l_buf[-pad:] == 7.0)
    assert torch.all(w_buf[:pad] == 0x5A) and torch.all(w_buf[-pad:] == 0x5A)
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], True)
    assert errs(to64(o), o_ref)["max_abs"] <= 1e-2 and errs(to64(lse), l_ref)["max_abs"] <= 1e-3


def test_splitkv_rejects_bad_arguments(lib):
    b = _binding()
    q = torch.zeros(1, 64, 1, 64, dtype=torch.bfloat16, device="cuda")
    for s in (0, 17):
        with pytest.raises(b.AttnError) as e:
            b.attn_fwd_splitkv(q, q, q, s, workspace=torch.empty(1 << 20, dtype=torch.uint8, device="cuda"))
        assert e.value.status == 1
    with pytest.raises(b.AttnError) as e:
        b.attn_fwd_splitkv(q, q, q, 2, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == 3
