"""attn_bwd_noalloc (the backward for callers that cannot allocate) against attn_bwd through
the C ABI: the same kernels on the library's fixed scratch, so dQ, dK, dV must be identical
bit for bit. Two calls in a row, the second on a smaller problem, so that the scratch still
holds the first call's statistics when the second runs."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import log

pytestmark = pytest.mark.gpu


def _case(B, N, H, d, dtype, causal, seed):
    from exact_tiled_attention_25_amd import binding
    x = workloads.make_inputs(B, N, H, d, dtype, seed, with_do=True)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = binding.attn_fwd(q, k, v, causal)
    ref = binding.attn_bwd(q, k, v, o, lse, do, causal)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    binding.attn_bwd_noalloc(q, k, v, o, lse, do, causal, dq=got[0], dk=got[1], dv=got[2])
    torch.cuda.synchronize()
    return ref, got


def test_bwd_noalloc_matches_attn_bwd_on_two_calls(lib):
    from exact_tiled_attention_25_amd import binding
    assert binding.attn_bwd_noalloc_max_rows() == 1 << 22
    for (B, N, H, d, dtype, causal, seed) in ((2, 1000, 4, 128, "bf16", True, 71), (1, 300, 2, 64, "fp16", False, 72)):
        log(f"bwd noalloc B={B} N={N} H={H} d={d} {dtype} causal={causal}")
        ref, got = _case(B, N, H, d, dtype, causal, seed)
        for name, r, g in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(r, g), (name, float((r.float() - g.float()).abs().max()))
    # beyond the fixed scratch: a clear error, nothing launched
    q = torch.empty(2, (1 << 17) + 1, 16, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(2, 16, (1 << 17) + 1, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.AttnError) as e:
        binding.attn_bwd_noalloc(q, q, q, q, lse, q, False, dq=q, dk=q, dv=q)
    assert e.value.status == 6
