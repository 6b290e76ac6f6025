"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it draws random numbers and casts them. Both
the GPU library and the oracle receive exactly the tensors it returns (the dtype values,
not the fp32 draws).

Recipe: torch.Generator('cpu').manual_seed(seed); standard-normal fp32 draws of shape
[B, N, H, d] in the order Q, K, V, dO; optional multiplication by `input_scale`; optional
outliers (after each tensor's base draw: U ~ uniform[0,1), Z ~ N(0,1) of the same shape,
and entries with U < outlier_frac become outlier_sigma * Z); finally a cast to the dtype.

The workloads follow the pages' benchmark sweep (sequence lengths 512..16K with a fixed
16K total tokens, head dims 64/128/256) and their synthetic-outlier FP8 accuracy test.
"""
import math

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}

# name -> shape/dtype/seed of each workload. "ragged" entries exercise partial tiles.
CONFIGS = {
    # tiny correctness case the oracle finishes in milliseconds
    "c1": dict(B=1, N=128, H=2, d=64, dtype="bf16", causal=(False, True), seed=1, bwd=True),
    # total tokens 16K, hidden 2048
    "c2_512_d128": dict(B=32, N=512, H=16, d=128, dtype="bf16", causal=(False,), seed=2),
    "c2_2048_d128": dict(B=8, N=2048, H=16, d=128, dtype="bf16", causal=(False,), seed=2),
    "c2_8192_d128": dict(B=2, N=8192, H=16, d=128, dtype="bf16", causal=(False,), seed=2),
    "c2_512_d64": dict(B=32, N=512, H=32, d=64, dtype="bf16", causal=(False,), seed=2),
    "c2_2048_d64": dict(B=8, N=2048, H=32, d=64, dtype="bf16", causal=(False,), seed=2),
    "c2_8192_d64": dict(B=2, N=8192, H=32, d=64, dtype="bf16", causal=(False,), seed=2),
    # causal forward + backward
    "c3_d128": dict(B=2, N=8192, H=16, d=128, dtype="bf16", causal=(True,), seed=3, bwd=True),
    "c3_d256": dict(B=2, N=8192, H=8, d=256, dtype="bf16", causal=(True,), seed=3, bwd=True),
    # long context, fp16, inputs scaled by 0.5
    "c4": dict(B=1, N=32768, H=16, d=128, dtype="fp16", causal=(True,), seed=4, input_scale=0.5),
    # fp8 accuracy with 0.1% N(0,10) outliers
    "c5": dict(B=2, N=8192, H=16, d=128, dtype="bf16", causal=(False,), seed=5,
               outlier_frac=1e-3, outlier_sigma=10.0),
}


def make_inputs(B, N, H, d, dtype="bf16", seed=0, input_scale=1.0, outlier_frac=0.0,
                outlier_sigma=10.0, with_do=False, device="cpu"):
    """Return dict(q, k, v[, do]) of [B, N, H, d] tensors in `dtype` on `device`."""
    g = torch.Generator("cpu").manual_seed(seed)
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    out = {}
    for name in names:
        x = torch.randn((B, N, H, d), generator=g, dtype=torch.float32)
        if outlier_frac > 0:
            u = torch.rand((B, N, H, d), generator=g, dtype=torch.float32)
            z = torch.randn((B, N, H, d), generator=g, dtype=torch.float32)
            x = torch.where(u < outlier_frac, outlier_sigma * z, x)
        if input_scale != 1.0:
            x = x * input_scale
        out[name] = x.to(DTYPES[dtype]).to(device)
    return out


def ragged_lengths(B, mean, seed, min_len=0):
    """B sequence lengths drawn uniformly from [min_len, 2*mean] (seeded): a mixed-length batch."""
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randint(min_len, 2 * mean + 1, (B,), generator=g).tolist()


def make_varlen_inputs(lengths, H, H_kv, d, dtype="bf16", seed=0, with_do=False, pad_rows=0, device="cpu"):
    """Packed variable-length batch: sequences of the given lengths stacked along the token axis
    (plus `pad_rows` trailing rows that belong to no sequence). Returns dict(q [T, H, d],
    k, v [T, H_kv, d][, do [T, H, d]], cu_seqlens int32 [B+1], max_seqlen), drawn in the order
    Q, K, V, dO as standard normals and cast to the dtype."""
    g = torch.Generator("cpu").manual_seed(seed)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    T = cu[-1] + pad_rows
    out = {}
    for name, heads in (("q", H), ("k", H_kv), ("v", H_kv)) + ((("do", H),) if with_do else ()):
        out[name] = torch.randn((T, heads, d), generator=g, dtype=torch.float32).to(DTYPES[dtype]).to(device)
    out["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=device)
    out["max_seqlen"] = max([int(n) for n in lengths], default=0)
    return out


def config_inputs(name, with_do=None, device="cpu", seed=None):
    c = CONFIGS[name]
    return make_inputs(c["B"], c["N"], c["H"], c["d"], c["dtype"], c["seed"] if seed is None else seed,
                       c.get("input_scale", 1.0), c.get("outlier_frac", 0.0), c.get("outlier_sigma", 10.0),
                       with_do=c.get("bwd", False) if with_do is None else with_do, device=device)


def default_scale(d):
    return 1.0 / math.sqrt(d)
