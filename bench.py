"""Benchmark of the exact tiled attention hot path on one MI355X.

One step = the whole path on one batch of synthetic input, the bf16 hdim-128 N=8K workload
(B=2, N=8192, H=16, d=128, non-causal, Q/K/V/dO ~ N(0,1)):
  attn_fwd (bf16) -> attn_bwd (bf16) -> attn_fp8_quantize (Q, K rotated; V not) ->
  attn_fwd_fp8 (e4m3 in, bf16 out).
FLOP convention: forward F = 4*B*H*N^2*d (halved when causal), backward 2.5*F, FP8 forward F;
the quantiser counts no FLOPs. value = counted FLOPs of a step / measured step time.

Per-kernel times come from HIP events recorded on the stream the kernels run on, over the
timed steps. `roofline` describes the kernel with the largest share of the step time.
`cpu_baseline` times the fp64 oracle on a bounded sample of the same work on the host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       [--workload NAME [--seq-len N] [--forward-only]]
The default is the workload above. --workload picks another shape of the workload table
(workloads.CONFIGS; its dtype and mask), --seq-len overrides its N (the long-context sweep),
and --forward-only times attn_fwd alone (the short-sequence and small-d cases, for rocprofv3
counter runs); stored HBM counters and the CPU baseline are only reported for the default
workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOPs/s and % of MFMA peak (bf16 & fp8, hdim 128, N=8K)"
WORKLOAD = dict(B=2, N=8192, H=16, d=128, causal=False, dtype="bf16", seed=2)
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp8": 5000.0}   # MI355X dense MFMA, published
PEAK_HBM_GBS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8, help="heads of the workload timed on the oracle")
    import workloads
    ap.add_argument("--workload", default=None, choices=sorted(workloads.CONFIGS),
                    help="a workloads.CONFIGS name instead of the default workload")
    ap.add_argument("--seq-len", type=int, default=None, help="override N of --workload")
    ap.add_argument("--forward-only", action="store_true", help="time attn_fwd alone")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration under rocprofv3 --pmc)")
    return ap.parse_args()


def source_hash():
    """Hash of the kernel sources, to tell whether stored HBM counters are still current."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_tiled_attention_25_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(kernel):
    """HBM bytes per launch of `kernel` (default workload) from the committed rocprofv3
    counter summary, or None when the summary is missing or was taken on different kernel
    sources."""
    try:
        rec = json.load(open(PROFILE_COUNTERS))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (heads shard across GPUs "
              "with no communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads
    from exact_tiled_attention_25_amd import binding

    binding.load()
    dev = torch.device("cuda:0")
    default = args.workload is None and args.seq_len is None and not args.forward_only
    if args.workload is None:
        w = dict(WORKLOAD)
        wname = "attention B=2 N=8192 H=16 d=128 non-causal"
    else:
        c = workloads.CONFIGS[args.workload]
        w = dict(B=c["B"], N=c["N"], H=c["H"], d=c["d"], causal=c["causal"][0], dtype=c["dtype"], seed=c["seed"],
                 input_scale=c.get("input_scale", 1.0), outlier_frac=c.get("outlier_frac", 0.0),
                 outlier_sigma=c.get("outlier_sigma", 10.0))
        wname = args.workload
    if args.seq_len is not None:
        w["N"] = args.seq_len
    B, N, H, d, causal, dt = w["B"], w["N"], w["H"], w["d"], w["causal"], w["dtype"]
    if not default:
        wname = (f"attention {wname}: B={B} N={N} H={H} d={d} {dt} {'causal' if causal else 'non-causal'}"
                 + (", forward only" if args.forward_only else ""))
    else:
        wname += ": bf16 fwd + bwd, fp8 quantize + fwd"
    x = workloads.make_inputs(B, N, H, d, dt, w["seed"], w.get("input_scale", 1.0), w.get("outlier_frac", 0.0),
                              w.get("outlier_sigma", 10.0), with_do=True)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    F = 4.0 * B * H * N * N * d * (0.5 if causal else 1.0)
    seed = 0x5EED

    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(max(binding.attn_bwd_workspace_bytes(B, H, N, d), 1), dtype=torch.uint8, device=dev)
    nblk = (N + 63) // 64
    q8, k8, v8 = (torch.empty(q.shape, dtype=torch.uint8, device=dev) for _ in range(3))
    dsq, dsk, dsv = (torch.empty((B, H, nblk), dtype=torch.float32, device=dev) for _ in range(3))
    o8 = torch.empty_like(q)
    lse8 = torch.empty_like(lse)

    # component name -> (callable, counted flops, algorithmic HBM bytes, peak key)
    elem = B * N * H * d
    comps = {
        f"attn_fwd_{dt}": (lambda: binding.attn_fwd(q, k, v, causal, o=o, lse=lse), F,
                           4 * elem * 2 + B * H * N * 4, dt),
        f"attn_bwd_{dt}": (lambda: binding.attn_bwd(q, k, v, o, lse, do, causal, dq=dq, dk=dk, dv=dv, workspace=ws),
                           2.5 * F, 8 * elem * 2 + B * H * N * 4 * 3, dt),
        "attn_fp8_quantize_qkv": (lambda: (binding.attn_fp8_quantize(q, True, seed, x8=q8, descale=dsq),
                                           binding.attn_fp8_quantize(k, True, seed, x8=k8, descale=dsk),
                                           binding.attn_fp8_quantize(v, False, seed, x8=v8, descale=dsv)),
                                  0.0, 3 * (elem * 2 + elem + B * H * nblk * 4), None),
        "attn_fwd_fp8": (lambda: binding.attn_fwd_fp8(q8, k8, v8, dsq, dsk, dsv, causal, hadamard_seed=seed,
                                                      o=o8, lse=lse8), F,
                         3 * elem + elem * 2 + B * H * N * 4 + 3 * B * H * nblk * 4, "fp8"),
    }
    if args.forward_only:
        comps = {f"attn_fwd_{dt}": comps[f"attn_fwd_{dt}"]}
    active = {}
    for name, c in comps.items():
        try:
            c[0]()
            torch.cuda.synchronize()
            active[name] = c
        except binding.AttnError as e:
            print(f"# {name}: not built ({e})", file=sys.stderr)
    if f"attn_fwd_{dt}" not in active:
        raise SystemExit("forward kernel failed")

    for _ in range(args.warmup):
        for c in active.values():
            c[0]()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for n in active}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for n, c in active.items():
            ev[n][i][0].record(stream)
            c[0]()
            ev[n][i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    comp_out = {}
    for n, (fn, flops, nbytes, pk) in active.items():
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev[n]]))
        rec = {"ms": round(ms, 4)}
        if flops:
            tf = flops / (ms * 1e-3) / 1e12
            rec.update(tflops=round(tf, 1), peak_tflops=PEAK_TFLOPS[pk], frac_peak=round(tf / PEAK_TFLOPS[pk], 4))
        rec["algorithmic_hbm_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        comp_out[n] = rec
    step_flops = sum(c[1] for c in active.values())
    ms_step = wall / args.steps * 1e3
    value = step_flops / (wall / args.steps) / 1e12

    dom = max(comp_out, key=lambda n: comp_out[n]["ms"])
    fn, flops, nbytes, pk = active[dom]
    ms = comp_out[dom]["ms"]
    traffic = stored_traffic(dom) if default else None
    if flops:
        ach = flops / (ms * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_TFLOPS[pk],
                "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS[pk], 4)}
    else:
        ach = nbytes / (ms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
    roof["traffic"] = traffic
    roof["algorithmic_bytes"] = nbytes

    cpu = None
    if default and not args.no_cpu_baseline:
        cpu = cpu_baseline(x, w, args.cpu_heads, list(active), seed)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOPs/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{dt}+fp8e4m3" if "attn_fwd_fp8" in active else dt, "data": "synthetic",
        "config": {"workload": wname,
                   "batch": B, "seq_len": N, "heads": H, "head_dim": d, "causal": causal,
                   "parallelism": "single GPU", "step": list(active)},
        "components": comp_out,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(x, w, heads, active, seed):
    """The fp64 oracle, as it stands, on `heads` heads of batch 0 of the same step."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = 1
    N, d = w["N"], w["d"]
    sub = {n: t[:1, :, :heads] for n, t in x.items()}
    flops = 0.0
    f1 = 4.0 * heads * N * N * d * (0.5 if w["causal"] else 1.0)
    t0 = time.perf_counter()
    oracle.forward(sub["q"], sub["k"], sub["v"], w["causal"])
    flops += f1
    if any(n.startswith("attn_bwd_") for n in active):
        oracle.backward(sub["q"], sub["k"], sub["v"], sub["do"], w["causal"])
        flops += 2.5 * f1
    if "attn_fwd_fp8" in active:
        q8, dq, _ = oracle.quantize_blocks(sub["q"], True, seed)
        k8, dk, _ = oracle.quantize_blocks(sub["k"], True, seed)
        v8, dv, _ = oracle.quantize_blocks(sub["v"], False, seed)
        oracle.fp8_emulated_forward(q8, k8, v8, dq, dk, dv, w["causal"])
        flops += f1
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOPs/s", "cores": int(cores), "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"batch 0, {heads} of {w['H']} heads (N={N}, d={d}) of the same step; "
                      f"numpy fp64, BLAS threads={cores}, elementwise ops single-threaded"}


if __name__ == "__main__":
    main()
