"""Benchmark of the exact tiled attention hot path on one MI355X.

One step = the whole path on one batch of synthetic input, the bf16 hdim-128 N=8K workload
(B=2, N=8192, H=16, d=128, non-causal, Q/K/V/dO ~ N(0,1)):
  attn_fwd (bf16) -> attn_bwd (bf16) -> attn_fp8_quantize (Q, K rotated; V not) ->
  attn_fwd_fp8 (e4m3 in, bf16 out).
FLOP convention: forward F = 4*B*H*N^2*d (halved when causal), backward 2.5*F, FP8 forward F;
the quantiser counts no FLOPs. value = counted FLOPs of a step / measured step time.

Per-kernel times come from HIP events recorded on the stream the kernels run on, over the
timed steps. `roofline` describes the kernel with the largest share of the step time.
`peak_probe` measures the matrix cores' sustained rate on random and on zero operands and
the cycle cost of the softmax's VALU instructions (libattn_probe.so); `valu_bound` is the
exponential/VALU co-bound of the forward kernels built from those costs (the softmax is
not a contraction, so the MFMA roofline alone does not bound them). `mfma_busy` and the
kernel clock per component come from the rocprofv3 counters stored in profiles/ (null when
the kernel sources have changed since they were taken). `cpu_baseline` times the fp64
oracle on a bounded sample of the same work on the host's cores, before the GPU is touched.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       [--no-peak-probe] [--workload NAME [--seq-len N] [--forward-only]]
       python bench.py --summarize-counters DIR
The default is the workload above. --workload picks another shape of the workload table
(workloads.CONFIGS; its dtype and mask), --seq-len overrides its N (the long-context sweep),
and --forward-only times attn_fwd alone (the short-sequence and small-d cases); stored
counters and the CPU baseline are only reported for the default workload.
--summarize-counters reads the rocprofv3 counter runs under DIR (pmc_fetch, pmc_write,
pmc_mfma: the commands are in profiles/attn_kernels_B2_N8192_H16_d128.md) and writes the
per-kernel and per-component figures to profiles/hbm_counters.json.
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
NOMINAL_CLOCK_GHZ = 2.4
N_SIMD = 1024            # 256 CUs x 4 SIMDs
N_XCD = 8                # GRBM_GUI_ACTIVE is summed over the 8 XCDs
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")
# kernels of each component (name prefix, launches per component call)
COMPONENT_KERNELS = {
    "attn_fwd_bf16": [("fwd_kernel<", 1)],
    "attn_bwd_bf16": [("bwd_", 1)],
    "attn_fp8_quantize_qkv": [("fp8_quant_kernel<", 3)],
    "attn_fwd_fp8": [("fwd_fp8_kernel<", 1)],
}
# VALU work per score element of the forward kernels' softmax, at its minimum: one
# exponential, and the scale-and-subtract FMA, the max, the row-sum add and half a packed
# convert (two scores per convert) on the full-rate VALU.
VALU_PER_SCORE = {"exp": 1.0, "fma": 3.0, "cvt": 0.5}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peak-probe", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=None,
                    help="heads of batch 0 timed on the oracle (default: one per worker process)")
    import workloads
    ap.add_argument("--workload", default=None, choices=sorted(workloads.CONFIGS),
                    help="a workloads.CONFIGS name instead of the default workload")
    ap.add_argument("--seq-len", type=int, default=None, help="override N of --workload")
    ap.add_argument("--forward-only", action="store_true", help="time attn_fwd alone")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration under rocprofv3 --pmc)")
    ap.add_argument("--summarize-counters", metavar="DIR", default=None,
                    help="write profiles/hbm_counters.json from rocprofv3 counter runs under DIR")
    return ap.parse_args()


def source_hash():
    """Hash of the kernel sources, to tell whether stored counters are still current."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_tiled_attention_25_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def stored_counters():
    """Per-component figures from the committed rocprofv3 counter summary, or {} when it is
    missing or was taken on different kernel sources."""
    try:
        rec = json.load(open(PROFILE_COUNTERS))
    except (OSError, ValueError):
        return {}
    if rec.get("source_hash") != source_hash():
        return {}
    return rec.get("components", {})


# ------------------------------------------------------------------ counter summary
def _short(name):
    import re
    m = re.search(r"::([A-Za-z0-9_]+<[^>]*>)\(", name) or re.search(r"([A-Za-z0-9_]+(<[^>]*>)?)\(", name)
    return m.group(1) if m else name


def _read_pmc(path):
    """Mean per dispatch of every counter, and mean dispatch duration (us), per kernel."""
    import csv
    from collections import defaultdict
    per, dur = defaultdict(lambda: defaultdict(float)), {}
    for r in csv.DictReader(open(path)):
        key = (_short(r["Kernel_Name"]), int(r["Dispatch_Id"]))
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        dur[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out = defaultdict(lambda: defaultdict(list))
    for (k, disp), cs in per.items():
        for c, v in cs.items():
            out[k][c].append(v)
        out[k]["dispatch_us"].append(dur[(k, disp)])
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in out.items()}


def summarize_counters(d):
    """profiles/hbm_counters.json from the three counter runs under directory d.

    HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what the same
    counter reads for a plain 1 GiB device copy in the same run. MFMA busy:
    SQ_VALU_MFMA_BUSY_CYCLES (MFMA-occupied cycles summed over the 1024 SIMDs) divided by
    (GRBM_GUI_ACTIVE / 8) x 1024, GRBM_GUI_ACTIVE being the GPU's busy cycles summed over its
    8 XCDs; the clock is GRBM_GUI_ACTIVE / 8 over the dispatch time."""
    import datetime
    fetch = _read_pmc(os.path.join(d, "pmc_fetch", "pmc_counter_collection.csv"))
    write = _read_pmc(os.path.join(d, "pmc_write", "pmc_counter_collection.csv"))
    mfma = _read_pmc(os.path.join(d, "pmc_mfma", "pmc_counter_collection.csv"))
    copyk = [k for k in fetch if "copyBuffer" in k][0]
    gib = 1 << 30
    cal = dict(copy_bytes=gib, fetch_counter_kib=fetch[copyk]["FETCH_SIZE"],
               write_counter_kib=write[copyk]["WRITE_SIZE"])
    cal["fetch_factor"] = gib / (cal["fetch_counter_kib"] * 1024)
    cal["write_factor"] = gib / (cal["write_counter_kib"] * 1024)
    raw = {}
    for k in sorted(set(fetch) | set(mfma)):
        if "copyBuffer" in k:
            continue
        r = {}
        if k in fetch and k in write:
            r.update(fetch_kib=fetch[k]["FETCH_SIZE"], write_kib=write[k]["WRITE_SIZE"])
        if k in mfma:
            r.update({c: v for c, v in mfma[k].items()})
        raw[k] = r
    comps = {}
    for comp, parts in COMPONENT_KERNELS.items():
        ks = [(k, n) for pre, n in parts for k in raw if k.startswith(pre)]
        if not ks:
            continue
        rec = {"kernels": [k for k, _ in ks]}
        if all("fetch_kib" in raw[k] for k, _ in ks):
            rd = sum(raw[k]["fetch_kib"] * 1024 * cal["fetch_factor"] * n for k, n in ks)
            wr = sum(raw[k]["write_kib"] * 1024 * cal["write_factor"] * n for k, n in ks)
            rec.update(hbm_read_bytes=rd, hbm_write_bytes=wr, hbm_bytes_per_launch=rd + wr)
        if all("GRBM_GUI_ACTIVE" in raw[k] for k, _ in ks):
            busy = sum(raw[k].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) * n for k, n in ks)
            cyc = sum(raw[k]["GRBM_GUI_ACTIVE"] / N_XCD * n for k, n in ks)
            us = sum(raw[k]["dispatch_us"] * n for k, n in ks)
            mops = sum((raw[k].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + raw[k].get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)
                        + raw[k].get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)) * n for k, n in ks)
            rec.update(mfma_busy=busy / (cyc * N_SIMD), clock_ghz=cyc / us / 1e3, mfma_flop=mops * 512,
                       counter_dispatch_us=us)
        comps[comp] = rec
    probes = {k: dict(mfma_busy=v["SQ_VALU_MFMA_BUSY_CYCLES"] / (v["GRBM_GUI_ACTIVE"] / N_XCD * N_SIMD),
                      clock_ghz=v["GRBM_GUI_ACTIVE"] / N_XCD / v["dispatch_us"] / 1e3)
              for k, v in raw.items() if k.startswith("mfma_probe_kernel") and "GRBM_GUI_ACTIVE" in v}
    rec = dict(source_hash=source_hash(), date=str(datetime.date.today()), calibration=cal,
               normalisation="mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 * 1024 SIMDs); "
                             "clock = GRBM_GUI_ACTIVE / 8 / dispatch time",
               raw=raw, components=comps, probes=probes)
    json.dump(rec, open(PROFILE_COUNTERS, "w"), indent=1)
    return rec


# ------------------------------------------------------------------ probes
def peak_probe(torch, dev):
    """The matrix cores' sustained rate (dependency-free MFMA loops on random and zero
    operands) and the cycle cost of v_exp_f32, v_fma_f32 and v_cvt_pk_fp8_f32 per wave64
    instruction on one wave per SIMD, with the shader clock seen during that loop."""
    import ctypes
    import numpy as np
    path = os.path.join(ROOT, "exact_tiled_attention_25_amd", "libattn_probe.so")
    L = ctypes.CDLL(path)
    L.probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                             ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
    L.probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream(dev).cuda_stream
    blocks = 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    res = {}
    ms = ctypes.c_float()
    for kind, name, flop, iters in ((0, "bf16", 32 * 32 * 16 * 2, 8192), (1, "fp8", 32 * 32 * 64 * 2, 4096)):
        for zero in (0, 1):
            rc = L.probe_mfma(kind, zero, blocks, iters // 8, stream, out.data_ptr(), ctypes.byref(ms))   # warm
            rc |= L.probe_mfma(kind, zero, blocks, iters, stream, out.data_ptr(), ctypes.byref(ms))
            if rc:
                raise RuntimeError(f"probe_mfma failed ({rc})")
            tf = blocks * 4 * iters * 8 * flop / (ms.value * 1e-3) / 1e12
            res[f"{name}_{'zero' if zero else 'random'}_tflops"] = round(tf, 1)
    buf = torch.empty(3 * 2048, dtype=torch.int64, device=dev)
    iters = 4096
    clocks = []
    # cycles per wave64 instruction per SIMD, with two waves per SIMD (as the attention
    # kernels run); one wave alone issues more slowly
    for wps in (2, 1):
        for op, name in ((0, "exp"), (1, "fma"), (2, "cvt_pk_fp8"), (3, "cvt_pk_bf16")):
            if L.probe_valu(op, iters, wps, stream, buf.data_ptr()):
                raise RuntimeError("probe_valu failed")
            v = buf[:3 * 1024 * wps].view(1024 * wps, 3).cpu().numpy().astype(np.float64)
            cyc, real = np.median(v[:, 0]), np.median(v[:, 1])
            res[f"{name}_cycles" + ("" if wps == 2 else "_one_wave")] = round(cyc / (wps * iters * 16), 2)
            clocks.append(cyc / real * 0.1)   # s_memrealtime runs at 100 MHz
    res["probe_clock_ghz"] = round(float(np.median(clocks)), 3)
    # fp32 atomic adds vs plain stores of 64 x 128 dQ tiles, per (head, 128-key tile): what
    # accumulating dQ from the key-outer pass would cost at B=2 N=8192 H=16 d=128, where
    # every one of the 64 key tiles of a head adds N x d fp32 (8.6 GB in all)
    L.probe_atomic.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                               ctypes.POINTER(ctypes.c_float)]
    ws = torch.zeros(2 * 8192 * 16 * 128, dtype=torch.float32, device=dev)
    nqt = 32
    for mode, name in ((0, "atomic_add_f32"), (1, "store_f32")):
        rc = L.probe_atomic(mode, ws.data_ptr(), 4, stream, ctypes.byref(ms))   # warm
        rc |= L.probe_atomic(mode, ws.data_ptr(), nqt, stream, ctypes.byref(ms))
        if rc:
            raise RuntimeError(f"probe_atomic failed ({rc})")
        res[f"{name}_tbps"] = round(2048 * nqt * 64 * 128 * 4 / (ms.value * 1e-3) / 1e12, 3)
    dq_bytes = 64 * 2 * 16 * 8192 * 128 * 4
    res["dq_atomic_accumulate_ms_bench_shape"] = round(dq_bytes / (res["atomic_add_f32_tbps"] * 1e12) * 1e3, 3)
    # LDS read bytes per clock per CU (8 waves, conflict-free): 16-byte row chunks and the
    # transposed 8-byte reads the P~V and backward products use
    L.probe_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lds_out = torch.empty(256 * 8, dtype=torch.int64, device=dev)
    iters = 2048
    for kind, name, bytes_per in ((0, "lds_read_b128_bytes_per_clk_cu", 1024), (1, "lds_read_tr16_bytes_per_clk_cu", 512)):
        if L.probe_lds(kind, 64, stream, lds_out.data_ptr()) or L.probe_lds(kind, iters, stream, lds_out.data_ptr()):
            raise RuntimeError("probe_lds failed")
        cyc = float(np.median(lds_out.cpu().numpy().astype(np.float64)))
        res[name] = round(bytes_per * iters * 8 * 8 / cyc, 1)
    return res


def valu_bound(scores, probe, t_ms, clock_ghz, fp8):
    """Time the softmax's minimum VALU work takes on the 1024 SIMDs: per score one v_exp_f32,
    three full-rate operations and half a packed convert (to e4m3 or bf16), at the probe's
    cycles per wave64 instruction; at the nominal clock and at the kernel's own clock (from
    its counters)."""
    cvt = probe["cvt_pk_fp8_cycles" if fp8 else "cvt_pk_bf16_cycles"]
    cyc = (VALU_PER_SCORE["exp"] * probe["exp_cycles"] + VALU_PER_SCORE["fma"] * probe["fma_cycles"]
           + VALU_PER_SCORE["cvt"] * cvt) * scores / 64 / N_SIMD
    rec = {"scores": scores, "ops_per_score": VALU_PER_SCORE, "cycles_per_simd": round(cyc),
           "t_min_ms_nominal_clock": round(cyc / NOMINAL_CLOCK_GHZ / 1e6, 4)}
    rec["frac_nominal_clock"] = round(rec["t_min_ms_nominal_clock"] / t_ms, 4)
    if clock_ghz:
        rec["kernel_clock_ghz"] = round(clock_ghz, 3)
        rec["t_min_ms_kernel_clock"] = round(cyc / clock_ghz / 1e6, 4)
        rec["frac_kernel_clock"] = round(rec["t_min_ms_kernel_clock"] / t_ms, 4)
    return rec


# ------------------------------------------------------------------ CPU baseline
def _oracle_head(args):
    """One (batch 0, head h) slice of the step on the oracle, single-threaded."""
    q, k, v, do, causal, with_bwd, with_fp8, seed = args
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        import oracle
        t0 = time.perf_counter()
        oracle.forward(q, k, v, causal)
        if with_bwd:
            oracle.backward(q, k, v, do, causal)
        if with_fp8:
            q8, dq, _ = oracle.quantize_blocks(q, True, seed)
            k8, dk, _ = oracle.quantize_blocks(k, True, seed)
            v8, dv, _ = oracle.quantize_blocks(v, False, seed)
            oracle.fp8_emulated_forward(q8, k8, v8, dq, dk, dv, causal)
        return time.perf_counter() - t0


def _warm_worker(_):
    import oracle  # noqa: F401
    from threadpoolctl import threadpool_limits  # noqa: F401
    return os.getpid()


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, w, heads, active, seed):
    """The fp64 oracle, as it stands, on heads of batch 0 of the same step: one process per
    head (a pool of fresh interpreters, started and closed before this process touches the
    GPU), one BLAS thread each, so the GEMMs and the elementwise work use every worker core.
    The timing covers the work only (the workers have imported the oracle beforehand)."""
    import multiprocessing as mp
    import numpy as np
    nproc = os.cpu_count() or 1
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else nproc
    workers = max(1, min(16, avail))
    heads = min(heads or workers, w["H"])
    N, d, causal = w["N"], w["d"], w["causal"]
    with_bwd = any(n.startswith("attn_bwd_") for n in active)
    with_fp8 = "attn_fwd_fp8" in active
    jobs = [tuple(x[n][:1, :, h:h + 1].float().numpy() for n in ("q", "k", "v", "do"))
            + (causal, with_bwd, with_fp8, seed) for h in range(heads)]
    with mp.get_context("spawn").Pool(min(workers, heads)) as pool:
        pool.map(_warm_worker, range(min(workers, heads)), chunksize=1)   # imports, outside the timing
        t0 = time.perf_counter()
        per = pool.map(_oracle_head, jobs, chunksize=1)
        dt = time.perf_counter() - t0
    f1 = 4.0 * N * N * d * (0.5 if causal else 1.0)
    flops = heads * f1 * (1 + (2.5 if with_bwd else 0) + (1 if with_fp8 else 0))
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOPs/s", "cores": min(workers, heads), "kind": "oracle",
            "seconds": round(dt, 2), "cpu_seconds": round(float(np.sum(per)), 1), "nproc": nproc,
            "cpus_available": avail, "cpu_model": _cpu_model(),
            "sample": f"batch 0, {heads} of {w['H']} heads (N={N}, d={d}) of the same step "
                      f"({'fwd' + (' + bwd' if with_bwd else '') + (' + fp8 quantise + emulated fp8 fwd' if with_fp8 else '')}); "
                      f"numpy fp64, one process per head, one BLAS thread each"}


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.summarize_counters:
        rec = summarize_counters(args.summarize_counters)
        print(json.dumps({"components": rec["components"], "probes": rec["probes"]}, indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (heads shard across GPUs "
              "with no communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads

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
    names = [f"attn_fwd_{dt}"] if args.forward_only else [f"attn_fwd_{dt}", f"attn_bwd_{dt}",
                                                             "attn_fp8_quantize_qkv", "attn_fwd_fp8"]
    seed = 0x5EED
    cpu = None
    if default and not args.no_cpu_baseline:
        cpu = cpu_baseline(x, w, args.cpu_heads, names, seed)   # before any GPU work

    from exact_tiled_attention_25_amd import binding
    binding.load()
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    F = 4.0 * B * H * N * N * d * (0.5 if causal else 1.0)
    scores = B * H * N * N * (0.5 if causal else 1.0)

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
    comps = {n: comps[n] for n in names}
    for name, c in comps.items():   # first call of each: any failure is an error
        c[0]()
        torch.cuda.synchronize()

    for _ in range(args.warmup):
        for c in comps.values():
            c[0]()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for n in comps}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for n, c in comps.items():
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

    stored = stored_counters() if default else {}
    comp_out = {}
    for n, (fn, flops, nbytes, pk) in comps.items():
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev[n]]))
        rec = {"ms": round(ms, 4)}
        if flops:
            tf = flops / (ms * 1e-3) / 1e12
            rec.update(tflops=round(tf, 1), peak_tflops=PEAK_TFLOPS[pk], frac_peak=round(tf / PEAK_TFLOPS[pk], 4))
        rec["algorithmic_hbm_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        s = stored.get(n, {})
        rec["mfma_busy"] = round(s["mfma_busy"], 4) if "mfma_busy" in s else None
        rec["clock_ghz"] = round(s["clock_ghz"], 3) if "clock_ghz" in s else None
        comp_out[n] = rec
    step_flops = sum(c[1] for c in comps.values())
    ms_step = wall / args.steps * 1e3
    value = step_flops / (wall / args.steps) / 1e12

    probe = None
    if not args.no_peak_probe:
        probe = peak_probe(torch, dev)
        for n, rec in comp_out.items():
            pk = comps[n][3]
            if "tflops" in rec and pk:
                ceil = probe["fp8_random_tflops" if pk == "fp8" else "bf16_random_tflops"]
                rec["frac_of_probe_ceiling"] = round(rec["tflops"] / ceil, 4)
    vb = {}
    if probe:
        for n in comps:
            if n.startswith("attn_fwd_"):
                vb[n] = valu_bound(scores, probe, comp_out[n]["ms"], comp_out[n].get("clock_ghz"), n == "attn_fwd_fp8")

    dom = max(comp_out, key=lambda n: comp_out[n]["ms"])
    fn, flops, nbytes, pk = comps[dom]
    ms = comp_out[dom]["ms"]
    if flops:
        ach = flops / (ms * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_TFLOPS[pk],
                "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS[pk], 4)}
    else:
        ach = nbytes / (ms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
    roof["traffic"] = stored.get(dom, {}).get("hbm_bytes_per_launch")
    roof["algorithmic_bytes"] = nbytes
    roof["mfma_busy"] = comp_out[dom]["mfma_busy"]

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOPs/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{dt}+fp8e4m3" if "attn_fwd_fp8" in comps else dt, "data": "synthetic",
        "config": {"workload": wname,
                   "batch": B, "seq_len": N, "heads": H, "head_dim": d, "causal": causal,
                   "parallelism": "single GPU", "step": list(comps)},
        "components": comp_out,
        "roofline": roof,
        "peak_probe": probe,
        "valu_bound": vb or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
