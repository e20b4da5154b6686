#!/usr/bin/env python3
"""Throughput of the whole hot path -- causal GQA RoPE attention forward + backward -- on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one forward call (operand preparation + attention) and one backward call
(preparation with Delta + dK/dV + dQ) over one batch of synthetic inputs already resident in
HBM.  Throughput counts algorithmic causal FLOPs only (unmasked (query, key) pairs,
N = T(T+1)/2 per head): forward 4*B*Hq*D*N, backward 10*B*Hq*D*N, step 14*B*Hq*D*N.
Per-kernel durations come from HIP events recorded by the library around each launch on the
stream it launches on; the whole-step time from the host clock around K synchronised steps.
Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_F16 = 2516.6    # TFLOP/s: 256 CUs x 4096 flop/clk x 2.4 GHz, dense fp16/bf16
MFMA_PEAK_F32 = 157.3     # TFLOP/s, dense fp32 MFMA
HBM_PEAK = 8000.0         # GB/s
METRIC = "causal GQA attention TFLOP/s fwd+bwd (1 MI355X) + % of MFMA peak"
KERNEL_SOURCES = ["causal_gqa_flashattention_rope_amd/csrc/ne_kernels.hip",
                  "causal_gqa_flashattention_rope_amd/csrc/ne_common.hpp"]


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^\s*([a-z_]+):\s*(\S+)\s*$", line)
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, sample_B):
    """Time the oracle (as it stands) on the first `sample_B` batch elements of the workload."""
    import oracle
    from causal_gqa_flashattention_rope_amd import inputs
    q, k, v, dO = (t[:sample_B].double().numpy() for t in inputs.make_inputs(w))
    t0 = time.perf_counter()
    oracle.fwd(q, k, v, w.rope_base)
    oracle.bwd(q, k, v, dO, w.rope_base)
    dt = time.perf_counter() - t0
    N = w.T * (w.T + 1) / 2
    flops = 14.0 * sample_B * w.Hq * w.D * N
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"fwd+bwd of batch elements 0..{sample_B - 1} of {w.B} (all {w.Hq} heads), "
                      f"float64, {dt:.2f} s wall"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wide_gqa_t2048_d128")
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (reference kernel "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--cpu-sample-batch", type=int, default=4)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path shards over "
              "(batch, KV head) groups with no exchange, so N GPUs would each run this same kernel on their "
              "own groups).", file=sys.stderr)
        sys.exit(2)

    import torch
    from causal_gqa_flashattention_rope_amd import binding, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS[args.workload]
    out_dt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    q, k, v, dO = (t.to(dev) for t in inputs.make_inputs(w))
    B, T, Hq, Hkv, D = w.B, w.T, w.Hq, w.Hkv, w.D
    o = torch.empty((B, T, Hq, D), dtype=out_dt, device=dev)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    dq = torch.empty((B, T, Hq, D), dtype=out_dt, device=dev)
    dk = torch.empty((B, T, Hkv, D), dtype=out_dt, device=dev)
    dv = torch.empty((B, T, Hkv, D), dtype=out_dt, device=dev)
    wsf = binding.alloc_workspace(binding.fwd_workspace_bytes(B, T, Hq, Hkv, D, q.dtype), dev)
    wsb = binding.alloc_workspace(binding.bwd_workspace_bytes(B, T, Hq, Hkv, D, q.dtype), dev)

    def step(ev_f=None, ev_b=None):
        binding.ne_rope_attn_fwd(q, k, v, w.rope_base, o=o, lse=lse, workspace=wsf, events=ev_f)
        binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, w.rope_base, dq=dq, dk=dk, dv=dv, workspace=wsb,
                                 events=ev_b)

    for _ in range(args.warmup):
        step()
    K = args.steps
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    for e in evf + evb:          # create the HIP events before the timed region
        for x in e:
            x.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(evf[i], evb[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    def avg(evs, i):
        return sum(e[2 * i].elapsed_time(e[2 * i + 1]) for e in evs) / len(evs)   # ms

    kern_ms = {"prep_fwd": avg(evf, 0), "attn_fwd": avg(evf, 1), "prep_bwd": avg(evb, 0),
               "attn_bwd_dkdv": avg(evb, 1), "attn_bwd_dq": avg(evb, 2)}
    N = T * (T + 1) / 2
    unit = B * Hq * D * N
    flops_step = 14.0 * unit
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    # executed-useful MFMA work per launch (the deterministic dQ pass recomputes S and dP)
    kern_flops = {"attn_fwd": 4.0 * unit, "attn_bwd_dkdv": 8.0 * unit, "attn_bwd_dq": 6.0 * unit}
    peak = MFMA_PEAK_F16 if q.dtype != torch.float32 else MFMA_PEAK_F32
    dominant = max(kern_flops, key=lambda n: kern_ms[n])
    achieved = kern_flops[dominant] / (kern_ms[dominant] * 1e-3) / 1e12
    traffic = read_traffic(dominant, args.workload)
    fwd_ms = kern_ms["prep_fwd"] + kern_ms["attn_fwd"]
    bwd_ms = kern_ms["prep_bwd"] + kern_ms["attn_bwd_dkdv"] + kern_ms["attn_bwd_dq"]
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if q.dtype != torch.float32 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "Hq": Hq, "Hkv": Hkv, "head_dim": D,
                   "rope_base": w.rope_base, "in_dtype": w.dtype, "mfma_operands": "f16",
                   "accumulate": "f32", "out_dtype": args.out_dtype, "backward": "deterministic",
                   "step": "fwd+bwd", "global_batch": B, "seq_len": T, "parallelism": "none"},
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        "fwd_tflops": round(4.0 * unit / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(10.0 * unit / (bwd_ms * 1e-3) / 1e12, 2),
        "kernel_ms": {n: round(t, 4) for n, t in kern_ms.items()},
        "roofline": {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                     "flops_per_launch": kern_flops[dominant]},
    }
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n * 4
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, min(args.cpu_sample_batch, w.B))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
