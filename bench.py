#!/usr/bin/env python3
"""Throughput of the whole hot path -- causal GQA RoPE attention forward + backward -- on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one forward call (operand preparation + attention) and one backward call (dO scale,
preparation with Delta, dK/dV, dQ) over one batch of synthetic inputs already resident in HBM.  The
headline runs the default backward: deterministic, O(T) workspace, the dQ pass recomputing S and dP.
Throughput counts algorithmic causal FLOPs only (unmasked (query, key) pairs, N = T(T+1)/2 per head):
forward 4*B*Hq*D*N, backward 10*B*Hq*D*N, step 14*B*Hq*D*N.  The RoPE table is built once per
workspace (ne_rope_table_init) before the warmup, outside the timed steps, and timed on its own.
The whole-step time comes from the host clock around K synchronised steps; inside them the library
records HIP events (on the stream it launches on) around the dominant kernel only, whose average
duration gives the roofline figure.  The per-kernel breakdown comes from a separate pass with every
launch bracketed, the fwd / bwd / fwd+bwd medians and minima from another pass with events between
the calls, and the GPU clock under load from amdsmi samples taken while the same step runs for about
a second.  Prints one JSON line.

The other measurements run first (each with its own warmup), the headline last:
  * the same step with the backward's other designs: the stored dS (NE_FLAG_STORE_DS, under
    "stored_ds") and dQ added with atomics in the dK/dV pass (NE_FLAG_NONDETERMINISTIC, "atomic_dq");
  * a sliding window of --window keys (default T/4, the short window of the nanochat guide's
    window_pattern; 0 skips it), counting the visible pairs N_W = W(W+1)/2 + (T-W)W per head;
  * the causal step with the QK norm on (gain 1.2, eps 1e-6), under "qk_norm";
  * the causal step with the half-split rotary pairing (NE_FLAG_ROPE_HALF_SPLIT), under "half_split";
  * the workload layer's QKV projection with the RoPE epilogue (2 M N C flops), "qkv_projection";
  * one decode step of the cached workload (--decode-batch sequences, each holding 8191 tokens of the
    long-context shape, Hq 32 / Hkv 8 / D 128, RoPE base 5e5, attending with one new token) as HBM
    bandwidth: bytes = the visible cached keys and values (fp16) + q + o, under "decode";
  * fwd / bwd of every other workload of the table (the fp32 path of the NanoEuler layer too),
    under "configs".
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
DECODE_SOURCES = ["causal_gqa_flashattention_rope_amd/csrc/ne_decode.hip",
                  "causal_gqa_flashattention_rope_amd/csrc/ne_common.hpp"]
QKV_SOURCES = ["causal_gqa_flashattention_rope_amd/csrc/ne_qkv.hip",
               "causal_gqa_flashattention_rope_amd/csrc/ne_common.hpp"]


# Executed MFMA work of each kernel per (query, key) pair and head, in units of D, for each backward
# design: the dQ pass recomputes S and dP (6 D), or reads the stored dS (2 D); with atomic dQ the
# dK/dV pass carries the dQ product (8 D + 2 D) and the dQ launch only converts the accumulator.
KERNEL_FLOPS_OVER_D = {
    "recompute": {"attn_fwd": 4.0, "attn_bwd_dkdv": 8.0, "attn_bwd_dq": 6.0},
    "stored_ds": {"attn_fwd": 4.0, "attn_bwd_dkdv": 8.0, "attn_bwd_dq": 2.0},
    "atomic": {"attn_fwd": 4.0, "attn_bwd_dkdv": 10.0, "attn_bwd_dq": 0.0},
}


class ClockSampler:
    """The GPU's current graphics clock (MHz), sampled from a background thread with amdsmi while the
    GPU runs a workload; None if amdsmi cannot be used."""

    def __init__(self):
        self.ok = False
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.smi = amdsmi
            self.handle = amdsmi.amdsmi_get_processor_handles()[0]
            self.read()
            self.ok = True
        except Exception:
            self.ok = False

    def read(self):
        info = self.smi.amdsmi_get_clock_info(self.handle, self.smi.AmdSmiClkType.GFX)
        return float(info["clk"])

    def sample_while(self, fn):
        import threading
        samples, stop = [], threading.Event()

        def loop():
            while not stop.is_set():
                try:
                    samples.append(self.read())
                except Exception:
                    pass
                time.sleep(0.002)
        th = threading.Thread(target=loop, daemon=True)
        if self.ok:
            th.start()
        try:
            fn()
        finally:
            stop.set()
            if self.ok:
                th.join()
        if not samples:
            return None
        samples.sort()
        return {"median": samples[len(samples) // 2], "min": samples[0], "max": samples[-1],
                "samples": len(samples), "unit": "MHz"}


def kernel_source_hash(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^\s*([a-z0-9_]+):\s*(\S+)\s*$", line)
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class _HipEvents:
    """Timing-only HIP events created with hipEventDisableSystemFence: recording one does not
    write back and invalidate the caches, so it neither slows the step nor the next kernel."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        import torch
        self.ct = ctypes
        name = "libamdhip64.so"
        for d in (os.path.join(os.path.dirname(torch.__file__), "lib"), "/opt/rocm/lib"):
            if os.path.exists(os.path.join(d, name)):
                name = os.path.join(d, name)
                break
        self.hip = ctypes.CDLL(name)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            h = self.ct.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(self.ct.byref(h), self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            out.append(h.value)
        return out

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value


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


def measure_configs(skip, hev, new_events):
    """Every other workload of the table: fwd, bwd and fwd+bwd times (median and min over the reps,
    HIP events around each call on the current stream), with fp32 outputs (the fp32 path for the fp32
    workload, and the NanoEuler layer on the fp32 path as well, against the fp32 MFMA peak).  The two
    smaller, HBM-relevant workloads also get a cold fwd+bwd number: 1 GiB is written between reps,
    which evicts the 256 MB last-level cache."""
    import statistics
    import torch
    from causal_gqa_flashattention_rope_amd import binding, inputs
    dev = torch.device("cuda:0")
    out = {}
    scrub = None
    runs = [(name, w, None) for name, w in inputs.WORKLOADS.items() if name != skip]
    runs.insert(2, ("nanoeuler_gpu_layer_f32", inputs.WORKLOADS["nanoeuler_gpu_layer"], "f32"))
    for name, w, dt in runs:
        q, k, v, dO = (t.to(dev) for t in inputs.make_inputs(w, dtype=dt))
        B, T, Hq, Hkv, D = w.B, w.T, w.Hq, w.Hkv, w.D
        o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
        dq = torch.empty_like(o)
        dk = torch.empty((B, T, Hkv, D), dtype=torch.float32, device=dev)
        dv = torch.empty_like(dk)
        ws = binding.new_workspace(True, q, k, w.rope_base)   # serves the forward too
        stream = torch.cuda.current_stream().cuda_stream

        def call(ev=None):
            if ev:
                hev.record(ev[0], stream)
            binding.ne_rope_attn_fwd(q, k, v, w.rope_base, o=o, lse=lse, workspace=ws)
            if ev:
                hev.record(ev[1], stream)
            binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, w.rope_base, dq=dq, dk=dk, dv=dv, workspace=ws)
            if ev:
                hev.record(ev[2], stream)

        reps = 20 if T >= 8192 else 50
        for _ in range(10):
            call()
        evs = [new_events(3) for _ in range(reps)]
        for e in evs:
            call(e)
        torch.cuda.synchronize()
        f = [hev.elapsed_ms(e[0], e[1]) for e in evs]
        b = [hev.elapsed_ms(e[1], e[2]) for e in evs]
        fb = [x + y for x, y in zip(f, b)]
        unit = B * Hq * D * T * (T + 1) / 2
        peak = MFMA_PEAK_F32 if q.dtype == torch.float32 else MFMA_PEAK_F16
        tf = 14.0 * unit / (statistics.median(fb) * 1e-3) / 1e12
        rec = {"shape": f"B{B} T{T} Hq{Hq} Hkv{Hkv} D{D}", "rope_base": w.rope_base,
               "in_dtype": dt or w.dtype, "out_dtype": "f32", "reps": reps,
               "fwd_ms": {"median": round(statistics.median(f), 4), "min": round(min(f), 4)},
               "bwd_ms": {"median": round(statistics.median(b), 4), "min": round(min(b), 4)},
               "fwd_bwd_ms": {"median": round(statistics.median(fb), 4), "min": round(min(fb), 4)},
               "fwd_bwd_tflops_median": round(tf, 2), "mfma_peak": peak,
               "frac_of_peak": round(tf / peak, 4)}
        if name in ("nanoeuler_gpu_layer", "gpt2_small_mha"):
            if scrub is None:
                scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
            cold = []
            for _ in range(10):
                scrub.fill_(1.0)
                e = new_events(3)
                call(e)
                torch.cuda.synchronize()
                cold.append(hev.elapsed_ms(e[0], e[2]))
            rec["cold_fwd_bwd_ms"] = {"median": round(statistics.median(cold), 4), "min": round(min(cold), 4),
                                      "reps": 10}
        out[name] = rec
        del q, k, v, dO, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return out


def measure_decode(Bd, K, hev, new_events):
    """One decode step (split-KV attention with the query rotation, then the merge) of Bd sequences of the
    long-context shape with 8191 cached tokens and one new token each."""
    import torch
    from causal_gqa_flashattention_rope_amd import binding, inputs
    dev = torch.device("cuda:0")
    Tcap, Hq, Hkv, D, base = 8192, 32, 8, 128, 5.0e5
    L = Tcap - 1                                       # tokens already in the cache
    cache = binding.new_kv_cache(Bd, Tcap, Hkv, D, torch.bfloat16, dev)
    lens = torch.zeros(Bd, dtype=torch.int32, device=dev)
    for c in range(0, Tcap, 1024):
        kc = inputs.gaussian((Bd, 1024, Hkv, D), 801 + c, 1.0, "bf16").to(dev)
        vc = inputs.gaussian((Bd, 1024, Hkv, D), 901 + c, 1.0, "bf16").to(dev)
        binding.ne_kv_cache_append(cache, lens, kc, vc, Tcap, base)
        lens += 1024
    lens.fill_(L)
    q = inputs.gaussian((Bd, 1, Hq, D), 990, 1.0, "bf16").to(dev)
    o = torch.empty((Bd, 1, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Bd, Hq, 1), dtype=torch.float32, device=dev)
    ws = binding.alloc_workspace(binding.decode_workspace_bytes(Bd, 1, Tcap, Hq, Hkv, D, torch.bfloat16), dev)

    def call(ev=None):
        binding.ne_rope_attn_decode(q, cache, lens, Tcap, Hkv, base, 0, o=o, lse=lse, workspace=ws, events=ev)

    # warm-up with every launch bracketed (per-kernel breakdown)
    Wd = 50
    evs = [new_events(4) for _ in range(Wd)]
    for i in range(Wd):
        call(evs[i])
    torch.cuda.synchronize()
    kern = {n: sum(hev.elapsed_ms(e[2 * i], e[2 * i + 1]) for e in evs[-10:]) / 10
            for i, n in enumerate(["decode_split", "decode_merge"])}
    # timed: K calls, events only around the split kernel
    tev = [new_events(2) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        call([tev[i][0], tev[i][1], None, None])
    torch.cuda.synchronize()
    ms_call = (time.perf_counter() - t0) * 1e3 / K
    split_ms = sum(hev.elapsed_ms(a, b) for a, b in tev) / K
    # append of one token per sequence (the other half of a serving step), timed alone
    k1 = inputs.gaussian((Bd, 1, Hkv, D), 991, 1.0, "bf16").to(dev)
    lens_app = torch.full((Bd,), L, dtype=torch.int32, device=dev)
    binding.ne_kv_cache_append(cache, lens_app, k1, k1, Tcap, base)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        binding.ne_kv_cache_append(cache, lens_app, k1, k1, Tcap, base)
    torch.cuda.synchronize()
    append_ms = (time.perf_counter() - t0) * 1e3 / K
    kv_bytes = 2.0 * Bd * Hkv * (L + 1) * D * 2        # visible keys and values, fp16
    io_bytes = Bd * Hq * D * 2 * 2 + Bd * Hq * 4       # q, o (bf16), lse
    split_bytes = kv_bytes + Bd * Hq * D * 2           # the split kernel reads the cache and q~
    return {
        "workload": f"decode_t8192_b{Bd}", "B": Bd, "cached_tokens": L, "new_tokens": 1, "Tcap": Tcap,
        "Hq": Hq, "Hkv": Hkv, "head_dim": D, "rope_base": base, "in_dtype": "bf16", "cache_dtype": "f16",
        "out_dtype": "bf16", "ms_per_call": round(ms_call, 4), "tokens_per_s": round(Bd / (ms_call * 1e-3), 1),
        "hbm_gb_s": round((kv_bytes + io_bytes) / (ms_call * 1e-3) / 1e9, 1),
        "kernel_ms": {n: round(t, 4) for n, t in kern.items()},
        "append_one_token_ms": round(append_ms, 4),
        "roofline": {"kernel": "decode_split", "bound": "hbm",
                     "achieved": round(split_bytes / (split_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK,
                     "unit": "GB/s", "frac": round(split_bytes / (split_ms * 1e-3) / 1e9 / HBM_PEAK, 4),
                     "traffic": read_traffic("decode_split", f"decode_t8192_b{Bd}", DECODE_SOURCES),
                     "bytes_per_launch": split_bytes, "launch_ms": round(split_ms, 4)},
    }


def measure_qkv(w, K, hev, new_events, peak):
    """The QKV projection of the workload's layer (C = Hq D, weight [(Hq + 2 Hkv) D][C]) with the RoPE
    epilogue: 2 M N C flops per call, M = B T."""
    import torch
    from causal_gqa_flashattention_rope_amd import binding, inputs
    dev = torch.device("cuda:0")
    B, T, Hq, Hkv, D = w.B, w.T, w.Hq, w.Hkv, w.D
    C = Hq * D
    N = (Hq + 2 * Hkv) * D
    x = inputs.gaussian((B, T, C), 1101, 1.0, "bf16").to(dev)
    wt = inputs.gaussian((N, C), 1102, C ** -0.5, "bf16").to(dev)
    q = torch.empty((B, T, Hq, D), dtype=torch.bfloat16, device=dev)
    k = torch.empty((B, T, Hkv, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty((B, T, Hkv, D), dtype=torch.bfloat16, device=dev)
    ws = binding.alloc_workspace(int(binding.lib().ne_qkv_rope_workspace_bytes(T, D)), dev)

    def call(ev=None):
        binding.ne_qkv_rope_proj(x, wt, Hq, Hkv, w.rope_base, q=q, k=k, v=v, workspace=ws, events=ev)

    evs = [new_events(4) for _ in range(50)]
    for i in range(50):
        call(evs[i])
    torch.cuda.synchronize()
    table_ms = sum(hev.elapsed_ms(e[0], e[1]) for e in evs[-10:]) / 10
    tev = [new_events(2) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        call([None, None, tev[i][0], tev[i][1]])
    torch.cuda.synchronize()
    ms_call = (time.perf_counter() - t0) * 1e3 / K
    gemm_ms = sum(hev.elapsed_ms(a, b) for a, b in tev) / K
    flops = 2.0 * B * T * N * C
    ach = flops / (gemm_ms * 1e-3) / 1e12
    return {"workload": f"qkv_proj_b{B}_t{T}_c{C}_n{N}", "M": B * T, "N": N, "C": C, "in_dtype": "bf16",
            "out_dtype": "bf16", "epilogue": "rope", "ms_per_call": round(ms_call, 4),
            "value": round(flops / (ms_call * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "kernel_ms": {"qkv_rope_table": round(table_ms, 4), "qkv_rope_gemm": round(gemm_ms, 4)},
            "roofline": {"kernel": "qkv_rope_gemm", "bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                         "traffic": read_traffic("qkv_rope_gemm", f"qkv_proj_b{B}_t{T}_c{C}_n{N}", QKV_SOURCES),
                         "flops_per_launch": flops, "launch_ms": round(gemm_ms, 4)}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100, help="untimed steps before the timed ones")
    ap.add_argument("--workload", default="wide_gqa_t2048_d128")
    ap.add_argument("--out-dtype", default="bf16", choices=["f32", "bf16"],
                    help="dtype of o, dq, dk, dv (the inputs are bf16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (reference kernel "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--cpu-sample-batch", type=int, default=4)
    ap.add_argument("--window", type=int, default=-1,
                    help="window of the sliding-window measurement (-1: T/4; 0: skip it)")
    ap.add_argument("--qkv", type=int, default=1, help="also measure the QKV projection with the RoPE epilogue")
    ap.add_argument("--qk-norm", type=int, default=1, help="also measure the step with the QK norm on (0: skip)")
    ap.add_argument("--half-split", type=int, default=1,
                    help="also measure the step with the half-split rotary pairing (0: skip)")
    ap.add_argument("--other-backwards", type=int, default=1,
                    help="also measure the step with the stored dS and with the atomic dQ (0: skip)")
    ap.add_argument("--configs", type=int, default=1,
                    help="also time fwd / bwd of every other workload of the table (0: skip)")
    ap.add_argument("--decode-batch", type=int, default=8,
                    help="sequences of the decode measurement (0: skip it)")
    ap.add_argument("--clock", type=int, default=1, help="sample the GPU clock under load (0: skip)")
    ap.add_argument("--flags", type=int, default=0,
                    help="backward flags of the headline step (0: the default, deterministic O(T) backward)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path shards over "
              "(batch, KV head) groups with no exchange, so N GPUs would each run this same kernel on their "
              "own groups).", file=sys.stderr)
        sys.exit(2)

    import statistics
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
    hev = _HipEvents()

    def new_events(n):              # created outside any timed region
        return hev.create(n)

    wss = {}

    def workspace(flags):
        """One backward workspace per flag set (it serves the forward too), its table built once."""
        if flags not in wss:
            n = binding.workspace_bytes(True, B, T, Hq, Hkv, D, w.rope_base, q.dtype, flags)
            wss[flags] = binding.alloc_workspace(n, dev)
            binding.ne_rope_table_init(wss[flags], T, D, w.rope_base)
        return wss[flags]

    def make_step(window=0, qk_norm=None, flags=0):
        ws = workspace(flags)

        def step(ev_f=None, ev_b=None):
            binding.ne_rope_attn_fwd(q, k, v, w.rope_base, o=o, lse=lse, workspace=ws, window=window,
                                     qk_norm=qk_norm, events=ev_f, flags=flags & binding.NE_FLAG_ROPE_HALF_SPLIT)
            binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, w.rope_base, dq=dq, dk=dk, dv=dv, workspace=ws,
                                     flags=flags, window=window, qk_norm=qk_norm, events=ev_b)
        return step

    def per_kernel_ms(evf, evb):
        def avg(evs, i):
            return sum(hev.elapsed_ms(e[2 * i], e[2 * i + 1]) for e in evs) / len(evs)   # ms
        return {"prep_fwd": avg(evf, 0), "attn_fwd": avg(evf, 1), "prep_bwd": avg(evb, 0),
                "attn_bwd_dkdv": avg(evb, 1), "attn_bwd_dq": avg(evb, 2)}

    slot = {"prep_fwd": ("f", 0), "attn_fwd": ("f", 1), "prep_bwd": ("b", 0), "attn_bwd_dkdv": ("b", 1),
            "attn_bwd_dq": ("b", 2)}

    def measure(step, warmup, K):
        """(ms per step, dominant kernel, its launch ms (mean, min, max), per-kernel breakdown)"""
        # warmup, every launch bracketed: picks the dominant kernel (the longest of the three
        # attention kernels) that the timed region brackets
        Wu = max(warmup, 1)
        evf = [new_events(4) for _ in range(Wu)]
        evb = [new_events(6) for _ in range(Wu)]
        for i in range(Wu):
            step(evf[i], evb[i])
        torch.cuda.synchronize()
        warm = per_kernel_ms(evf, evb)
        dominant = max(["attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq"], key=lambda n: warm[n])

        # timed region: K steps; HIP events only around the dominant kernel (each event record
        # costs stream time, so bracketing every launch would slow the step being measured)
        side, idx = slot[dominant]
        tev = [new_events(2) for _ in range(K)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            pair = [None] * (4 if side == "f" else 6)
            pair[2 * idx], pair[2 * idx + 1] = tev[i]
            if side == "f":
                step(pair, None)
            else:
                step(None, pair)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_per_step = (t1 - t0) * 1e3 / K
        dl = [hev.elapsed_ms(a, b) for a, b in tev]

        # per-kernel breakdown from a separate, untimed pass with every launch bracketed
        Kb = min(K, 10)
        evf = [new_events(4) for _ in range(Kb)]
        evb = [new_events(6) for _ in range(Kb)]
        torch.cuda.synchronize()
        for i in range(Kb):
            step(evf[i], evb[i])
        torch.cuda.synchronize()
        return ms_per_step, dominant, (sum(dl) / K, min(dl), max(dl)), per_kernel_ms(evf, evb)

    N = T * (T + 1) / 2
    unit = B * Hq * D * N
    flops_step = 14.0 * unit
    peak = MFMA_PEAK_F16 if q.dtype != torch.float32 else MFMA_PEAK_F32

    def roofline(design, dominant, dom, flops_unit, traffic_key=None):
        kf = KERNEL_FLOPS_OVER_D[design][dominant] * flops_unit
        ach = kf / (dom[0] * 1e-3) / 1e12
        return {"kernel": dominant, "bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4),
                "traffic": read_traffic(dominant, traffic_key) if traffic_key else None,
                "flops_per_launch": kf, "launch_ms": round(dom[0], 4),
                "launch_ms_min": round(dom[1], 4), "launch_ms_max": round(dom[2], 4),
                "launch_ms_source": "HIP events around this kernel in every timed step"}

    def side_line(step, design, flops_unit, K):
        ms, dom_k, dom, kern = measure(step, 20, K)
        return {"value": round(14.0 * flops_unit / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                "ms_per_step": round(ms, 4), "steps": K, "warmup": 20,
                "kernel_ms": {n: round(t, 4) for n, t in kern.items()},
                "roofline": roofline(design, dom_k, dom, flops_unit)}

    result = {}
    K = args.steps
    # ---- the other measurements first (each with its own warmup), the headline last ----
    if args.other_backwards and q.dtype != torch.float32:
        result["stored_ds"] = dict(side_line(make_step(flags=binding.NE_FLAG_STORE_DS), "stored_ds", unit, K),
                                   flags="NE_FLAG_STORE_DS", dq_pass="stored_ds", deterministic=True,
                                   workspace_bytes=binding.workspace_bytes(True, B, T, Hq, Hkv, D, w.rope_base,
                                                                           q.dtype, binding.NE_FLAG_STORE_DS))
        result["atomic_dq"] = dict(side_line(make_step(flags=binding.NE_FLAG_NONDETERMINISTIC), "atomic", unit, K),
                                   flags="NE_FLAG_NONDETERMINISTIC", dq_pass="atomic adds in dK/dV",
                                   deterministic=False,
                                   workspace_bytes=binding.workspace_bytes(True, B, T, Hq, Hkv, D, w.rope_base,
                                                                           q.dtype, binding.NE_FLAG_NONDETERMINISTIC))
    Wn = T // 4 if args.window < 0 else args.window
    if 0 < Wn < T:
        unit_w = B * Hq * D * (Wn * (Wn + 1) / 2 + (T - Wn) * Wn)
        result["sliding_window"] = dict(window=Wn, pairs_per_head=Wn * (Wn + 1) // 2 + (T - Wn) * Wn,
                                        **side_line(make_step(window=Wn), "recompute", unit_w, K))
    if args.qk_norm:
        result["qk_norm"] = dict(gain=1.2, eps=1e-6, **side_line(make_step(qk_norm=(1.2, 1e-6)), "recompute", unit, K))
    if args.half_split and w.rope_base > 0:
        result["half_split"] = dict(flags="NE_FLAG_ROPE_HALF_SPLIT", pairs="(i, i + D/2)",
                                    **side_line(make_step(flags=binding.NE_FLAG_ROPE_HALF_SPLIT), "recompute", unit, K))
    if args.qkv:
        result["qkv_projection"] = measure_qkv(w, K, hev, new_events, MFMA_PEAK_F16)
    if args.decode_batch > 0:
        result["decode"] = measure_decode(args.decode_batch, K, hev, new_events)
    if args.configs:
        result["configs"] = measure_configs(args.workload, hev, new_events)

    # ---- the headline: the default backward (or --flags) ----
    design = ("atomic" if args.flags & binding.NE_FLAG_NONDETERMINISTIC else
              "stored_ds" if args.flags & binding.NE_FLAG_STORE_DS else "recompute")
    step = make_step(flags=args.flags)
    # the RoPE table, built once per workspace outside the timed steps, timed on its own
    tbl = new_events(2)
    torch.cuda.synchronize()
    hev.record(tbl[0], torch.cuda.current_stream().cuda_stream)
    binding.ne_rope_table_init(wss[args.flags], T, D, w.rope_base)
    hev.record(tbl[1], torch.cuda.current_stream().cuda_stream)
    ms_per_step, dominant, dom, kern_ms = measure(step, args.warmup, K)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    # fwd / bwd / fwd+bwd medians and minima (events between the calls), then the clock under load
    stream = torch.cuda.current_stream().cuda_stream
    Ks = 50
    sev = [new_events(3) for _ in range(Ks)]
    for e in sev:
        hev.record(e[0], stream)
        binding.ne_rope_attn_fwd(q, k, v, w.rope_base, o=o, lse=lse, workspace=wss[args.flags])
        hev.record(e[1], stream)
        binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, w.rope_base, dq=dq, dk=dk, dv=dv, workspace=wss[args.flags],
                                 flags=args.flags)
        hev.record(e[2], stream)
    torch.cuda.synchronize()
    fl = [hev.elapsed_ms(e[0], e[1]) for e in sev]
    bl = [hev.elapsed_ms(e[1], e[2]) for e in sev]
    fbl = [a + b for a, b in zip(fl, bl)]

    def med_min(x, flops):
        return {"median_ms": round(statistics.median(x), 4), "min_ms": round(min(x), 4),
                "tflops_median": round(flops / (statistics.median(x) * 1e-3) / 1e12, 2),
                "tflops_max": round(flops / (min(x) * 1e-3) / 1e12, 2)}
    clock = None
    if args.clock:
        sampler = ClockSampler()

        def load():
            t_end = time.perf_counter() + 1.0
            while time.perf_counter() < t_end:
                for _ in range(20):
                    step()
                torch.cuda.synchronize()
        clock = sampler.sample_while(load)

    traffic_key = args.workload if design == "recompute" and args.out_dtype == "bf16" else None
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
                   "accumulate": "f32", "out_dtype": args.out_dtype, "flags": args.flags,
                   "backward": "deterministic" if design != "atomic" else "atomic dQ (not bit-reproducible)",
                   "dq_pass": design, "workspace": "O(T)" if design == "recompute" else "O(T^2) stored dS"
                   if design == "stored_ds" else "O(T) + fp32 dQ accumulator",
                   "step": "fwd+bwd", "global_batch": B, "seq_len": T, "parallelism": "none"},
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        "fwd_tflops": round(4.0 * unit / ((kern_ms["prep_fwd"] + kern_ms["attn_fwd"]) * 1e-3) / 1e12, 2),
        "bwd_tflops": round(10.0 * unit / ((kern_ms["prep_bwd"] + kern_ms["attn_bwd_dkdv"] + kern_ms["attn_bwd_dq"])
                                           * 1e-3) / 1e12, 2),
        "spread": {"fwd": med_min(fl, 4.0 * unit), "bwd": med_min(bl, 10.0 * unit),
                   "fwd_bwd": med_min(fbl, flops_step), "reps": Ks,
                   "note": "HIP events between the calls of separate steps after the timed region"},
        "gpu_clock_under_load": clock,
        "rope_table_init_ms": round(hev.elapsed_ms(*tbl), 4),
        "kernel_ms": {n: round(t, 4) for n, t in kern_ms.items()},
        "kernel_ms_note": f"separate pass of {min(K, 10)} steps with every launch bracketed by HIP events "
                          "(prep_bwd includes the dO scale pass)",
        "roofline": roofline(design, dominant, dom, unit, traffic_key),
        **result,
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
