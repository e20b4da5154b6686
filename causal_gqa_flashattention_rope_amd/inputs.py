"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module holds no attention arithmetic: it only draws Gaussian tensors from
numpy's PCG64 generator and rounds them to the storage dtype.  The same values
(widened to float64) go to the oracle, so both sides see identical inputs.

Workload shapes follow the pages' models: the NanoEuler CPU showcase model
(dim 128, 4 q / 2 kv heads, context 128) and GPU model (dim 768, 12 q / 4 kv heads,
context 512, head dim 64) from "NanoEuler: 使用 C 和 CUDA 从零开始构建的 GPT-2 规模 LLM",
table "模型配置"; a GPT-2-small-shaped MHA layer (llm.c guide, GPT-2 d12 with -t 1024);
and two wider/longer GQA stress shapes.  No dataset is involved: attention inputs
are activations, and N(0, 1) tensors stand in for them.
"""
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    rope_base: float      # <= 0 disables RoPE
    qk_scale: float       # Q and K are drawn as qk_scale * N(0, 1)
    seeds: tuple          # (q, k, v, dO)
    dtype: str            # storage dtype of q, k, v, dO: "f32" | "bf16" | "f16"
    description: str

    @property
    def G(self):
        return self.Hq // self.Hkv


WORKLOADS = {
    "tiny_cpu_model": Workload(
        "tiny_cpu_model", 1, 128, 4, 2, 32, 1.0e4, 1.0, (101, 102, 103, 104), "f32",
        "NanoEuler CPU-model attention layer: B1 T128 Hq4 Hkv2 D32, fp32"),
    "nanoeuler_gpu_layer": Workload(
        "nanoeuler_gpu_layer", 8, 512, 12, 4, 64, 1.0e4, 1.0, (201, 202, 203, 204), "bf16",
        "NanoEuler GPU-model attention layer: B8 T512 Hq12 Hkv4 D64, bf16 in"),
    "gpt2_small_mha": Workload(
        "gpt2_small_mha", 16, 1024, 12, 12, 64, 0.0, 1.0, (301, 302, 303, 304), "bf16",
        "GPT-2-small-shaped MHA: B16 T1024 H12 D64, no RoPE, bf16 in"),
    "wide_gqa_t2048_d128": Workload(
        "wide_gqa_t2048_d128", 4, 2048, 12, 4, 128, 1.0e4, 2.0, (401, 402, 403, 404), "bf16",
        "Wider-head GQA: B4 T2048 Hq12 Hkv4 D128, Q,K ~ 2 N(0,1), bf16 in"),
    "long_ctx_t8192": Workload(
        "long_ctx_t8192", 1, 8192, 32, 8, 128, 5.0e5, 1.0, (501, 502, 503, 504), "bf16",
        "Long-context stress: B1 T8192 Hq32 Hkv8 D128, RoPE base 5e5, bf16 in"),
    "long_ctx_t8192_shard8": Workload(
        "long_ctx_t8192_shard8", 1, 8192, 4, 1, 128, 5.0e5, 1.0, (511, 512, 513, 514), "bf16",
        "One GPU's share of the long-context layer split over 8 GPUs by KV head: B1 T8192 Hq4 Hkv1 "
        "D128 (one KV group), RoPE base 5e5, bf16 in"),
}

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def torch_dtype(name):
    return _TORCH_DT[name]


def gaussian(shape, seed, scale=1.0, dtype="f32"):
    """scale * N(0,1) drawn in float32 from PCG64(seed), rounded (RNE) to `dtype`.

    Returns a CPU torch tensor of the storage dtype.
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    return torch.from_numpy(x).to(_TORCH_DT[dtype])


def make_inputs(w: Workload, dtype=None, B=None, T=None):
    """q, k, v, dO for a workload as CPU tensors of the storage dtype.

    B and T may be overridden (smaller parity cases of the same recipe)."""
    dt = dtype or w.dtype
    B = w.B if B is None else B
    T = w.T if T is None else T
    sq, sk, sv, sd = w.seeds
    q = gaussian((B, T, w.Hq, w.D), sq, w.qk_scale, dt)
    k = gaussian((B, T, w.Hkv, w.D), sk, w.qk_scale, dt)
    v = gaussian((B, T, w.Hkv, w.D), sv, 1.0, dt)
    dO = gaussian((B, T, w.Hq, w.D), sd, 1.0, dt)
    return q, k, v, dO


def random_case(B, T, Hq, Hkv, D, seed, dtype="f32", qk_scale=1.0):
    """q, k, v, dO for an arbitrary (edge-case) shape from one base seed."""
    q = gaussian((B, T, Hq, D), seed, qk_scale, dtype)
    k = gaussian((B, T, Hkv, D), seed + 1, qk_scale, dtype)
    v = gaussian((B, T, Hkv, D), seed + 2, 1.0, dtype)
    dO = gaussian((B, T, Hq, D), seed + 3, 1.0, dtype)
    return q, k, v, dO
