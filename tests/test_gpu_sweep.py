"""A seeded sweep of shapes, dtypes, backward designs and options against the double-precision oracle
(needs an MI355X).

The cases are drawn once, from a fixed seed, over the space the ABI supports: head_dim 32, 64, 128;
group sizes 1-8; one to three KV heads and one or two batch elements (few groups make the host plans
split the longest causal blocks over several workgroups, or run single dK/dV key blocks); ragged T up
to 1500; bf16 and fp16 inputs with fp32 or 16-bit outputs, and the fp32 path; the three backward
designs; RoPE on (two bases) or off, with either rotary pairing; a sliding window in a quarter of the
cases and the QK norm in a quarter.  Bars and the zero-reference scale are those of test_gpu_parity.
"""
import numpy as np
import pytest
import torch

import oracle
from causal_gqa_flashattention_rope_amd import binding, inputs
from tests.test_gpu_parity import BWD_FLAGS, DEV, check, f64, zero_ref_scale

pytestmark = pytest.mark.gpu

HALF = binding.NE_FLAG_ROPE_HALF_SPLIT
_NAME = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}


def _cases(n=64, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([32, 64, 128]))
        G = int(rng.choice([1, 2, 3, 4, 6, 8]))
        Hkv = int(rng.integers(1, 4))
        B = int(rng.integers(1, 3))
        T = int(rng.integers(1, 1501)) if i % 4 else int(rng.integers(1, 130))
        in_dt = [torch.bfloat16, torch.float16, torch.float32][int(rng.choice(3, p=[0.45, 0.35, 0.2]))]
        out_dt = torch.float32 if (in_dt == torch.float32 or rng.random() < 0.6) else in_dt
        flags = BWD_FLAGS[int(rng.integers(0, 3))] if in_dt != torch.float32 else 0
        base = float(rng.choice([1.0e4, 5.0e5, 0.0]))
        if rng.random() < 0.4:
            flags |= HALF
        window = int(rng.integers(1, T + 1)) if rng.random() < 0.25 else 0
        qkn = (1.2, 1e-6) if rng.random() < 0.25 else None
        out.append((B, T, G * Hkv, Hkv, D, in_dt, out_dt, flags, base, window, qkn, 7000 + i))
    return out


CASES = _cases()


def _id(c):
    B, T, Hq, Hkv, D, i, o, fl, base, w, qkn, _ = c
    return (f"B{B}T{T}Hq{Hq}Hkv{Hkv}D{D}-{_NAME[i]}-{_NAME[o]}-f{fl}-b{base:g}-w{w}"
            f"-{'qkn' if qkn else 'plain'}")


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_sweep_parity(case):
    B, T, Hq, Hkv, D, in_dt, out_dt, flags, base, window, qkn, seed = case
    half = bool(flags & HALF) and base > 0
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=seed, dtype=_NAME[in_dt])
    qd, kd, vd, dOd = (t.to(DEV) for t in (q, k, v, dO))
    ws = binding.alloc_workspace(binding.workspace_bytes(True, B, T, Hq, Hkv, D, base, q.dtype, flags), DEV)
    binding.ne_rope_table_init(ws, T, D, base)
    o, lse = binding.ne_rope_attn_fwd(qd, kd, vd, base, out_dtype=out_dt, workspace=ws, flags=flags & HALF,
                                      window=window, qk_norm=qkn)
    dq, dk, dv = binding.ne_rope_attn_bwd(qd, kd, vd, o, lse, dOd, base, workspace=ws, flags=flags, window=window,
                                          qk_norm=qkn)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (t.cpu() for t in (o, lse, dq, dk, dv))
    ro, rlse = oracle.fwd(f64(q), f64(k), f64(v), base, window=window, qk_norm=qkn, half_split=half)
    if out_dt == torch.float32:
        r = oracle.bwd(f64(q), f64(k), f64(v), f64(dO), base, window=window, qk_norm=qkn, half_split=half)
    else:
        r = oracle.bwd_given_o(f64(q), f64(k), f64(v), f64(o), f64(dO), base, window=window, qk_norm=qkn,
                               half_split=half)
    gscale = zero_ref_scale(in_dt, r)
    for name, g, ref in (("o", o, ro), ("lse", lse, rlse), ("dq", dq, r[0]), ("dk", dk, r[1]), ("dv", dv, r[2])):
        check(name, g, ref, in_dt, out_dt, zero_scale=gscale)


def test_sweep_covers_the_plans_designs_and_options():
    """The drawn cases include every head_dim, input dtype and backward design, 16-bit outputs, no-RoPE
    calls, both pairings with RoPE on, windows, the QK norm, single-group calls long enough for the
    plans to split, and T = 1-class short sequences."""
    assert {c[4] for c in CASES} == {32, 64, 128}
    assert {c[5] for c in CASES} == {torch.bfloat16, torch.float16, torch.float32}
    assert {c[7] & ~HALF for c in CASES} == set(BWD_FLAGS)
    assert any(c[6] not in (torch.float32,) for c in CASES) and any(c[8] == 0.0 for c in CASES)
    assert any(c[7] & HALF and c[8] > 0 for c in CASES) and any(not c[7] & HALF and c[8] > 0 for c in CASES)
    assert any(c[9] > 0 for c in CASES) and any(c[10] is not None for c in CASES)
    assert any(c[0] * c[3] == 1 and c[1] > 600 for c in CASES)
    assert any(c[1] < 130 for c in CASES)
