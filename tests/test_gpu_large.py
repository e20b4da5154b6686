"""Tensors of 2^31 elements and more (needs an MI355X and about 35 GB of its memory).

The ABI limits one (batch, KV head) group's T * G * head_dim operand bytes to below 2^31 (its rows are
addressed with 32-bit offsets), not the whole tensor: q of B1 T2^19 Hq32 D128 holds exactly 2^31
elements.  The call runs with a short sliding window, so every output row depends on a few hundred
positions, and sampled rows are compared with the oracle run on just those positions: a query row t
sees keys t - W + 1 .. t, key row j is seen by queries j .. j + W - 1, and RoPE scores depend only on
position differences, so the oracle on a slice of the sequence (positions renumbered from 0) gives
those rows exactly.  Bars as in test_gpu_parity (bf16 inputs and outputs: 2e-3 of the scale plus half
an ulp).  Inputs are drawn on the device from a seeded generator.
"""
import pytest
import torch

import oracle
from tests.test_gpu_parity import DEV, check, f64

pytestmark = pytest.mark.gpu


B, T, Hq, Hkv, D, W, BASE = 1, 1 << 19, 32, 8, 128, 128, 5.0e5
G = Hq // Hkv
QROWS = (0, 5, W - 1, W, (1 << 18) + 777, T - 1)          # query rows checked (o, lse, dq)
KROWS = (0, 3, W, (1 << 18) + 4321, T - W, T - 1)          # key rows checked (dk, dv)
GROUPS = (0, Hkv - 1)



def _run_large():
    """Runs the call and returns, on the host, every input and output row the checks need (the
    ~30 GB of device tensors are released when this returns)."""
    from causal_gqa_flashattention_rope_amd import binding
    gen = torch.Generator(device=DEV).manual_seed(20261202)
    q = torch.randn((B, T, Hq, D), generator=gen, device=DEV, dtype=torch.bfloat16)
    k = torch.randn((B, T, Hkv, D), generator=gen, device=DEV, dtype=torch.bfloat16)
    v = torch.randn((B, T, Hkv, D), generator=gen, device=DEV, dtype=torch.bfloat16)
    dO = torch.randn((B, T, Hq, D), generator=gen, device=DEV, dtype=torch.bfloat16)
    ws = binding.new_workspace(True, q, k, BASE)
    o, lse = binding.ne_rope_attn_fwd(q, k, v, BASE, out_dtype=torch.bfloat16, workspace=ws, window=W)
    dq, dk, dv = binding.ne_rope_attn_bwd(q, k, v, o, lse, dO, BASE, workspace=ws, window=W)
    torch.cuda.synchronize()
    spans = [(max(0, t - W + 1), t + 1) for t in QROWS] + [(max(0, j - W + 1), min(T, j + W)) for j in KROWS]
    host = {}
    for s0, s1 in spans:
        host[(s0, s1)] = {n: x[:, s0:s1].cpu() for n, x in (("q", q), ("k", k), ("v", v), ("dO", dO), ("o", o),
                                                            ("dq", dq), ("dk", dk), ("dv", dv))}
        host[(s0, s1)]["lse"] = lse[:, :, s0:s1].cpu()
    return host


def test_tensors_beyond_2_31_elements_with_a_window():
    assert B * T * Hq * D == 1 << 31
    print(f"large: B{B} T{T} Hq{Hq} Hkv{Hkv} D{D} window {W}", flush=True)
    host = _run_large()
    torch.cuda.empty_cache()
    bf = torch.bfloat16
    for t in QROWS:           # query rows: the positions t - W + 1 .. t
        s0 = max(0, t - W + 1)
        x = host[(s0, t + 1)]
        for g in GROUPS:
            hs = slice(g * G, (g + 1) * G)
            qs, ks, vs = f64(x["q"][:, :, hs]), f64(x["k"][:, :, g:g + 1]), f64(x["v"][:, :, g:g + 1])
            ro, rlse = oracle.fwd(qs, ks, vs, BASE, window=W)
            rdq, _, _ = oracle.bwd_given_o(qs, ks, vs, f64(x["o"][:, :, hs]), f64(x["dO"][:, :, hs]), BASE, window=W)
            r = t - s0
            check("o", x["o"][:, r:r + 1, hs], ro[:, r:r + 1], bf, bf)
            check("lse", x["lse"][:, hs, r:r + 1], rlse[:, :, r:r + 1], bf, bf)
            check("dq", x["dq"][:, r:r + 1, hs], rdq[:, r:r + 1], bf, bf, zero_scale=1e-3)
    for j in KROWS:           # key rows: queries j .. j + W - 1 see them, and keys from j - W + 1
        s0, s1 = max(0, j - W + 1), min(T, j + W)
        x = host[(s0, s1)]
        for g in GROUPS:
            hs = slice(g * G, (g + 1) * G)
            qs, ks, vs = f64(x["q"][:, :, hs]), f64(x["k"][:, :, g:g + 1]), f64(x["v"][:, :, g:g + 1])
            _, rdk, rdv = oracle.bwd_given_o(qs, ks, vs, f64(x["o"][:, :, hs]), f64(x["dO"][:, :, hs]), BASE, window=W)
            r = j - s0
            check("dk", x["dk"][:, r:r + 1, g:g + 1], rdk[:, r:r + 1], bf, bf, zero_scale=1e-3)
            check("dv", x["dv"][:, r:r + 1, g:g + 1], rdv[:, r:r + 1], bf, bf)
